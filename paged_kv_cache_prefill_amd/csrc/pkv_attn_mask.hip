// Attention kernel instantiations with the custom topology mask (see pkv_attn.h).
#include "pkv_attn.h"

namespace pkv {

hipError_t launch_attention_mask(int tile_kind, int dtype, int head_dim, const AttnArgs& a, hipStream_t s) {
  return launch_attention_var<1>(tile_kind, dtype, head_dim, a, s);
}

}  // namespace pkv
