// Attention kernel instantiations over FP8 E4M3 K/V caches (see pkv_attn.h).
#include "pkv_attn.h"

namespace pkv {

hipError_t launch_attention_fp8(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                hipStream_t s) {
  return launch_attention_var<4>(tile_kind, dtype, head_dim, a, s);
}

}  // namespace pkv
