// Attention kernel instantiations over FP8 E4M3 K/V caches with the custom topology mask
// (see pkv_attn.h).
#include "pkv_attn.h"

namespace pkv {

hipError_t launch_attention_fp8_mask(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                     hipStream_t s) {
  return launch_attention_var<5>(tile_kind, dtype, head_dim, a, s);
}

}  // namespace pkv
