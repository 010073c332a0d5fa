// Attention kernel instantiations over FP8 E4M3 K/V caches with the custom topology mask and logits soft-cap
// (see pkv_attn.h).
#include "pkv_attn.h"

namespace pkv {

hipError_t launch_attention_fp8_mask_cap(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                         hipStream_t s) {
  return launch_attention_var<7>(tile_kind, dtype, head_dim, a, s);
}

}  // namespace pkv
