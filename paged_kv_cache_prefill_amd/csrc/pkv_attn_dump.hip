// Gather-check instantiations of the attention kernel (see pkv_attn.h, VAR bit
// 3): the production task list, page addressing, loads, waits and barriers of
// the plain and FP8 kernels, with every landed K/V tile copied out of LDS
// instead of attended, so that page gathering can be compared bit for bit.
#include "pkv_attn.h"

namespace pkv {

hipError_t launch_attention_dump(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                 hipStream_t s) {
  if (a.kv_fp8) return launch_attention_var<12>(tile_kind, dtype, head_dim, a, s);
  return launch_attention_var<8>(tile_kind, dtype, head_dim, a, s);
}

}  // namespace pkv
