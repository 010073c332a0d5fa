// Internal types shared by the host scheduler (pkv_host.cpp) and the HIP
// kernels (pkv_kernels.hip).  Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Per-request facts the kernels need (all derived and validated by plan).
struct ReqInfo {
  int32_t qo_start;      // first query row of the request in q / o
  int32_t qo_len;        // query rows
  int32_t kv_len;        // keys: (pages - 1) * page_size + last_page_len
  int32_t page_off;      // first page-table entry of the request
  int32_t window;        // window_left after normalisation (-1 = no window)
  int32_t kv_out_start;  // first row of the request in a debug gather output
  int32_t mask_off;      // custom mask: byte offset of the request's bits
  int32_t mask_full;     // custom mask: keys [0, mask_full) are set for every row
};

// One work-group task: a tile of packed (position, head-in-group) rows of one
// kv head of one request, against keys [tile_begin, kv_end) loaded tile by
// tile; keys below key_lo or at/after kv_end are masked.  slot >= 0 sends the
// result to fp32 partial slot `slot` (one chunk of a split query tile).
struct WorkItem {
  int32_t b, kvh, row0, nrows;
  int32_t key_lo, kv_end, slot, tile_begin;
};

// A query tile whose keys were split over `nslots` consecutive partial slots.
struct MergeItem {
  int32_t b, kvh, row0, nrows;
  int32_t slot0, nslots, pad0, pad1;
};

// Tile shapes the kernels are instantiated for.
enum TileKind : int32_t {
  TILE_PREFILL = 1,   // 4 waves along rows: 128 rows x 64 keys per iteration
  TILE_SHORT16 = 2,   // 4 waves along keys: 16 rows x 128 keys per iteration
  TILE_SHORT32 = 3,   // 4 waves along keys: 32 rows x 128 keys per iteration
};

// Rows and keys per tile.  head_dim 256 has only the prefill kind, at 64
// rows x 32 keys (16 rows per wave keep its accumulators in registers).
inline int tile_rows(int kind, int head_dim) {
  if (head_dim == 256) return 64;
  return kind == TILE_PREFILL ? 128 : (kind == TILE_SHORT16 ? 16 : 32);
}
inline int tile_keys(int kind, int head_dim) {
  if (head_dim == 256) return 32;
  return kind == TILE_PREFILL ? 64 : 128;
}

// Multiply-shift constants for j / page_size over 0 <= j < 2^31: a power of
// two 2^l uses (1, l); otherwise m = floor(2^(31+l) / P) + 1 with
// l = ceil(log2 P) and shift 31 + l (round-up reciprocal; the error
// j * (m - 2^(31+l)/P) / 2^(31+l) stays below 1/P, so the floor is exact).
inline void page_divider(uint32_t page_size, uint32_t* magic, uint32_t* shift) {
  uint32_t l = 0;
  while ((1ull << l) < page_size) ++l;
  if ((1u << l) == page_size) {
    *magic = 1;
    *shift = l;
  } else {
    *magic = (uint32_t)(((1ull << (31 + l)) / page_size) + 1);
    *shift = 31 + l;
  }
}

struct AttnArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;              // nullable
  const int32_t* pages;    // device copy of kv_page_indices
  const ReqInfo* reqs;
  const WorkItem* work;
  const uint8_t* mask;     // custom mask bits (device copy), or nullptr
  float* part_o;           // [slots][tile_rows][head_dim] fp32
  float* part_lse;         // [slots][tile_rows] fp32, log2 domain
  int64_t q_s_tok, q_s_head;
  // pool strides in elements; the host guarantees that every in-page offset
  // (slot * s_tok + head * s_head + head_dim) fits in 31 bits
  uint32_t k_s_page, k_s_tok, k_s_head;
  uint32_t v_s_page, v_s_tok, v_s_head;
  int32_t num_work;
  int32_t group;           // num_qo_heads / num_kv_heads
  int32_t num_qo_heads;
  int32_t page_size;
  // page index of key j: (j * page_magic) >> page_shift, exact for 0 <= j < 2^31
  uint32_t page_magic;
  uint32_t page_shift;
  int32_t causal;
  float scale_log2;        // sm_scale * log2(e)
  // logits soft-cap, log2 domain: s' = cap_out * tanh(raw * cap_in)
  // = cap * log2(e) * tanh(sm_scale * raw / cap); cap_out = 0: no cap
  float cap_in;            // sm_scale / cap
  float cap_out;           // cap * log2(e)
  int32_t cap_series;      // 1: caps above 1024, tanh through its Taylor series near 0
  int32_t kv_fp8;          // 1: K/V are FP8 E4M3 codes (k_scale folded into scale_log2)
  float v_scale;           // FP8 V: value = code * v_scale
  // gather check only: [sum kv_len, Hkv, D] outputs of the K and V tiles as loaded
  void* gather_k;
  void* gather_v;
  // dyn_base > 0: work groups dyn_base.. take tasks dyn_base.. in the order
  // they start, from the counter dyn_next (zero between launches: the group
  // that takes the last task puts it back)
  int32_t dyn_base;
  int32_t* dyn_next;
};

struct SplitMergeArgs {
  void* o;
  float* lse;              // nullable
  const ReqInfo* reqs;
  const MergeItem* items;
  const float* part_o;
  const float* part_lse;
  int32_t num_items;
  int32_t group;
  int32_t num_qo_heads;
  int32_t tile_rows;
};

struct AppendArgs {
  const void* ak;
  const void* av;
  void* k;
  void* v;
  const int32_t* batch_indices;
  const int32_t* positions;
  const int32_t* kv_indptr;
  const int32_t* pages;
  int32_t* err_count;      // nullable
  int64_t num_tokens, num_indices, num_pages;
  int64_t ak_s_tok, ak_s_head, av_s_tok, av_s_head;
  uint32_t k_s_page, k_s_tok, k_s_head;
  uint32_t v_s_page, v_s_tok, v_s_head;
  int32_t heads, head_dim, batch, page_size;
  uint32_t page_magic, page_shift;
};

struct SampleArgs {
  const float* draft_probs;    // [batch][num_spec][vocab]
  const int32_t* draft_ids;    // [batch][num_spec]
  const float* target_probs;   // [batch][num_spec + 1][vocab]
  const float* accept_u;       // [batch][num_spec]
  const float* sample_u;       // [batch]
  int32_t* out_ids;            // [batch][num_spec + 1]
  int32_t* num_accepted;       // [batch]
  int32_t batch, num_spec, vocab;
};

// dtype: 0 fp16, 1 bf16, 2 fp32 (merge_states only).
hipError_t launch_attention(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                            hipStream_t stream);
// variants of launch_attention, one per file: custom mask, soft-cap, both
hipError_t launch_attention_mask(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                 hipStream_t stream);
hipError_t launch_attention_cap(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                hipStream_t stream);
hipError_t launch_attention_mask_cap(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                     hipStream_t stream);
// FP8 E4M3 K/V caches: plain, custom mask, soft-cap, both
hipError_t launch_attention_fp8(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                hipStream_t stream);
hipError_t launch_attention_fp8_mask(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                     hipStream_t stream);
hipError_t launch_attention_fp8_cap(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                    hipStream_t stream);
hipError_t launch_attention_fp8_mask_cap(int tile_kind, int dtype, int head_dim,
                                         const AttnArgs& a, hipStream_t stream);
hipError_t launch_split_merge(int dtype, int head_dim, const SplitMergeArgs& a,
                              hipStream_t stream);
hipError_t launch_merge_states(int dtype, const void* o_a, const float* lse_a,
                               const void* o_b, const float* lse_b, void* o_out,
                               float* lse_out, int64_t rows, int32_t heads,
                               int32_t head_dim, hipStream_t stream);
// the gather check: the attention kernel's task list and loads, every landed
// K/V tile copied out to a.gather_k / a.gather_v (plain or FP8 caches)
hipError_t launch_attention_dump(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                 hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, hipStream_t stream);
// bytes (a multiple of 16) from device-visible pinned host memory to device memory
hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t stream);
size_t spec_sample_workspace_bytes(int32_t batch, int32_t vocab);
hipError_t launch_spec_sample(const SampleArgs& a, void* workspace, hipStream_t stream);
// Size of the library's own per-device tile-sum array (allocation-free
// sampling entry point) and its device address on the GPU that runs `stream`.
constexpr size_t kSpecScratchBytes = size_t(4) << 20;
hipError_t spec_sample_scratch(hipStream_t stream, void** ptr);

}  // namespace pkv
