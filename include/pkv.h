/*
 * pkv.h -- C ABI of a paged-KV attention prefill library for AMD MI355X (gfx950).
 *
 * The library computes, for a batch of requests whose keys and values live in
 * a paged KV cache, masked softmax(sm_scale * Q K^T) V with grouped-query
 * heads, plus the per-row log-sum-exp, and merges partial (o, lse) states.
 *
 * Sources (web pages of the AMD-Ecosystem FlashInfer fork):
 *   PR #339 "Route non-causal windowed prefill to AITER's masked kernel",
 *     section "Why window_size_right stays -1": the sliding window keeps key j
 *     for query row i only when j + qo_len + window_left >= kv_len + i; it is
 *     left-only, anchored bottom-right and applied independently of causal;
 *     window_left = -1 means no window.  Section "What changed": a window at
 *     least as wide as the sequence is normalised to -1, with a signed compare.
 *   PR #362 "Support speculative-decode verify on ROCm, and stop auto routing
 *     short-query prefill to AITER", Summary: the causal mask is bottom-right
 *     aligned (the last query row sees every key), which is exactly chain
 *     speculative-verify semantics: verify is a causal prefill whose
 *     qo_indptr advances by the draft length.  Review notes: kv_len comes from
 *     the paged metadata (indptr and last_page_len), and kv_len < qo_len under
 *     the causal mask gives a silently wrong answer.
 *   PR #399 "Refuse attention inputs the ROCm kernels would compute wrongly",
 *     What changed: strided last dimensions, run() tensors that disagree with
 *     plan() (token counts are minimums), and head counts the GQA group cannot
 *     divide (or zero kv heads) are refused; a rejected plan leaves the
 *     previous one usable; partial (o, lse) states are merged in place.
 *
 * Conventions for every entry point:
 *   - Host arrays are read during the call only; nothing keeps a view of them.
 *   - Device pointers are caller-owned (allocated by PyTorch or hipMalloc).
 *   - `stream` is a hipStream_t (NULL = the default stream); all device work is
 *     stream-ordered on it and no call synchronises the host with the device.
 *   - Strides are in elements; the last (head_dim) dimension is always packed.
 *     Device base pointers must be 16-byte aligned and token / head / page
 *     strides multiples of 8 elements (16-byte vector loads).
 *   - A refused call returns a non-zero status before any device write or
 *     kernel launch; pkv_last_error() then names the field, the expected value
 *     and the given value.
 */
#ifndef PKV_H_
#define PKV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_OK = 0,
  PKV_EINVAL = 1,      /* argument out of range (lengths, window, page ids, dtype, ...) */
  PKV_ELAYOUT = 2,     /* stride / alignment / packing not supported */
  PKV_EGQA = 3,        /* num_qo_heads not a positive multiple of num_kv_heads */
  PKV_EMISMATCH = 4,   /* run() tensors disagree with the plan */
  PKV_ENOTPLANNED = 5, /* plan handle missing or built without a workspace */
  PKV_EHIP = 6,        /* a HIP runtime call failed */
  PKV_EWORKSPACE = 7   /* workspace missing or too small */
} pkv_status;

typedef enum { PKV_FP16 = 0, PKV_BF16 = 1, PKV_FP32 = 2, PKV_FP8_E4M3 = 3 } pkv_dtype;

typedef struct pkv_plan_s* pkv_plan_t;

/* Optional plan knobs (pass NULL for the defaults). */
typedef struct {
  /* 0: the scheduler chooses how many KV chunks each query tile is split into.
     >0: split every request's keys [0, kv_len) into this many equal chunks in
     the request's own key coordinates (sizes rounded up to the key tile), each
     chunk producing a partial (o, lse) that run() merges. */
  int32_t num_kv_chunks;
  /* Restrict every request to keys in [kv_begin, kv_end) of its own key
     coordinates (kv_end < 0: no upper limit).  The mask is still evaluated in
     those coordinates, so the result is the partial state of that key range:
     rows that see no key there get o = 0 and lse = -inf. */
  int32_t kv_begin;
  int32_t kv_end;
  /* 0: automatic; 1: prefill tile (128 packed rows x 64 keys);
     2: short-query tile (16 or 32 packed rows x 128 keys). */
  int32_t tile;
  /* > 0: split every task's key range into chunks of this many key tiles
     (partials merged by run), instead of the automatic choice; 0: automatic. */
  int32_t split_tiles;
  int32_t reserved[3];
  /* Topology mask for tree-draft verification (PR #362, Architecture /
     design notes: a causal mask verifies chain drafts only, tree drafts need
     a custom mask).  Host arrays, or NULL for none.  Request b's mask is the
     row-major [qo_len, kv_len] bit matrix (query i, key j) -> bit
     i * kv_len + j, little-endian within each byte (bit k in byte k / 8 at
     bit k % 8), starting at byte mask_indptr[b]; mask_indptr has batch + 1
     non-decreasing entries, each segment holding at least
     ceil(qo_len * kv_len / 8) bytes, mask_indptr[batch] <= 2^28.  Key j is
     attended by row i when its bit is set and the left window (if any)
     allows it; causal must be 0 (the mask replaces it).  The plan copies the
     bits into its int workspace. */
  const uint8_t* custom_mask;
  const int64_t* mask_indptr;
  /* Logits soft-cap (PR #362, Architecture / design notes and per-commit
     messages gate on it; the formula is the reading taken): with cap > 0
     every scaled logit s = sm_scale * q.k becomes cap * tanh(s / cap) before
     the softmax, and lse is taken over the capped logits.  0: no cap.
     Caps up to 1024 evaluate tanh as 1 - 2 / (1 + e^(2y)), whose capped
     logit is within about 2e-7 * cap of the exact one; larger caps switch
     to a Taylor series near 0 (relative error below 1e-6). */
  float logits_soft_cap;
  /* K/V cache format (PR #362, per-commit messages: fp8 prefill on the
     paged route; the format is the reading taken).  0: the query dtype.
     PKV_FP8_E4M3: one byte per element, OCP E4M3 (bias 7, no infinities,
     S.1111.111 NaN); key and value values are code * k_scale and
     code * v_scale (0 means 1).  Cache strides are then in bytes and must be
     multiples of 16.  Combines with custom_mask and logits_soft_cap (the
     capped logit is sm_scale * q.k over the decoded keys).  q and o stay in
     the pkv_run dtype. */
  int32_t kv_dtype;
  float k_scale;
  float v_scale;
} pkv_plan_options;

/* Scheduling summary of a plan. */
typedef struct {
  int64_t total_q_rows;      /* qo_indptr[batch] */
  int64_t num_page_indices;  /* kv_indptr[batch] */
  int32_t batch_size;
  int32_t num_work_items;    /* attention work-group tasks */
  int32_t num_merge_items;   /* query tiles whose KV was split */
  int32_t num_partial_slots; /* fp32 partial states in the float workspace */
  int32_t tile_rows;         /* packed (position, head) rows per task */
  int32_t tile_keys;         /* keys per inner iteration */
  int32_t max_page_index;    /* largest page id referenced (-1 if none) */
  int32_t has_device_copy;   /* 1 when built with a workspace (runnable) */
  int64_t int_ws_bytes;
  int64_t float_ws_bytes;
  int64_t total_kv_len;      /* sum of the requests' kv_len (rows of a debug gather) */
} pkv_plan_info;

/*
 * Workspace sizes for a plan with these arguments (host-only; no device call).
 * Arguments are those of pkv_plan.  Fails with the same refusals as pkv_plan.
 */
pkv_status pkv_workspace_size(const int32_t* qo_indptr, const int32_t* kv_indptr,
                              const int32_t* kv_page_indices, int64_t num_indices,
                              const int32_t* kv_last_page_len, int32_t batch_size,
                              int32_t num_qo_heads, int32_t num_kv_heads,
                              int32_t head_dim, int32_t page_size, int32_t causal,
                              int32_t window_left, const pkv_plan_options* opts,
                              size_t* int_ws_bytes, size_t* float_ws_bytes);

/*
 * plan: validate the batch and schedule it.
 *   qo_indptr[batch+1]   host; request b owns query rows [qo_indptr[b], qo_indptr[b+1]).
 *   kv_indptr[batch+1]   host; request b owns page-table entries [kv_indptr[b], kv_indptr[b+1]).
 *   kv_page_indices[num_indices]  host; physical page ids.  num_indices must
 *                        equal kv_indptr[batch] (the page table's length).
 *   kv_last_page_len[batch]  host; keys on the request's last page, in [1, page_size]
 *                        when it has a page.  kv_len = (pages - 1) * page_size + last.
 *   num_qo_heads / num_kv_heads: q head h reads kv head h / (num_qo_heads / num_kv_heads).
 *   head_dim in {64, 128, 256} (256: prefill tile only); page_size >= 1;
 *   causal 0/1 (bottom-right aligned);
 *   window_left >= -1 (-1 = no window); sm_scale finite and > 0 (the kernels take
 *   each row's maximum before scaling); dtype PKV_FP16 or PKV_BF16.
 *   int_ws / float_ws: device workspaces of at least the sizes pkv_workspace_size
 *   reports.  The plan writes its task list into int_ws (one async copy on
 *   `stream`) and run() keeps fp32 partial states in float_ws: both must stay
 *   allocated and otherwise untouched while the plan is in use.  int_ws = NULL
 *   with int_ws_bytes = 0 builds a host-only plan (inspectable, not runnable).
 *   The upload is built outside stream capture: a runnable plan on a stream
 *   that is capturing is refused (pkv_run may be captured).
 * Refused (no handle is returned, earlier plans stay valid): decreasing indptr,
 *   indptr[0] != 0, kv_indptr[batch] != num_indices, last_page_len out of
 *   range, negative page ids, head counts GQA cannot divide, head_dim not
 *   64/128/256, window_left < -1, sm_scale <= 0 or not finite, a causal request
 *   with kv_len < qo_len, a request with query rows and no key, a too-small
 *   workspace, a capturing stream.
 * On success *out_plan owns a copy of everything it needs; free it with
 * pkv_plan_destroy.
 */
pkv_status pkv_plan(const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_page_indices, int64_t num_indices,
                    const int32_t* kv_last_page_len, int32_t batch_size,
                    int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t page_size, int32_t causal, int32_t window_left,
                    float sm_scale, pkv_dtype dtype, void* int_ws, size_t int_ws_bytes,
                    void* float_ws, size_t float_ws_bytes, void* stream,
                    const pkv_plan_options* opts, pkv_plan_t* out_plan);

/*
 * run: attention over the planned batch.
 *   q  [q_rows, q_heads, q_dim] at q + row*q_s_tok + head*q_s_head (+ d).
 *   k, v: paged pools, logical order [pages, page_size, heads, head_dim] at
 *     base + page*s_page + slot*s_tok + head*s_head (+ d): NHD, HND and
 *     combined K/V caches are all views of this with the right strides.
 *   o  [o_rows, num_qo_heads, head_dim] packed, in dtype; row r of request b is
 *     o[qo_indptr[b] + r].
 *   lse [lse_rows, num_qo_heads] packed fp32, natural log; NULL to skip
 *     (lse_rows is then ignored).
 * Shapes are checked against the plan: heads, head_dim (q, k, v separately),
 * page_size and dtype must match; q_rows, o_rows and lse_rows are minimums
 * (callers pad); every referenced page id must be below k_pages and v_pages.
 * A run uses its plan's workspaces (fp32 partials of split query tiles in
 * float_ws; in int_ws a task counter that is back at zero when the launch
 * ends), so runs of one plan must not overlap (one stream, or synchronised
 * streams); runs of different plans may.
 */
pkv_status pkv_run(pkv_plan_t plan,
                   const void* q, int64_t q_rows, int32_t q_heads, int32_t q_dim,
                   int64_t q_s_tok, int64_t q_s_head,
                   const void* k, int64_t k_pages, int32_t k_page_size, int32_t k_heads,
                   int32_t k_dim, int64_t k_s_page, int64_t k_s_tok, int64_t k_s_head,
                   const void* v, int64_t v_pages, int32_t v_page_size, int32_t v_heads,
                   int32_t v_dim, int64_t v_s_page, int64_t v_s_tok, int64_t v_s_head,
                   pkv_dtype dtype, void* o, int64_t o_rows, float* lse, int64_t lse_rows,
                   void* stream);

/*
 * merge_states: combine two partial attention states over disjoint key sets
 * (PR #399, What changed / graph-mode partial_state merge; PR #362's split-KV
 * tests).  With M = max(lse_a, lse_b), w_x = exp(lse_x - M):
 *   o = (w_a o_a + w_b o_b) / (w_a + w_b),  lse = M + log(w_a + w_b);
 * two -inf inputs give (0, -inf), and a -inf side leaves the other unchanged.
 *   o_a, o_b, o_out: [rows, heads, head_dim] packed, dtype PKV_FP16/BF16/FP32.
 *   lse_a, lse_b, lse_out: [rows, heads] packed fp32 (natural log).
 * o_out / lse_out may alias o_a / lse_a (in-place merge).  Device pointers.
 */
pkv_status pkv_merge_states(const void* o_a, const float* lse_a, const void* o_b,
                            const float* lse_b, void* o_out, float* lse_out,
                            int64_t rows, int32_t heads, int32_t head_dim,
                            pkv_dtype dtype, void* stream);

/*
 * append_kv: write new key/value rows into a paged cache, the step before an
 * attention call over the same page table (PR #399, per-commit messages, the
 * torch.compile aliasing commit: an append writes scattered pages).  Token t
 * belongs to request batch_indices[t] at logical position positions[t] and
 * lands on page kv_page_indices[kv_indptr[b] + positions[t] / page_size],
 * slot positions[t] % page_size; K and V rows are copied bit for bit.  The
 * caller owns kv_last_page_len: a position may lie anywhere on the request's
 * pages.  Two tokens naming one slot race (the surviving row is unspecified).
 * The kernel runs on `stream` and, like every entry point, does not
 * synchronise.
 *   append_k, append_v: [num_tokens, num_kv_heads, head_dim] device arrays
 *     (token / head strides in elements, head_dim packed).
 *   batch_indices, positions [num_tokens], kv_indptr [batch_size + 1],
 *     kv_page_indices [num_indices]: device int32 arrays.
 *   k, v: page pools as in pkv_run, written in place.
 *   err_count: optional device int32, incremented once for every token whose
 *     request, position, page-table entry or page id is out of range; such a
 *     token is skipped and nothing outside the arrays is read or written.
 * Refused on the host: dtype not fp16/bf16, head_dim not a positive multiple
 * of 8, k and v shapes that differ, strides or alignment as for pkv_run.
 */
pkv_status pkv_append_kv(const void* append_k, int64_t ak_s_tok, int64_t ak_s_head,
                         const void* append_v, int64_t av_s_tok, int64_t av_s_head,
                         int64_t num_tokens, int32_t num_kv_heads, int32_t head_dim,
                         const int32_t* batch_indices, const int32_t* positions,
                         const int32_t* kv_indptr, int32_t batch_size,
                         const int32_t* kv_page_indices, int64_t num_indices,
                         void* k, int64_t k_pages, int32_t k_page_size, int64_t k_s_page,
                         int64_t k_s_tok, int64_t k_s_head,
                         void* v, int64_t v_pages, int32_t v_page_size, int64_t v_s_page,
                         int64_t v_s_tok, int64_t v_s_head,
                         pkv_dtype dtype, int32_t* err_count, void* stream);

/*
 * chain_speculative_sampling: accept or reject each request's chain of draft
 * tokens against the target model's probabilities, the step after verify
 * (PR #362, Summary and Architecture / design notes: the acceptance sampler
 * runs over (batch_size, num_speculate_tokens) and handles chain drafts only).
 * For request b and draft position t with drafted token x: accept while
 * accept_u[b][t] * draft_probs[b][t][x] < target_probs[b][t][x] (float32);
 * at the first rejection emit one token drawn from max(target - draft, 0)
 * at that position (the target row itself if that is all zero) and stop; if
 * all are accepted, emit a bonus token drawn from target_probs[b][n].  A draw
 * takes the smallest index whose running weight sum exceeds
 * sample_u[b] * (total weight), else the last index with positive weight.
 * The pages name the step without its formulas; this is standard
 * speculative (rejection) sampling with the randomness passed in.
 *   draft_probs [batch][n][vocab], target_probs [batch][n + 1][vocab],
 *   accept_u [batch][n], sample_u [batch]: packed device float32 arrays;
 *   draft_token_ids [batch][n]: device int32 (an id outside [0, vocab) is
 *   rejected, never read).
 *   output_token_ids [batch][n + 1]: device int32, the accepted drafts, the
 *   drawn token, then -1; num_accepted [batch]: device int32.
 *   workspace: device scratch of at least
 *   pkv_chain_speculative_sampling_workspace_size(batch, vocab) bytes,
 *   16-byte aligned, not read before it is written; calls that share a
 *   workspace must be ordered on one stream.
 * Refused on the host: batch < 0, n < 0, vocab outside [1, 2^20], NULL
 * pointers when batch > 0, pointers not 4-byte aligned, a small or
 * unaligned workspace.
 */
pkv_status pkv_chain_speculative_sampling(const float* draft_probs,
                                          const int32_t* draft_token_ids,
                                          const float* target_probs, const float* accept_u,
                                          const float* sample_u, int32_t batch,
                                          int32_t num_speculate_tokens, int32_t vocab_size,
                                          int32_t* output_token_ids, int32_t* num_accepted,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream);

/* Device workspace bytes pkv_chain_speculative_sampling needs (per-tile sums
   of the drawn rows): batch * ceil(vocab / 1024) * 16.  Host-only. */
size_t pkv_chain_speculative_sampling_workspace_size(int32_t batch_size, int32_t vocab_size);

/*
 * chain_speculative_sampling without a workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, rule, kernels and results
 * as pkv_chain_speculative_sampling, minus the workspace: the per-tile sums
 * live in a 4 MiB array the library holds on each GPU it runs on (the GPU of
 * `stream`, the current one for the null stream; from the first call on that
 * GPU until the process ends).  Nothing is allocated by
 * this call.  Limit: batch * ceil(vocab / 1024) <= 262144 tiles (e.g. batch
 * 256 at a 2^20 vocabulary); larger sizes are refused (PKV_EINVAL) before any
 * device call.  Every call on one GPU shares that array, and each call writes
 * every entry it reads before reading it: calls on one GPU must be ordered
 * (one stream, or synchronised streams) -- calls that overlap on one GPU race.
 * The first call on each GPU looks up the array's device address
 * (hipGetSymbolAddress, with that GPU made current for the lookup and the
 * caller's current device restored): make it outside graph capture.
 */
pkv_status pkv_chain_speculative_sampling_no_alloc(const float* draft_probs,
                                                   const int32_t* draft_token_ids,
                                                   const float* target_probs,
                                                   const float* accept_u, const float* sample_u,
                                                   int32_t batch, int32_t num_speculate_tokens,
                                                   int32_t vocab_size, int32_t* output_token_ids,
                                                   int32_t* num_accepted, void* stream);

/*
 * debug_gather: the attention kernel's own page gathering, for bit-exact
 * checks (PR #362, Review notes: kv_len and every key address come from the
 * paged metadata; PR #399, What changed: token, page and head strides are
 * honoured).  It launches the kernel pkv_run launches for this plan -- same
 * task list, tile shape, page addressing, loads, waits and barriers -- but
 * instead of attending, each K/V tile that lands in LDS is written out
 * (un-swizzled) to k_out / v_out, packed [total_kv_len, kv_heads, head_dim]
 * in request order (request b's key j at row kv_out_start(b) + j, where
 * kv_out_start(b) is the sum of the kv_len of the requests before it).
 * Keys that no task of the plan loads (outside every row's causal / window
 * band, or outside a kv_begin / kv_end range) are left untouched, so the
 * caller pre-fills the outputs.  FP8 E4M3 caches give the decoded codes
 * (without k_scale / v_scale) in the plan's dtype.  Arguments as in pkv_run
 * (the plan's dtype); out_rows >= pkv_plan_info.total_kv_len.
 */
pkv_status pkv_debug_gather(pkv_plan_t plan,
                            const void* k, int64_t k_pages, int32_t k_page_size,
                            int32_t k_heads, int32_t k_dim, int64_t k_s_page,
                            int64_t k_s_tok, int64_t k_s_head,
                            const void* v, int64_t v_pages, int32_t v_page_size,
                            int32_t v_heads, int32_t v_dim, int64_t v_s_page,
                            int64_t v_s_tok, int64_t v_s_head, pkv_dtype dtype,
                            void* k_out, void* v_out, int64_t out_rows, void* stream);

/* Scheduling summary of a plan (host-only). */
pkv_status pkv_plan_get_info(pkv_plan_t plan, pkv_plan_info* info);

/*
 * Copy the plan's task list to host memory as int32 records of 8 fields:
 * {request, kv_head, row0, num_rows, kv_begin, kv_end, partial_slot, tile_begin}
 * in launch order (record i is work group i).  Rows are packed (position,
 * head-in-group) rows of that kv head; the task loads key tiles from
 * tile_begin (<= kv_begin, on the request's key-tile grid) up to kv_end and
 * masks keys below kv_begin; a partial_slot >= 0 marks one chunk of a split
 * query tile.  Lists grouped by XCD are padded with empty records
 * (num_rows 0, partial_slot -1).  Writes at most `capacity` records and
 * stores the total count in *count.  Host-only.
 */
pkv_status pkv_plan_get_work(pkv_plan_t plan, int32_t* out, int64_t capacity,
                             int64_t* count);

/* Release a plan (never touches the workspaces).  NULL is a no-op. */
void pkv_plan_destroy(pkv_plan_t plan);

/* Message of the last failed call on this thread ("" if none). */
const char* pkv_last_error(void);

/* Library version string. */
const char* pkv_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H_ */
