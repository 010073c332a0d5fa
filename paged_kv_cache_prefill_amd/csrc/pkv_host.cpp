// Host side of the paged-KV attention prefill library: argument validation,
// the scheduler that turns a batch into work-group tasks, and the C ABI.
//
// Sources (web pages of the AMD-Ecosystem FlashInfer fork):
//   PR #362 "Support speculative-decode verify on ROCm, and stop auto routing
//     short-query prefill to AITER", Review notes: kv_len is derived from the
//     paged metadata (kv_indptr and last_page_len), and a causal request whose
//     kv_len is below its qo_len gives a silently wrong answer on the batch
//     paged path.  Architecture notes: the graph-mode row bound
//     total_num_rows - batch_size + 1 inflates tiles; this planner sees every
//     request's lengths and needs no such bound.
//   PR #339 "Route non-causal windowed prefill to AITER's masked kernel",
//     What changed: a window at least as wide as the sequence is normalised
//     to -1 (with a signed compare); the batch planner there could not do it
//     per request because it knew only the maximum kv_len.  This one does.
//   PR #399 "Refuse attention inputs the ROCm kernels would compute
//     wrongly", What changed / Architecture notes: strided last dimensions,
//     head counts the GQA group cannot divide (and zero kv heads), and run()
//     tensors that disagree with plan() are refused; token counts are
//     minimums because graph callers pad; validation precedes the first
//     write so a rejected plan leaves earlier plans usable; the plan keeps its
//     own copy of every host array (a kept view of a caller's CPU indptr gave
//     wrong answers there).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <functional>
#include <numeric>
#include <string>
#include <vector>

#include "../../include/pkv.h"
#include "pkv_internal.h"

using namespace pkv;

namespace {

thread_local std::string g_err;

pkv_status fail(pkv_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

const char* dtype_name(int d) {
  return d == PKV_FP16 ? "fp16" : d == PKV_BF16 ? "bf16" : d == PKV_FP32 ? "fp32"
       : d == PKV_FP8_E4M3 ? "fp8_e4m3" : "unknown";
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

constexpr int kNumCUs = 256;               // MI355X compute units
constexpr int kTargetTasks = 2 * kNumCUs;  // work groups wanted per launch

struct Schedule {
  int32_t batch = 0, hq = 0, hkv = 0, group = 0, head_dim = 0, page_size = 0;
  int32_t causal = 0, window_left = -1, tile_kind = 0, rows = 0, keys = 0;
  int64_t total_q = 0, num_indices = 0, total_kv = 0;
  int32_t max_page = -1, max_kv_len = 0, num_slots = 0;
  std::vector<ReqInfo> reqs;
  std::vector<WorkItem> work;
  std::vector<MergeItem> merges;
  // int workspace layout
  size_t off_reqs = 0, off_work = 0, off_merge = 0, off_dyn = 0, off_pages = 0, int_bytes = 0;
  int32_t dyn_base = 0;   // > 0: tasks from here on are taken in work-group start order
  size_t off_mask = 0, mask_bytes = 0;   // custom mask bits (0 bytes: none)
  // float workspace layout
  size_t off_part_lse = 0, float_bytes = 0;
};

// Bits [bit0, bit0 + n) of a little-endian packed mask are all set?  Returns
// the index (relative to bit0) of the first clear bit, or n.
int64_t first_clear_bit(const uint8_t* m, int64_t bit0, int64_t n) {
  int64_t k = 0;
  while (k < n && ((bit0 + k) & 7) != 0) {
    if (!((m[(bit0 + k) >> 3] >> ((bit0 + k) & 7)) & 1)) return k;
    ++k;
  }
  while (k + 64 <= n) {   // whole bytes, eight at a time
    uint64_t w;
    std::memcpy(&w, m + ((bit0 + k) >> 3), 8);
    if (w != ~0ull) break;
    k += 64;
  }
  for (; k < n; ++k)
    if (!((m[(bit0 + k) >> 3] >> ((bit0 + k) & 7)) & 1)) return k;
  return n;
}

// Validate the custom mask of a plan and record, per request, the byte offset
// of its bits and the length of the key prefix every row keeps (those key
// tiles need no per-element test).
pkv_status check_custom_mask(const pkv_plan_options& o, int32_t batch, int32_t causal,
                             Schedule* S) {
  if (!o.custom_mask || !o.mask_indptr)
    return fail(PKV_EINVAL, "custom_mask / mask_indptr: expected both or neither, given %s",
                o.custom_mask ? "no mask_indptr" : "no custom_mask");
  if (causal)
    return fail(PKV_EINVAL, "causal: expected 0 with a custom mask (the mask replaces it), "
                            "given 1");
  if (batch > 0 && o.mask_indptr[0] < 0)
    return fail(PKV_EINVAL, "mask_indptr[0]: expected >= 0, given %lld",
                (long long)o.mask_indptr[0]);
  for (int32_t b = 0; b < batch; ++b) {
    const ReqInfo& r = S->reqs[b];
    const int64_t need = ((int64_t)r.qo_len * r.kv_len + 7) / 8;
    const int64_t have = o.mask_indptr[b + 1] - o.mask_indptr[b];
    if (have < need)
      return fail(PKV_EINVAL, "mask_indptr: request %d needs >= %lld bytes (qo_len=%d x kv_len=%d "
                              "bits), given %lld", b, (long long)need, r.qo_len, r.kv_len,
                  (long long)have);
  }
  const int64_t total = batch > 0 ? o.mask_indptr[batch] : 0;
  if (total > (1ll << 28))
    return fail(PKV_EINVAL, "mask_indptr[%d]: expected <= 2^28 bytes, given %lld", batch,
                (long long)total);
  for (int32_t b = 0; b < batch; ++b) {
    ReqInfo& r = S->reqs[b];
    r.mask_off = (int32_t)o.mask_indptr[b];
    int64_t full = r.kv_len;
    for (int32_t i = 0; i < r.qo_len && full > 0; ++i)
      full = first_clear_bit(o.custom_mask, (int64_t)r.mask_off * 8 + (int64_t)i * r.kv_len, full);
    r.mask_full = (int32_t)full;
  }
  S->mask_bytes = (size_t)total;
  return PKV_OK;
}

struct RowTask {
  int32_t b, kvh, row0, nrows;
  int32_t key_lo, key_hi;  // inclusive visible key range of the task (key_lo > key_hi: none)
  int32_t tile_begin;
};

// Temporaries of the scheduler, kept per thread so that their capacity is
// reused from one plan to the next (a plan is otherwise dominated by
// allocation and first-touch of these arrays).
struct SchedScratch {
  std::vector<int64_t> hist, rem, cnt, pieces, gcost;
  std::vector<int32_t> start, gid, gorder, gxcd, costs;
  std::vector<RowTask> tasks;
  std::vector<WorkItem> items;
  std::vector<std::pair<int32_t, int32_t>> chunks;
};
thread_local SchedScratch g_scr;

// Chunk size (key tiles) for the automatic split of a launch with few tasks:
// the candidate whose longest-first schedule over `slots` concurrent work
// groups ends first, each work item costing its key tiles plus kItemTiles
// (its start-up latency and, when split, its share of the merge; fitted on
// the short-query verify batches), if it beats the even-share size
// `fallback` by 10%.  0 = no split.
constexpr int64_t kItemTiles = 4;
int64_t choose_chunk_tiles(const std::vector<int64_t>& pieces, int64_t slots, int64_t min_tiles,
                           int64_t fallback) {
  int64_t longest = 0, total = 0;
  for (int64_t n : pieces) {
    longest = std::max(longest, n);
    total += std::max<int64_t>(n, 0);
  }
  if (longest <= 0 || slots <= 0) return 0;
  std::vector<int64_t>& hist = g_scr.hist;   // pieces by length
  hist.assign((size_t)longest + 1, 0);
  for (int64_t n : pieces)
    if (n > 0) ++hist[(size_t)n];
  std::vector<int64_t>& rem = g_scr.rem;     // remainders by length
  std::vector<int64_t>& cnt = g_scr.cnt;     // slots by load (offset from the lowest initial load)
  // Longest-first list schedule of the chunks of size c (c = 0: unsplit):
  // full chunks first (all the same size: dealt out evenly), then the shorter
  // remainders, longest first, each to a least loaded slot.  Loads only grow
  // from the minimum, so the minimum never decreases: slots are counted per
  // load value and a pointer walks up to the lowest occupied one, which gives
  // the same makespan as a heap in time linear in pieces and load range.
  auto makespan = [&](int64_t c) {
    const int64_t len = c > 0 ? c - 1 : longest;
    rem.assign((size_t)len + 1, 0);
    int64_t full = 0, work = 0;
    // q, r: n / c and n % c, stepped along with n (no division per length)
    for (int64_t n = 1, q = 0, r = 1; n <= longest; ++n, ++r) {
      if (c > 0 && r == c) {
        r = 0;
        ++q;
      }
      const int64_t h = hist[(size_t)n];
      if (h == 0) continue;
      full += h * q;
      rem[(size_t)r] += h;
      if (r > 0) work += h * (r + kItemTiles);
    }
    const int64_t per = c + kItemTiles, base = full / slots, extra = full % slots;
    const int64_t base_load = base * per;
    int64_t m = (base + (extra > 0 ? 1 : 0)) * per;
    // every assignment lands on a slot at most the average load above the
    // lowest initial load, plus one item
    const int64_t span = per + (work + slots - 1) / slots + len + kItemTiles + 2;
    cnt.assign((size_t)span, 0);
    cnt[0] = slots - extra;
    if (extra > 0) cnt[(size_t)per] += extra;
    int64_t lo = 0;
    for (int64_t r = len; r >= 1; --r) {
      int64_t left = rem[(size_t)r];
      while (left > 0) {
        while (cnt[(size_t)lo] == 0) ++lo;
        const int64_t t = std::min(left, cnt[(size_t)lo]);
        const int64_t to = lo + r + kItemTiles;
        cnt[(size_t)lo] -= t;
        cnt[(size_t)to] += t;
        m = std::max(m, base_load + to);
        left -= t;
      }
    }
    return m;
  };
  // the even-share chunk size is kept unless the model expects a schedule at
  // least 10% shorter (its estimates are only that good)
  const int64_t fallback_m = makespan(fallback);
  // Only a candidate below both the unsplit schedule and the fallback can be
  // returned, so the search starts from the lower of the two (same result).
  int64_t best = 0, best_m = std::min(makespan(0), fallback_m);
  for (int64_t c : {4, 6, 8, 12, 16, 24, 32, 48, 64, 96, 128}) {
    if (c < min_tiles || c >= longest) continue;
    // a full chunk exists (c < longest), so no schedule ends before one chunk
    if (c + kItemTiles >= best_m) continue;
    int64_t items = 0;   // far more items than slots never wins: skip those
    for (int64_t n = 1, k = 1, r = 1; n <= longest; ++n, ++r) {   // k = ceil(n / c)
      if (r > c) {
        r = 1;
        ++k;
      }
      items += hist[(size_t)n] * k;
    }
    if (items > 4 * slots) continue;
    // no schedule beats the average load: skip candidates that cannot win
    if ((total + items * kItemTiles + slots - 1) / slots >= best_m) continue;
    const int64_t m = makespan(c);
    if (m < best_m) {
      best = c;
      best_m = m;
    }
  }
  return best_m * 10 <= fallback_m * 9 ? best : fallback;
}


// Work-group i of a launch runs on XCD i % 8, and each XCD has its own L2.
// Tasks of one (request, kv head) read the same K/V rows, so when there are
// enough such groups they are bin-packed onto XCDs (largest group first, to
// the least loaded XCD) and each XCD's list is interleaved into slots x,
// x + 8, x + 16, ...; lists are padded with empty tasks (num_rows 0).  Within
// an XCD, and in the fallback with too few groups, tasks run longest first
// (a stable counting sort on the tile count), so the tail of the launch is
// made of short tasks.
constexpr int kNumXcds = 8;


// Returns true when it grouped tasks by XCD (the order must then stay fixed).
bool order_for_xcds(const std::vector<WorkItem>& items, const std::vector<int32_t>& costs,
                    int32_t batch, int32_t hkv, std::vector<WorkItem>* work) {
  SchedScratch& T = g_scr;
  const size_t n = items.size();
  int32_t max_cost = 0;
  for (int32_t c : costs) max_cost = std::max(max_cost, c);
  // positions of a stable sort by cost, largest first
  T.start.assign((size_t)max_cost + 2, 0);
  for (int32_t c : costs) ++T.start[max_cost - c + 1];
  for (int32_t c = 1; c <= max_cost + 1; ++c) T.start[c] += T.start[c - 1];
  auto longest_first = [&] {
    work->resize(n);
    for (size_t i = 0; i < n; ++i) (*work)[T.start[max_cost - costs[i]]++] = items[i];
    return false;
  };
  // Reuse exists only when a group has several query tiles (chunks of one
  // tile read disjoint keys).  Tasks of one tile are emitted consecutively.
  bool reuse = false;
  for (size_t i = 1; i < n && !reuse; ++i)
    reuse = items[i].b == items[i - 1].b && items[i].kvh == items[i - 1].kvh &&
            items[i].row0 != items[i - 1].row0;
  if (!reuse) return longest_first();
  // group costs, keyed by request * hkv + kv head
  T.gcost.assign((size_t)batch * hkv, 0);
  T.gid.resize(n);
  int64_t total = 0;
  for (size_t i = 0; i < n; ++i) {
    const int32_t g = items[i].b * hkv + items[i].kvh;
    T.gid[i] = g;
    T.gcost[g] += costs[i];
    total += costs[i];
  }
  int64_t groups = 0, gmax = 0;
  for (int64_t c : T.gcost) {
    groups += c > 0;
    gmax = std::max(gmax, c);
  }
  if (groups < 2 * kNumXcds || gmax * kNumXcds > total + total / 2) return longest_first();
  T.gorder.resize(T.gcost.size());
  std::iota(T.gorder.begin(), T.gorder.end(), 0);
  // largest group first, ties in group order
  std::sort(T.gorder.begin(), T.gorder.end(), [&](int32_t a, int32_t b) {
    return T.gcost[a] != T.gcost[b] ? T.gcost[a] > T.gcost[b] : a < b;
  });
  T.gxcd.assign(T.gcost.size(), 0);
  int64_t load[kNumXcds] = {0};
  for (int32_t g : T.gorder) {
    int best = 0;
    for (int x = 1; x < kNumXcds; ++x)
      if (load[x] < load[best]) best = x;
    T.gxcd[g] = best;
    load[best] += T.gcost[g];
  }
  // each XCD's list in longest-first order (ties in task order): walk the
  // tasks in the global stable order and deal each to its XCD's next slot
  size_t len[kNumXcds] = {0};
  for (size_t i = 0; i < n; ++i) ++len[T.gxcd[T.gid[i]]];
  size_t longest = 0;
  for (size_t l : len) longest = std::max(longest, l);
  T.pieces.resize(n);   // task index at each sorted position
  for (size_t i = 0; i < n; ++i) T.pieces[T.start[max_cost - costs[i]]++] = (int64_t)i;
  WorkItem empty{};  // num_rows 0: the kernel returns at once
  empty.slot = -1;
  work->assign(longest * kNumXcds, empty);
  size_t next[kNumXcds] = {0};
  for (size_t k = 0; k < n; ++k) {
    const size_t i = (size_t)T.pieces[k];
    const int x = T.gxcd[T.gid[i]];
    (*work)[next[x]++ * kNumXcds + x] = items[i];
  }
  return true;
}

// Smallest and largest page id (the plan scans every page-table entry; the
// AVX2 clone does it 8 entries per instruction where the host has AVX2).
__attribute__((target_clones("avx2", "default"))) void page_id_range(
    const int32_t* __restrict ids, int64_t n, int32_t* lo, int32_t* hi) {
  int32_t mn = *lo, mx = *hi;
  for (int64_t i = 0; i < n; ++i) {
    mn = std::min(mn, ids[i]);
    mx = std::max(mx, ids[i]);
  }
  *lo = mn;
  *hi = mx;
}

pkv_status schedule(const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_page_indices, int64_t num_indices,
                    const int32_t* kv_last_page_len, int32_t batch, int32_t hq, int32_t hkv,
                    int32_t head_dim, int32_t page_size, int32_t causal, int32_t window_left,
                    const pkv_plan_options* opts, Schedule* S) {
  if (batch < 0) return fail(PKV_EINVAL, "batch_size: expected >= 0, given %d", batch);
  if (num_indices < 0)
    return fail(PKV_EINVAL, "num_indices: expected >= 0, given %lld", (long long)num_indices);
  if (hkv <= 0)
    return fail(PKV_EGQA, "num_kv_heads: expected a positive head count, given %d", hkv);
  if (hq <= 0 || hq % hkv != 0)
    return fail(PKV_EGQA,
                "num_qo_heads: expected a positive multiple of num_kv_heads=%d, given %d", hkv,
                hq);
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PKV_EINVAL, "head_dim: expected 64, 128 or 256, given %d", head_dim);
  if (page_size < 1) return fail(PKV_EINVAL, "page_size: expected >= 1, given %d", page_size);
  if (causal != 0 && causal != 1)
    return fail(PKV_EINVAL, "causal: expected 0 or 1, given %d", causal);
  if (window_left < -1)
    return fail(PKV_EINVAL, "window_left: expected -1 (no window) or >= 0, given %d",
                window_left);
  if (batch > 0 && (!qo_indptr || !kv_indptr || !kv_last_page_len))
    return fail(PKV_EINVAL, "qo_indptr / kv_indptr / kv_last_page_len: expected host arrays, "
                            "given NULL");
  pkv_plan_options o{};
  o.kv_end = -1;
  if (opts) o = *opts;
  if (o.num_kv_chunks < 0)
    return fail(PKV_EINVAL, "opts.num_kv_chunks: expected >= 0, given %d", o.num_kv_chunks);
  if (o.kv_begin < 0) return fail(PKV_EINVAL, "opts.kv_begin: expected >= 0, given %d", o.kv_begin);
  if (o.kv_end >= 0 && o.kv_end < o.kv_begin)
    return fail(PKV_EINVAL, "opts.kv_end: expected >= kv_begin=%d or < 0, given %d", o.kv_begin,
                o.kv_end);
  if (o.tile < 0 || o.tile > 2)
    return fail(PKV_EINVAL, "opts.tile: expected 0, 1 or 2, given %d", o.tile);
  if (o.split_tiles < 0)
    return fail(PKV_EINVAL, "opts.split_tiles: expected >= 0, given %d", o.split_tiles);
  if (!(o.logits_soft_cap >= 0.f) || !std::isfinite(o.logits_soft_cap))
    return fail(PKV_EINVAL, "opts.logits_soft_cap: expected a finite value >= 0, given %g",
                (double)o.logits_soft_cap);
  if (o.kv_dtype != 0 && o.kv_dtype != PKV_FP8_E4M3)
    return fail(PKV_EINVAL, "opts.kv_dtype: expected 0 (the query dtype) or fp8_e4m3 (%d), given %d",
                (int)PKV_FP8_E4M3, o.kv_dtype);
  if (o.kv_dtype == PKV_FP8_E4M3) {
    for (float sc : {o.k_scale, o.v_scale})
      if (!(sc >= 0.f) || !std::isfinite(sc))
        return fail(PKV_EINVAL, "opts.k_scale / v_scale: expected finite values >= 0, given %g",
                    (double)sc);
  }
  const int64_t opt_end = o.kv_end < 0 ? INT64_MAX : o.kv_end;

  const int32_t qi0 = batch > 0 ? qo_indptr[0] : 0;
  const int32_t ki0 = batch > 0 ? kv_indptr[0] : 0;
  if (qi0 != 0) return fail(PKV_EINVAL, "qo_indptr[0]: expected 0, given %d", qi0);
  if (ki0 != 0) return fail(PKV_EINVAL, "kv_indptr[0]: expected 0, given %d", ki0);
  // the page table must be exactly as long as kv_indptr says: the scheduler
  // reads kv_indptr[batch] entries of it
  const int64_t kv_n = batch > 0 ? kv_indptr[batch] : 0;
  if (kv_n != num_indices)
    return fail(PKV_EINVAL, "num_indices: expected kv_indptr[%d]=%lld page-table entries, given %lld",
                batch, (long long)kv_n, (long long)num_indices);

  S->batch = batch;
  S->hq = hq;
  S->hkv = hkv;
  S->group = hq / hkv;
  S->head_dim = head_dim;
  S->page_size = page_size;
  S->causal = causal;
  S->window_left = window_left;
  S->reqs.assign(batch, ReqInfo{});
  int64_t max_rows = 0, kv_acc = 0;
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t ql = (int64_t)qo_indptr[b + 1] - qo_indptr[b];
    const int64_t np = (int64_t)kv_indptr[b + 1] - kv_indptr[b];
    if (ql < 0)
      return fail(PKV_EINVAL, "qo_indptr[%d]: expected >= qo_indptr[%d]=%d, given %d", b + 1, b,
                  qo_indptr[b], qo_indptr[b + 1]);
    if (np < 0)
      return fail(PKV_EINVAL, "kv_indptr[%d]: expected >= kv_indptr[%d]=%d, given %d", b + 1, b,
                  kv_indptr[b], kv_indptr[b + 1]);
    int64_t L = 0;
    if (np > 0) {
      const int32_t last = kv_last_page_len[b];
      if (last < 1 || last > page_size)
        return fail(PKV_EINVAL, "kv_last_page_len[%d]: expected in [1, page_size=%d], given %d",
                    b, page_size, last);
      L = (np - 1) * page_size + last;
    }
    if (L > INT32_MAX / 2)
      return fail(PKV_EINVAL, "kv_len of request %d: expected < 2^30, given %lld", b,
                  (long long)L);
    if (ql > 0 && L == 0)
      return fail(PKV_EINVAL, "request %d: expected kv_len >= 1 for qo_len=%lld, given kv_len=0",
                  b, (long long)ql);
    if (causal && L < ql)
      return fail(PKV_EINVAL,
                  "request %d: causal mask needs kv_len >= qo_len=%lld, given kv_len=%lld", b,
                  (long long)ql, (long long)L);
    if (ql * S->group > INT32_MAX / 2)
      return fail(PKV_EINVAL, "request %d: qo_len * group too large (%lld)", b,
                  (long long)(ql * S->group));
    ReqInfo& r = S->reqs[b];
    r.qo_start = qo_indptr[b];
    r.qo_len = (int32_t)ql;
    r.kv_len = (int32_t)L;
    r.page_off = kv_indptr[b];
    // A window of kv_len - 1 or more keeps every key (j >= i - qo_len + 1 - ...
    // <= 0 for every row): normalise it away per request, signed compare.
    r.window = (window_left >= 0 && (int64_t)window_left < L - 1) ? window_left : -1;
    r.kv_out_start = (int32_t)kv_acc;
    kv_acc += L;
    S->max_kv_len = std::max<int32_t>(S->max_kv_len, (int32_t)L);
    max_rows = std::max<int64_t>(max_rows, ql * S->group);
  }
  if (o.custom_mask || o.mask_indptr) {
    pkv_status ms = check_custom_mask(o, batch, causal, S);
    if (ms != PKV_OK) return ms;
  }
  S->total_q = batch > 0 ? qo_indptr[batch] : 0;
  S->num_indices = num_indices;
  S->total_kv = kv_acc;
  if (S->num_indices > 0 && !kv_page_indices)
    return fail(PKV_EINVAL, "kv_page_indices: expected %lld entries, given NULL",
                (long long)S->num_indices);
  {
    // one branch-free pass (min and max), then the first bad entry if any
    int32_t pmin = INT32_MAX, pmax = -1;
    page_id_range(kv_page_indices, S->num_indices, &pmin, &pmax);
    if (S->num_indices > 0 && pmin < 0)
      for (int64_t i = 0; i < S->num_indices; ++i)
        if (kv_page_indices[i] < 0)
          return fail(PKV_EINVAL, "kv_page_indices[%lld]: expected >= 0, given %d", (long long)i,
                      kv_page_indices[i]);
    S->max_page = pmax;
  }

  // ---- tile shape
  int kind;
  if (head_dim == 256 && o.tile == 2)
    return fail(PKV_EINVAL, "opts.tile: the short-query tile has no head_dim 256 form, given 2");
  if (o.tile == 1 || head_dim == 256) kind = TILE_PREFILL;
  else if (o.tile == 2) kind = max_rows <= 16 ? TILE_SHORT16 : TILE_SHORT32;
  else kind = max_rows <= 16 ? TILE_SHORT16 : (max_rows <= 32 ? TILE_SHORT32 : TILE_PREFILL);
  S->tile_kind = kind;
  S->rows = tile_rows(kind, head_dim);
  S->keys = tile_keys(kind, head_dim);
  const int MR = S->rows, NK = S->keys, G = S->group;
  // key tiles are 32, 64 or 128 keys: key offsets (never negative) divide by shifts
  const int nk_sh = __builtin_ctz((unsigned)NK);

  // ---- row tasks with their visible key ranges
  SchedScratch& T = g_scr;
  std::vector<RowTask>& tasks = T.tasks;
  tasks.clear();
  {
    int64_t n = 0;
    for (int32_t b = 0; b < batch; ++b) n += ((int64_t)S->reqs[b].qo_len * G + MR - 1) / MR;
    tasks.reserve((size_t)(n * hkv));
  }
  for (int32_t b = 0; b < batch; ++b) {
    const ReqInfo& r = S->reqs[b];
    const int32_t R = r.qo_len * G;
    const int32_t sh = r.kv_len - r.qo_len;
    for (int32_t kvh = 0; kvh < hkv; ++kvh) {
      for (int32_t row0 = 0; row0 < R; row0 += MR) {
        RowTask t;
        t.b = b;
        t.kvh = kvh;
        t.row0 = row0;
        t.nrows = std::min(MR, R - row0);
        const int32_t pmin = row0 / G, pmax = (row0 + t.nrows - 1) / G;
        int64_t lo = r.window >= 0 ? std::max<int64_t>(0, (int64_t)pmin + sh - r.window) : 0;
        int64_t hi = causal ? (int64_t)pmax + sh : (int64_t)r.kv_len - 1;
        hi = std::min<int64_t>(hi, r.kv_len - 1);
        lo = std::max<int64_t>(lo, o.kv_begin);
        hi = std::min<int64_t>(hi, opt_end - 1);
        t.key_lo = (int32_t)std::min<int64_t>(lo, INT32_MAX / 2);
        t.key_hi = (int32_t)std::max<int64_t>(hi, -1);
        t.tile_begin = t.key_lo <= t.key_hi ? (t.key_lo >> nk_sh) << nk_sh : 0;
        tasks.push_back(t);
      }
    }
  }

  // ---- split decision: fixed chunk boundaries when asked for, and when the
  // launch would have fewer than kTargetTasks work groups, the ranges are cut
  // into chunks of the size choose_chunk_tiles picks (partials are merged
  // either way)
  auto cost = [&](const RowTask& t) -> int64_t {
    return t.key_lo > t.key_hi ? 0 : (t.key_hi + 1 - t.tile_begin + NK - 1) >> nk_sh;
  };
  int64_t chunk_tiles = 0;  // 0: no automatic split
  {
    // pieces: the requested chunks each task's range meets, else the tasks
    std::vector<int64_t>& pieces = T.pieces;
    pieces.clear();
    for (const RowTask& t : tasks) {
      if (o.num_kv_chunks > 0 && t.key_lo <= t.key_hi) {
        const int64_t L = S->reqs[t.b].kv_len;
        int64_t clen = (L + o.num_kv_chunks - 1) / o.num_kv_chunks;
        clen = std::max<int64_t>(NK, ((clen + NK - 1) >> nk_sh) << nk_sh);
        for (int64_t c0 = t.key_lo / clen * clen; c0 <= t.key_hi; c0 += clen) {
          const int64_t a = std::max<int64_t>(c0, t.key_lo);
          const int64_t e = std::min<int64_t>(c0 + clen, (int64_t)t.key_hi + 1);
          pieces.push_back(e > a ? ((e - 1) >> nk_sh) - (a >> nk_sh) + 1 : 0);
        }
      } else {
        pieces.push_back(cost(t));
      }
    }
    if (o.split_tiles > 0) {
      chunk_tiles = o.split_tiles;
    } else if ((int64_t)pieces.size() < kTargetTasks) {
      // concurrent work groups: two per CU for the 128-row tile at head_dim
      // <= 128 (64 KB of LDS, two waves per SIMD), one otherwise
      const int64_t per_cu = (kind == TILE_PREFILL && head_dim <= 128) ? 2 : 1;
      const int64_t min_tiles = (kind == TILE_PREFILL) ? 8 : 4;
      int64_t total = 0;
      for (int64_t n : pieces) total += n;
      const int64_t even = std::max<int64_t>(min_tiles, (total + kTargetTasks - 1) / kTargetTasks);
      chunk_tiles = choose_chunk_tiles(pieces, per_cu * kNumCUs, min_tiles, even);
    }
  }
  std::vector<WorkItem>& items = T.items;
  std::vector<int32_t>& costs = T.costs;
  items.clear();
  costs.clear();
  std::vector<std::pair<int32_t, int32_t>>& chunks = T.chunks;  // [c0, c1) ranges of one task
  auto emit = [&](const RowTask& t, int32_t lo, int32_t end, int32_t tb, int32_t slot) {
    WorkItem w;
    w.b = t.b;
    w.kvh = t.kvh;
    w.row0 = t.row0;
    w.nrows = t.nrows;
    w.key_lo = lo;
    w.kv_end = end;
    w.slot = slot;
    w.tile_begin = tb;
    items.push_back(w);
    costs.push_back(end > tb ? (end - tb + NK - 1) >> nk_sh : 0);
  };
  int32_t slots = 0;
  const bool splitting = chunk_tiles > 0 || o.num_kv_chunks > 0;
  items.reserve(tasks.size());
  costs.reserve(tasks.size());
  if (splitting) S->merges.reserve(tasks.size());
  for (const RowTask& t : tasks) {
    if (!splitting) {   // one item per task, its whole visible range
      if (t.key_lo > t.key_hi)
        emit(t, 0, 0, 0, -1);
      else
        emit(t, t.key_lo, t.key_hi + 1, t.tile_begin, -1);
      continue;
    }
    if (t.key_lo > t.key_hi) {  // nothing visible (only with a key-range option)
      emit(t, 0, 0, 0, -1);
      continue;
    }
    chunks.clear();
    // base chunks: the requested equal split in the request's key coordinates
    // (tile-aligned), else the whole visible range
    auto add = [&](int64_t a, int64_t e) {   // sub-split [a, e) at tile-aligned steps
      if (a >= e) return;
      if (chunk_tiles <= 0) {
        chunks.emplace_back((int32_t)a, (int32_t)e);
        return;
      }
      const int64_t step = chunk_tiles * NK;
      int64_t c = a;
      while (c < e) {
        const int64_t nxt = std::min<int64_t>(((c >> nk_sh) << nk_sh) + step, e);
        chunks.emplace_back((int32_t)c, (int32_t)nxt);
        c = nxt;
      }
    };
    if (o.num_kv_chunks > 0) {
      const int64_t L = S->reqs[t.b].kv_len;
      int64_t clen = (L + o.num_kv_chunks - 1) / o.num_kv_chunks;
      clen = std::max<int64_t>(NK, ((clen + NK - 1) >> nk_sh) << nk_sh);
      for (int64_t c0 = 0; c0 < L; c0 += clen)
        add(std::max<int64_t>(c0, t.key_lo), std::min<int64_t>(c0 + clen, (int64_t)t.key_hi + 1));
    } else {
      add(t.key_lo, (int64_t)t.key_hi + 1);
    }
    if (chunks.size() == 1) {
      emit(t, chunks[0].first, chunks[0].second, t.tile_begin, -1);
      continue;
    }
    MergeItem m;
    m.b = t.b;
    m.kvh = t.kvh;
    m.row0 = t.row0;
    m.nrows = t.nrows;
    m.slot0 = slots;
    m.nslots = (int32_t)chunks.size();
    m.pad0 = m.pad1 = 0;
    S->merges.push_back(m);
    for (const auto& c : chunks) {
      const int32_t tb = std::max(t.tile_begin, (c.first >> nk_sh) << nk_sh);
      emit(t, c.first, c.second, tb, slots++);
    }
  }
  S->num_slots = slots;
  if (items.size() > (size_t)INT32_MAX / 2)
    return fail(PKV_EINVAL, "batch too large: %zu tasks", items.size());
  const bool grouped = order_for_xcds(items, costs, batch, hkv, &S->work);
  // short tiles (one work group per CU): when the list is plain longest-first
  // and longer than one work group per CU, the tasks beyond the first round
  // are taken in the order their work groups start
  S->dyn_base = (kind != TILE_PREFILL && !grouped && (int64_t)S->work.size() > kNumCUs)
                    ? kNumCUs : 0;

  // ---- workspace layouts
  size_t off = 0;
  S->off_reqs = off;
  off = align_up(off + S->reqs.size() * sizeof(ReqInfo), 256);
  S->off_work = off;
  off = align_up(off + S->work.size() * sizeof(WorkItem), 256);
  S->off_merge = off;
  off = align_up(off + S->merges.size() * sizeof(MergeItem), 256);
  S->off_dyn = off;   // the start-order task counter, uploaded as zero
  off = align_up(off + sizeof(int32_t), 256);
  S->off_pages = off;
  off = align_up(off + (size_t)S->num_indices * sizeof(int32_t), 256);
  S->off_mask = off;
  off = align_up(off + S->mask_bytes, 256);
  S->int_bytes = std::max<size_t>(off, 256);
  const size_t part_o = (size_t)slots * MR * head_dim * sizeof(float);
  S->off_part_lse = align_up(part_o, 256);
  S->float_bytes = slots > 0 ? align_up(S->off_part_lse + (size_t)slots * MR * sizeof(float), 256) : 0;
  return PKV_OK;
}

// ---- pinned staging buffers for the one host-to-device copy per plan --------
struct Staging {
  void* host = nullptr;
  void* dev_view = nullptr;   // the same pinned memory as the device addresses it
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  int device = -1;
  bool in_flight = false;
};
std::mutex g_staging_mu;
std::vector<Staging*> g_staging;

// Upload `bytes` (a multiple of 256) to dst on `stream`: `fill` writes them
// straight into a free pinned staging buffer, which a copy kernel then reads.
// Buffers and their events belong to the GPU that runs `stream` (the current
// device for the null stream), which need not be the current device.
template <typename Fill>
pkv_status copy_to_device(void* dst, size_t bytes, const Fill& fill, hipStream_t stream) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(PKV_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return fail(PKV_EHIP, "hipStreamGetDevice: %s", hipGetErrorString(e));
    dev = (int)d;
  }
  std::lock_guard<std::mutex> lock(g_staging_mu);
  Staging* s = nullptr;
  for (Staging* c : g_staging) {
    if (c->device != dev || c->cap < bytes) continue;
    if (c->in_flight && hipEventQuery(c->ev) != hipSuccess) continue;
    s = c;
    break;
  }
  if (!s) {
    s = new Staging();
    s->device = dev;
    s->cap = std::max<size_t>(bytes, 1 << 16);
    e = hipHostMalloc(&s->host, s->cap, hipHostMallocDefault);
    if (e != hipSuccess) {
      delete s;
      return fail(PKV_EHIP, "hipHostMalloc(%zu): %s", bytes, hipGetErrorString(e));
    }
    e = hipHostGetDevicePointer(&s->dev_view, s->host, 0);
    if (e != hipSuccess) {
      (void)hipHostFree(s->host);
      delete s;
      return fail(PKV_EHIP, "hipHostGetDevicePointer: %s", hipGetErrorString(e));
    }
    // the event is recorded on `stream`: create it on that stream's device
    if (dev != cur && (e = hipSetDevice(dev)) == hipSuccess) {
      e = hipEventCreateWithFlags(&s->ev, hipEventDisableTiming);
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    } else if (dev == cur) {
      e = hipEventCreateWithFlags(&s->ev, hipEventDisableTiming);
    }
    if (e != hipSuccess) {
      (void)hipHostFree(s->host);
      delete s;
      return fail(PKV_EHIP, "hipEventCreate: %s", hipGetErrorString(e));
    }
    g_staging.push_back(s);
  }
  fill(static_cast<uint8_t*>(s->host));
  e = launch_upload(dst, s->dev_view, bytes, stream);
  if (e != hipSuccess) return fail(PKV_EHIP, "plan upload launch: %s", hipGetErrorString(e));
  e = hipEventRecord(s->ev, stream);
  if (e != hipSuccess) return fail(PKV_EHIP, "hipEventRecord: %s", hipGetErrorString(e));
  s->in_flight = true;
  return PKV_OK;
}

// The schedule pkv_workspace_size computed, kept for the pkv_plan call that
// normally follows it with the same arguments (callers size the workspaces,
// then plan): that call takes it instead of scheduling again.  It is handed
// over once and dropped by the next call of either function, so nothing is
// reused across plans.
struct PendingSchedule {
  std::vector<uint8_t> key;   // every input the scheduler reads, serialized
  Schedule S;
  bool valid = false;
};
thread_local PendingSchedule g_pending;

template <typename X>
void put(std::vector<uint8_t>& k, const X* p, size_t n) {
  const uint8_t* b = reinterpret_cast<const uint8_t*>(p);
  if (n) k.insert(k.end(), b, b + n * sizeof(X));
}

// Serialized scheduler inputs; empty when the arrays cannot be read (the
// scheduler reports those errors itself).
std::vector<uint8_t> schedule_key(const int32_t* qo, const int32_t* kv, const int32_t* idx,
                                  int64_t num_indices, const int32_t* last, int32_t batch,
                                  int32_t hq, int32_t hkv, int32_t head_dim, int32_t page_size,
                                  int32_t causal, int32_t window_left,
                                  const pkv_plan_options* opts) {
  std::vector<uint8_t> k;
  if (batch < 0 || (batch > 0 && (!qo || !kv || !last))) return k;
  if (num_indices < 0 || (num_indices > 0 && !idx)) return k;
  const int32_t sc[8] = {batch, hq, hkv, head_dim, page_size, causal, window_left, 0};
  put(k, sc, 8);
  put(k, &num_indices, 1);
  if (batch > 0) {
    put(k, qo, (size_t)batch + 1);
    put(k, kv, (size_t)batch + 1);
    put(k, last, (size_t)batch);
  }
  put(k, idx, (size_t)num_indices);
  if (opts) {
    pkv_plan_options o = *opts;
    o.custom_mask = nullptr;
    o.mask_indptr = nullptr;
    put(k, &o, 1);
    if (opts->custom_mask && opts->mask_indptr && batch > 0) {
      put(k, opts->mask_indptr, (size_t)batch + 1);
      const int64_t bytes = opts->mask_indptr[batch];
      if (bytes < 0) return {};
      put(k, opts->custom_mask, (size_t)bytes);
    }
  }
  return k;
}

}  // namespace

struct pkv_plan_s {
  Schedule S;
  pkv_dtype dtype;
  float sm_scale;
  float soft_cap = 0.f;
  bool kv_fp8 = false;
  float k_scale = 1.f, v_scale = 1.f;
  uint32_t page_magic = 1, page_shift = 0;
  uint8_t* int_ws = nullptr;
  float* float_ws = nullptr;
  bool has_device_copy = false;
};

extern "C" {

const char* pkv_last_error(void) { return g_err.c_str(); }

const char* pkv_version(void) { return "pkv 0.1 (gfx950)"; }

pkv_status pkv_workspace_size(const int32_t* qo_indptr, const int32_t* kv_indptr,
                              const int32_t* kv_page_indices, int64_t num_indices,
                              const int32_t* kv_last_page_len, int32_t batch_size,
                              int32_t num_qo_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t page_size, int32_t causal, int32_t window_left,
                              const pkv_plan_options* opts, size_t* int_ws_bytes,
                              size_t* float_ws_bytes) {
  g_err.clear();
  g_pending.valid = false;
  Schedule S;
  pkv_status st = schedule(qo_indptr, kv_indptr, kv_page_indices, num_indices, kv_last_page_len,
                           batch_size, num_qo_heads, num_kv_heads, head_dim, page_size, causal,
                           window_left, opts, &S);
  if (st != PKV_OK) return st;
  if (int_ws_bytes) *int_ws_bytes = S.int_bytes;
  if (float_ws_bytes) *float_ws_bytes = S.float_bytes;
  g_pending.key = schedule_key(qo_indptr, kv_indptr, kv_page_indices, num_indices,
                               kv_last_page_len, batch_size, num_qo_heads, num_kv_heads, head_dim,
                               page_size, causal, window_left, opts);
  if (!g_pending.key.empty()) {
    g_pending.S = std::move(S);
    g_pending.valid = true;
  }
  return PKV_OK;
}

pkv_status pkv_plan(const int32_t* qo_indptr, const int32_t* kv_indptr,
                    const int32_t* kv_page_indices, int64_t num_indices,
                    const int32_t* kv_last_page_len, int32_t batch_size, int32_t num_qo_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t page_size, int32_t causal,
                    int32_t window_left, float sm_scale, pkv_dtype dtype, void* int_ws,
                    size_t int_ws_bytes, void* float_ws, size_t float_ws_bytes, void* stream,
                    const pkv_plan_options* opts, pkv_plan_t* out_plan) {
  g_err.clear();
  if (!out_plan) return fail(PKV_EINVAL, "out_plan: expected a pointer, given NULL");
  *out_plan = nullptr;
  if (dtype != PKV_FP16 && dtype != PKV_BF16)
    return fail(PKV_EINVAL, "dtype: expected fp16 or bf16, given %s", dtype_name(dtype));
  // The kernels take each row's maximum of the raw scores before scaling and
  // give masked scores -inf before the scale: both assume sm_scale > 0.
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
    return fail(PKV_EINVAL, "sm_scale: expected a finite value > 0, given %g", (double)sm_scale);
  const bool dry = (int_ws == nullptr && int_ws_bytes == 0);
  pkv_plan_s* p = new pkv_plan_s();
  pkv_status st = PKV_OK;
  bool reused = false;
  if (g_pending.valid) {
    g_pending.valid = false;
    if (schedule_key(qo_indptr, kv_indptr, kv_page_indices, num_indices, kv_last_page_len,
                     batch_size, num_qo_heads, num_kv_heads, head_dim, page_size, causal,
                     window_left, opts) == g_pending.key) {
      p->S = std::move(g_pending.S);
      reused = true;
    }
  }
  if (!reused)
    st = schedule(qo_indptr, kv_indptr, kv_page_indices, num_indices, kv_last_page_len,
                  batch_size, num_qo_heads, num_kv_heads, head_dim, page_size, causal,
                  window_left, opts, &p->S);
  if (st != PKV_OK) {
    delete p;
    return st;
  }
  const Schedule& S = p->S;
  p->dtype = dtype;
  p->sm_scale = sm_scale;
  p->soft_cap = opts ? opts->logits_soft_cap : 0.f;
  if (opts && opts->kv_dtype == PKV_FP8_E4M3) {
    p->kv_fp8 = true;
    p->k_scale = opts->k_scale > 0.f ? opts->k_scale : 1.f;
    p->v_scale = opts->v_scale > 0.f ? opts->v_scale : 1.f;
  }
  page_divider((uint32_t)page_size, &p->page_magic, &p->page_shift);
  if (!dry) {
    // The task list is uploaded from a pinned staging buffer that is reused
    // once an event recorded after the upload has completed.  Under stream
    // capture that event is never recorded, so a captured upload could read a
    // buffer another plan has refilled: plans are built outside capture.
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    const hipError_t ce = hipStreamIsCapturing(static_cast<hipStream_t>(stream), &cs);
    if (ce != hipSuccess) {
      delete p;
      return fail(PKV_EHIP, "hipStreamIsCapturing: %s", hipGetErrorString(ce));
    }
    if (cs != hipStreamCaptureStatusNone) {
      delete p;
      return fail(PKV_EINVAL, "stream: expected a stream that is not capturing (plan runs "
                              "outside graph capture; run() may be captured), given a "
                              "capturing stream");
    }
    if (!int_ws || int_ws_bytes < S.int_bytes) {
      delete p;
      return fail(PKV_EWORKSPACE, "int_ws: expected >= %zu bytes, given %zu%s", S.int_bytes,
                  int_ws_bytes, int_ws ? "" : " (NULL)");
    }
    if (reinterpret_cast<uintptr_t>(int_ws) % 256 != 0) {
      delete p;
      return fail(PKV_ELAYOUT, "int_ws: expected 256-byte alignment");
    }
    if (S.float_bytes > 0 && (!float_ws || float_ws_bytes < S.float_bytes)) {
      delete p;
      return fail(PKV_EWORKSPACE, "float_ws: expected >= %zu bytes, given %zu%s", S.float_bytes,
                  float_ws_bytes, float_ws ? "" : " (NULL)");
    }
    if (S.float_bytes > 0 && reinterpret_cast<uintptr_t>(float_ws) % 256 != 0) {
      delete p;
      return fail(PKV_ELAYOUT, "float_ws: expected 256-byte alignment");
    }
    // the int workspace image: each region, then zeros up to the next one
    auto fill = [&](uint8_t* dst) {
      size_t at = 0;
      auto put_region = [&](size_t off, const void* src, size_t n) {
        std::memset(dst + at, 0, off - at);
        if (n) std::memcpy(dst + off, src, n);
        at = off + n;
      };
      put_region(S.off_reqs, S.reqs.data(), S.reqs.size() * sizeof(ReqInfo));
      put_region(S.off_work, S.work.data(), S.work.size() * sizeof(WorkItem));
      put_region(S.off_merge, S.merges.data(), S.merges.size() * sizeof(MergeItem));
      put_region(S.off_pages, kv_page_indices, (size_t)S.num_indices * sizeof(int32_t));
      put_region(S.off_mask, S.mask_bytes ? opts->custom_mask : nullptr, S.mask_bytes);
      std::memset(dst + at, 0, S.int_bytes - at);
    };
    st = copy_to_device(int_ws, S.int_bytes, fill, static_cast<hipStream_t>(stream));
    if (st != PKV_OK) {
      delete p;
      return st;
    }
    p->int_ws = static_cast<uint8_t*>(int_ws);
    p->float_ws = static_cast<float*>(float_ws);
    p->has_device_copy = true;
  }
  *out_plan = p;
  return PKV_OK;
}

void pkv_plan_destroy(pkv_plan_t plan) { delete plan; }

pkv_status pkv_plan_get_info(pkv_plan_t p, pkv_plan_info* info) {
  g_err.clear();
  if (!p) return fail(PKV_ENOTPLANNED, "plan: expected a plan handle, given NULL");
  if (!info) return fail(PKV_EINVAL, "info: expected a pointer, given NULL");
  const Schedule& S = p->S;
  info->total_q_rows = S.total_q;
  info->num_page_indices = S.num_indices;
  info->batch_size = S.batch;
  info->num_work_items = (int32_t)S.work.size();
  info->num_merge_items = (int32_t)S.merges.size();
  info->num_partial_slots = S.num_slots;
  info->tile_rows = S.rows;
  info->tile_keys = S.keys;
  info->max_page_index = S.max_page;
  info->has_device_copy = p->has_device_copy ? 1 : 0;
  info->int_ws_bytes = (int64_t)S.int_bytes;
  info->float_ws_bytes = (int64_t)S.float_bytes;
  info->total_kv_len = S.total_kv;
  return PKV_OK;
}

pkv_status pkv_plan_get_work(pkv_plan_t p, int32_t* out, int64_t capacity, int64_t* count) {
  g_err.clear();
  if (!p) return fail(PKV_ENOTPLANNED, "plan: expected a plan handle, given NULL");
  const auto& W = p->S.work;
  if (count) *count = (int64_t)W.size();
  if (!out) return PKV_OK;
  const int64_t n = std::min<int64_t>(capacity, (int64_t)W.size());
  for (int64_t i = 0; i < n; ++i) {
    const WorkItem& w = W[i];
    int32_t* r = out + 8 * i;
    r[0] = w.b;
    r[1] = w.kvh;
    r[2] = w.row0;
    r[3] = w.nrows;
    r[4] = w.key_lo;
    r[5] = w.kv_end;
    r[6] = w.slot;
    r[7] = w.tile_begin;
  }
  return PKV_OK;
}

}  // extern "C"

namespace {

pkv_status check_cache(const pkv_plan_s* p, const char* name, const void* ptr, int64_t pages,
                       int32_t psize, int32_t heads, int32_t dim, int64_t s_page, int64_t s_tok,
                       int64_t s_head) {
  const Schedule& S = p->S;
  if (heads != S.hkv)
    return fail(PKV_EMISMATCH, "%s num_kv_heads: planned %d, given %d", name, S.hkv, heads);
  if (dim != S.head_dim)
    return fail(PKV_EMISMATCH, "%s head_dim: planned %d, given %d", name, S.head_dim, dim);
  if (psize != S.page_size)
    return fail(PKV_EMISMATCH, "%s page_size: planned %d, given %d", name, S.page_size, psize);
  if (S.max_page >= 0 && pages <= S.max_page)
    return fail(PKV_EINVAL, "%s num_pages: page id %d is referenced, given a pool of %lld pages",
                name, S.max_page, (long long)pages);
  if (S.total_kv > 0 && !ptr) return fail(PKV_EINVAL, "%s: expected a device pointer, given NULL", name);
  if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
    return fail(PKV_ELAYOUT, "%s: expected 16-byte alignment", name);
  const int g = p->kv_fp8 ? 16 : 8;   // elements per 16 bytes
  if (s_page < 0 || s_tok < 0 || s_head < 0 || s_page % g || s_tok % g || s_head % g)
    return fail(PKV_ELAYOUT,
                "%s strides (page %lld, token %lld, head %lld): expected non-negative multiples "
                "of %d elements with a packed head_dim",
                name, (long long)s_page, (long long)s_tok, (long long)s_head, g);
  // the kernels address a key as page * s_page (64-bit) + an in-page offset (32-bit)
  const int64_t in_page = (int64_t)(psize - 1) * s_tok + (int64_t)(heads - 1) * s_head + dim;
  if (s_page >= (1ll << 31) || in_page >= (1ll << 31))
    return fail(PKV_ELAYOUT,
                "%s strides (page %lld, token %lld, head %lld): one page must span fewer than "
                "2^31 elements",
                name, (long long)s_page, (long long)s_tok, (long long)s_head);
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_run(pkv_plan_t p, const void* q, int64_t q_rows, int32_t q_heads, int32_t q_dim,
                   int64_t q_s_tok, int64_t q_s_head, const void* k, int64_t k_pages,
                   int32_t k_page_size, int32_t k_heads, int32_t k_dim, int64_t k_s_page,
                   int64_t k_s_tok, int64_t k_s_head, const void* v, int64_t v_pages,
                   int32_t v_page_size, int32_t v_heads, int32_t v_dim, int64_t v_s_page,
                   int64_t v_s_tok, int64_t v_s_head, pkv_dtype dtype, void* o, int64_t o_rows,
                   float* lse, int64_t lse_rows, void* stream) {
  g_err.clear();
  if (!p) return fail(PKV_ENOTPLANNED, "plan: run before a successful plan");
  const Schedule& S = p->S;
  if (dtype != p->dtype)
    return fail(PKV_EMISMATCH, "dtype: planned %s, given %s", dtype_name(p->dtype),
                dtype_name(dtype));
  if (q_heads != S.hq)
    return fail(PKV_EMISMATCH, "q num_qo_heads: planned %d, given %d", S.hq, q_heads);
  if (q_dim != S.head_dim)
    return fail(PKV_EMISMATCH, "q head_dim: planned %d, given %d", S.head_dim, q_dim);
  if (q_rows < S.total_q)
    return fail(PKV_EMISMATCH, "q rows: planned at least %lld, given %lld", (long long)S.total_q,
                (long long)q_rows);
  if (o_rows < S.total_q)
    return fail(PKV_EMISMATCH, "o rows: planned at least %lld, given %lld", (long long)S.total_q,
                (long long)o_rows);
  if (lse != nullptr && lse_rows < S.total_q)
    return fail(PKV_EMISMATCH, "lse rows: planned at least %lld, given %lld",
                (long long)S.total_q, (long long)lse_rows);
  pkv_status st = check_cache(p, "k", k, k_pages, k_page_size, k_heads, k_dim, k_s_page, k_s_tok,
                              k_s_head);
  if (st != PKV_OK) return st;
  st = check_cache(p, "v", v, v_pages, v_page_size, v_heads, v_dim, v_s_page, v_s_tok, v_s_head);
  if (st != PKV_OK) return st;
  if (S.total_q > 0) {
    if (!q) return fail(PKV_EINVAL, "q: expected a device pointer, given NULL");
    if (!o) return fail(PKV_EINVAL, "o: expected a device pointer, given NULL");
  }
  if (reinterpret_cast<uintptr_t>(q) % 16 != 0)
    return fail(PKV_ELAYOUT, "q: expected 16-byte alignment");
  if (q_s_tok < 0 || q_s_head < 0 || q_s_tok % 8 || q_s_head % 8)
    return fail(PKV_ELAYOUT,
                "q strides (token %lld, head %lld): expected non-negative multiples of 8 "
                "elements with a packed head_dim",
                (long long)q_s_tok, (long long)q_s_head);
  if (reinterpret_cast<uintptr_t>(o) % 16 != 0)
    return fail(PKV_ELAYOUT, "o: expected 16-byte alignment");
  if (reinterpret_cast<uintptr_t>(lse) % 4 != 0)
    return fail(PKV_ELAYOUT, "lse: expected 4-byte alignment");
  // every argument check above runs on host-only plans too (no device call)
  if (!p->has_device_copy)
    return fail(PKV_ENOTPLANNED, "plan: built without a workspace (host-only), not runnable");
  if (S.work.empty()) return PKV_OK;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  AttnArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.pages = reinterpret_cast<const int32_t*>(p->int_ws + S.off_pages);
  a.reqs = reinterpret_cast<const ReqInfo*>(p->int_ws + S.off_reqs);
  a.work = reinterpret_cast<const WorkItem*>(p->int_ws + S.off_work);
  a.mask = S.mask_bytes > 0 ? p->int_ws + S.off_mask : nullptr;
  a.part_o = p->float_ws;
  a.part_lse = p->float_ws ? reinterpret_cast<float*>(reinterpret_cast<uint8_t*>(p->float_ws) +
                                                      S.off_part_lse)
                           : nullptr;
  a.dyn_base = S.dyn_base;
  a.dyn_next = reinterpret_cast<int32_t*>(p->int_ws + S.off_dyn);
  a.q_s_tok = q_s_tok;
  a.q_s_head = q_s_head;
  a.k_s_page = (uint32_t)k_s_page;
  a.k_s_tok = (uint32_t)k_s_tok;
  a.k_s_head = (uint32_t)k_s_head;
  a.v_s_page = (uint32_t)v_s_page;
  a.v_s_tok = (uint32_t)v_s_tok;
  a.v_s_head = (uint32_t)v_s_head;
  a.num_work = (int32_t)S.work.size();
  a.group = S.group;
  a.num_qo_heads = S.hq;
  a.page_size = S.page_size;
  a.page_magic = p->page_magic;
  a.page_shift = p->page_shift;
  a.causal = S.causal;
  a.scale_log2 = p->sm_scale * 1.4426950408889634f * (p->kv_fp8 ? p->k_scale : 1.f);
  a.kv_fp8 = p->kv_fp8 ? 1 : 0;
  a.v_scale = p->v_scale;
  // the kernel's raw score is q . codes; the logit is sm_scale * k_scale times it
  a.cap_in = p->soft_cap > 0.f ? p->sm_scale * (p->kv_fp8 ? p->k_scale : 1.f) / p->soft_cap : 0.f;
  a.cap_out = p->soft_cap > 0.f ? p->soft_cap * 1.4426950408889634f : 0.f;
  a.cap_series = p->soft_cap > 1024.f ? 1 : 0;
  hipError_t e = launch_attention(S.tile_kind, (int)p->dtype, S.head_dim, a, hs);
  if (e != hipSuccess) return fail(PKV_EHIP, "attention launch: %s", hipGetErrorString(e));
  if (!S.merges.empty()) {
    SplitMergeArgs m;
    m.o = o;
    m.lse = lse;
    m.reqs = a.reqs;
    m.items = reinterpret_cast<const MergeItem*>(p->int_ws + S.off_merge);
    m.part_o = a.part_o;
    m.part_lse = a.part_lse;
    m.num_items = (int32_t)S.merges.size();
    m.group = S.group;
    m.num_qo_heads = S.hq;
    m.tile_rows = S.rows;
    e = launch_split_merge((int)p->dtype, S.head_dim, m, hs);
    if (e != hipSuccess) return fail(PKV_EHIP, "split merge launch: %s", hipGetErrorString(e));
  }
  return PKV_OK;
}

pkv_status pkv_merge_states(const void* o_a, const float* lse_a, const void* o_b,
                            const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                            int32_t heads, int32_t head_dim, pkv_dtype dtype, void* stream) {
  g_err.clear();
  if (dtype != PKV_FP16 && dtype != PKV_BF16 && dtype != PKV_FP32)
    return fail(PKV_EINVAL, "dtype: expected fp16, bf16 or fp32, given %d", (int)dtype);
  if (rows < 0 || heads < 0 || head_dim < 0)
    return fail(PKV_EINVAL, "shape [%lld, %d, %d]: expected non-negative sizes", (long long)rows,
                heads, head_dim);
  if (rows * heads > 0 && head_dim > 0 &&
      (!o_a || !o_b || !o_out || !lse_a || !lse_b || !lse_out))
    return fail(PKV_EINVAL, "merge_states: expected device pointers, given NULL");
  hipError_t e = launch_merge_states((int)dtype, o_a, lse_a, o_b, lse_b, o_out, lse_out, rows,
                                     heads, head_dim, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "merge_states launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

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
                         pkv_dtype dtype, int32_t* err_count, void* stream) {
  g_err.clear();
  if (dtype != PKV_FP16 && dtype != PKV_BF16)
    return fail(PKV_EINVAL, "dtype: expected fp16 or bf16, given %s", dtype_name(dtype));
  if (num_tokens < 0) return fail(PKV_EINVAL, "num_tokens: expected >= 0, given %lld", (long long)num_tokens);
  if (num_kv_heads <= 0) return fail(PKV_EINVAL, "num_kv_heads: expected > 0, given %d", num_kv_heads);
  if (head_dim <= 0 || head_dim % 8)
    return fail(PKV_EINVAL, "head_dim: expected a positive multiple of 8, given %d", head_dim);
  if (batch_size < 0) return fail(PKV_EINVAL, "batch_size: expected >= 0, given %d", batch_size);
  if (num_indices < 0) return fail(PKV_EINVAL, "num_indices: expected >= 0, given %lld", (long long)num_indices);
  if (k_page_size < 1) return fail(PKV_EINVAL, "page_size: expected >= 1, given %d", k_page_size);
  if (v_page_size != k_page_size)
    return fail(PKV_EMISMATCH, "v page_size: k has %d, given %d", k_page_size, v_page_size);
  if (v_pages != k_pages)
    return fail(PKV_EMISMATCH, "v num_pages: k has %lld, given %lld", (long long)k_pages, (long long)v_pages);
  if (num_tokens == 0) return PKV_OK;
  if (!append_k || !append_v || !batch_indices || !positions || !kv_indptr ||
      (num_indices > 0 && !kv_page_indices) || !k || !v)
    return fail(PKV_EINVAL, "append_kv: expected device pointers, given NULL");
  for (const void* ptr : {append_k, append_v, (const void*)k, (const void*)v})
    if (reinterpret_cast<uintptr_t>(ptr) % 16 != 0)
      return fail(PKV_ELAYOUT, "append_kv: expected 16-byte aligned k / v / append pointers");
  for (int64_t st : {ak_s_tok, ak_s_head, av_s_tok, av_s_head})
    if (st < 0 || st % 8)
      return fail(PKV_ELAYOUT, "append strides: expected non-negative multiples of 8 elements, given %lld",
                  (long long)st);
  const int64_t in_k = (int64_t)(k_page_size - 1) * k_s_tok + (int64_t)(num_kv_heads - 1) * k_s_head + head_dim;
  const int64_t in_v = (int64_t)(v_page_size - 1) * v_s_tok + (int64_t)(num_kv_heads - 1) * v_s_head + head_dim;
  for (int64_t st : {k_s_page, k_s_tok, k_s_head, v_s_page, v_s_tok, v_s_head})
    if (st < 0 || st % 8 || st >= (1ll << 31))
      return fail(PKV_ELAYOUT, "cache strides: expected non-negative multiples of 8 elements below 2^31, "
                               "given %lld", (long long)st);
  if (in_k >= (1ll << 31) || in_v >= (1ll << 31))
    return fail(PKV_ELAYOUT, "cache strides: one page must span fewer than 2^31 elements");
  AppendArgs a;
  a.ak = append_k;
  a.av = append_v;
  a.k = k;
  a.v = v;
  a.batch_indices = batch_indices;
  a.positions = positions;
  a.kv_indptr = kv_indptr;
  a.pages = kv_page_indices;
  a.err_count = err_count;
  a.num_tokens = num_tokens;
  a.num_indices = num_indices;
  a.num_pages = k_pages;
  a.ak_s_tok = ak_s_tok;
  a.ak_s_head = ak_s_head;
  a.av_s_tok = av_s_tok;
  a.av_s_head = av_s_head;
  a.k_s_page = (uint32_t)k_s_page;
  a.k_s_tok = (uint32_t)k_s_tok;
  a.k_s_head = (uint32_t)k_s_head;
  a.v_s_page = (uint32_t)v_s_page;
  a.v_s_tok = (uint32_t)v_s_tok;
  a.v_s_head = (uint32_t)v_s_head;
  a.heads = num_kv_heads;
  a.head_dim = head_dim;
  a.batch = batch_size;
  a.page_size = k_page_size;
  page_divider((uint32_t)k_page_size, &a.page_magic, &a.page_shift);
  hipError_t e = launch_append(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "append launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"

namespace {

// Arguments of both speculative-sampling entry points, checked on the host.
pkv_status sampling_args(const float* draft_probs, const int32_t* draft_token_ids,
                         const float* target_probs, const float* accept_u,
                         const float* sample_u, int32_t batch, int32_t num_speculate_tokens,
                         int32_t vocab_size, int32_t* output_token_ids, int32_t* num_accepted,
                         SampleArgs* a) {
  if (batch < 0) return fail(PKV_EINVAL, "batch_size: expected >= 0, given %d", batch);
  if (num_speculate_tokens < 0)
    return fail(PKV_EINVAL, "num_speculate_tokens: expected >= 0, given %d", num_speculate_tokens);
  if (vocab_size < 1 || vocab_size > (1 << 20))
    return fail(PKV_EINVAL, "vocab_size: expected in [1, 2^20], given %d", vocab_size);
  if (batch == 0) return PKV_OK;
  const bool need_draft = num_speculate_tokens > 0;
  if (!target_probs || !sample_u || !output_token_ids || !num_accepted ||
      (need_draft && (!draft_probs || !draft_token_ids || !accept_u)))
    return fail(PKV_EINVAL, "chain_speculative_sampling: expected device pointers, given NULL");
  for (const void* ptr : {(const void*)draft_probs, (const void*)draft_token_ids,
                          (const void*)target_probs, (const void*)accept_u,
                          (const void*)sample_u, (const void*)output_token_ids,
                          (const void*)num_accepted})
    if (reinterpret_cast<uintptr_t>(ptr) % 4 != 0)
      return fail(PKV_ELAYOUT, "chain_speculative_sampling: expected 4-byte aligned pointers");
  a->draft_probs = draft_probs;
  a->draft_ids = draft_token_ids;
  a->target_probs = target_probs;
  a->accept_u = accept_u;
  a->sample_u = sample_u;
  a->out_ids = output_token_ids;
  a->num_accepted = num_accepted;
  a->batch = batch;
  a->num_spec = num_speculate_tokens;
  a->vocab = vocab_size;
  return PKV_OK;
}

}  // namespace

extern "C" {

pkv_status pkv_chain_speculative_sampling(const float* draft_probs,
                                          const int32_t* draft_token_ids,
                                          const float* target_probs, const float* accept_u,
                                          const float* sample_u, int32_t batch,
                                          int32_t num_speculate_tokens, int32_t vocab_size,
                                          int32_t* output_token_ids, int32_t* num_accepted,
                                          void* workspace, size_t workspace_bytes,
                                          void* stream) {
  g_err.clear();
  SampleArgs a{};
  pkv_status st = sampling_args(draft_probs, draft_token_ids, target_probs, accept_u, sample_u,
                                batch, num_speculate_tokens, vocab_size, output_token_ids,
                                num_accepted, &a);
  if (st != PKV_OK || batch == 0) return st;
  const size_t need = spec_sample_workspace_bytes(batch, vocab_size);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_EWORKSPACE, "workspace: expected >= %zu bytes, given %zu%s", need,
                workspace_bytes, workspace ? "" : " (NULL)");
  if (reinterpret_cast<uintptr_t>(workspace) % 16 != 0)
    return fail(PKV_ELAYOUT, "workspace: expected 16-byte alignment");
  hipError_t e = launch_spec_sample(a, workspace, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "speculative sampling launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

pkv_status pkv_chain_speculative_sampling_no_alloc(const float* draft_probs,
                                                   const int32_t* draft_token_ids,
                                                   const float* target_probs,
                                                   const float* accept_u, const float* sample_u,
                                                   int32_t batch, int32_t num_speculate_tokens,
                                                   int32_t vocab_size, int32_t* output_token_ids,
                                                   int32_t* num_accepted, void* stream) {
  g_err.clear();
  SampleArgs a{};
  pkv_status st = sampling_args(draft_probs, draft_token_ids, target_probs, accept_u, sample_u,
                                batch, num_speculate_tokens, vocab_size, output_token_ids,
                                num_accepted, &a);
  if (st != PKV_OK || batch == 0) return st;
  const size_t need = spec_sample_workspace_bytes(batch, vocab_size);
  if (need > kSpecScratchBytes)
    return fail(PKV_EINVAL, "batch_size * ceil(vocab_size / 1024): expected <= %zu tiles of the "
                            "library's %zu-byte scratch, given %d * %d = %zu tiles",
                kSpecScratchBytes / 16, kSpecScratchBytes, batch, (vocab_size + 1023) / 1024,
                need / 16);
  void* ws = nullptr;   // the library's own per-device array: no allocation
  hipError_t e = spec_sample_scratch(static_cast<hipStream_t>(stream), &ws);
  if (e != hipSuccess) return fail(PKV_EHIP, "scratch address: %s", hipGetErrorString(e));
  e = launch_spec_sample(a, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "speculative sampling launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

size_t pkv_chain_speculative_sampling_workspace_size(int32_t batch_size, int32_t vocab_size) {
  if (batch_size <= 0 || vocab_size <= 0) return 0;
  return spec_sample_workspace_bytes(batch_size, vocab_size);
}

pkv_status pkv_debug_gather(pkv_plan_t p, const void* k, int64_t k_pages, int32_t k_page_size,
                            int32_t k_heads, int32_t k_dim, int64_t k_s_page, int64_t k_s_tok,
                            int64_t k_s_head, const void* v, int64_t v_pages,
                            int32_t v_page_size, int32_t v_heads, int32_t v_dim,
                            int64_t v_s_page, int64_t v_s_tok, int64_t v_s_head,
                            pkv_dtype dtype, void* k_out, void* v_out, int64_t out_rows,
                            void* stream) {
  g_err.clear();
  if (!p) return fail(PKV_ENOTPLANNED, "plan: debug_gather before a successful plan");
  const Schedule& S = p->S;
  if (dtype != p->dtype)
    return fail(PKV_EMISMATCH, "dtype: planned %s, given %s", dtype_name(p->dtype),
                dtype_name(dtype));
  pkv_status st = check_cache(p, "k", k, k_pages, k_page_size, k_heads, k_dim, k_s_page, k_s_tok,
                              k_s_head);
  if (st != PKV_OK) return st;
  st = check_cache(p, "v", v, v_pages, v_page_size, v_heads, v_dim, v_s_page, v_s_tok, v_s_head);
  if (st != PKV_OK) return st;
  if (out_rows < S.total_kv)
    return fail(PKV_EMISMATCH, "gather rows: planned at least %lld, given %lld",
                (long long)S.total_kv, (long long)out_rows);
  if (S.total_kv > 0 && (!k_out || !v_out))
    return fail(PKV_EINVAL, "k_out / v_out: expected device pointers, given NULL");
  if (reinterpret_cast<uintptr_t>(k_out) % 16 || reinterpret_cast<uintptr_t>(v_out) % 16)
    return fail(PKV_ELAYOUT, "k_out / v_out: expected 16-byte alignment");
  if (!p->has_device_copy)
    return fail(PKV_ENOTPLANNED, "plan: built without a workspace (host-only), not runnable");
  if (S.work.empty()) return PKV_OK;
  // The attention kernel's own task list and load path (same tile kind, page
  // addressing and schedule as pkv_run), copying each landed tile out.
  AttnArgs a{};
  a.k = k;
  a.v = v;
  a.pages = reinterpret_cast<const int32_t*>(p->int_ws + S.off_pages);
  a.reqs = reinterpret_cast<const ReqInfo*>(p->int_ws + S.off_reqs);
  a.work = reinterpret_cast<const WorkItem*>(p->int_ws + S.off_work);
  a.k_s_page = (uint32_t)k_s_page;
  a.k_s_tok = (uint32_t)k_s_tok;
  a.k_s_head = (uint32_t)k_s_head;
  a.v_s_page = (uint32_t)v_s_page;
  a.v_s_tok = (uint32_t)v_s_tok;
  a.v_s_head = (uint32_t)v_s_head;
  a.num_work = (int32_t)S.work.size();
  a.group = S.group;
  a.num_qo_heads = S.hq;
  a.page_size = S.page_size;
  a.page_magic = p->page_magic;
  a.page_shift = p->page_shift;
  a.causal = S.causal;
  a.kv_fp8 = p->kv_fp8 ? 1 : 0;
  a.gather_k = k_out;
  a.gather_v = v_out;
  hipError_t e = launch_attention_dump(S.tile_kind, (int)p->dtype, S.head_dim, a,
                                       static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(PKV_EHIP, "debug gather launch: %s", hipGetErrorString(e));
  return PKV_OK;
}

}  // extern "C"
