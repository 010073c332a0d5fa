// HIP kernels for paged-KV attention prefill on CDNA4 (gfx950).
//
// What is computed (web pages of the AMD-Ecosystem FlashInfer fork):
//   - PR #339 "Route non-causal windowed prefill to AITER's masked kernel",
//     section "Why window_size_right stays -1": key j is kept for query row i
//     when j + qo_len + window_left >= kv_len + i (left-only band, bottom-right
//     anchored, independent of causal; -1 = no window).
//   - PR #362 "Support speculative-decode verify on ROCm, ...", Summary: the
//     causal mask is bottom-right aligned, j <= i + kv_len - qo_len, which is
//     also chain speculative-verify semantics.
//   - PR #399 "Refuse attention inputs the ROCm kernels would compute
//     wrongly", What changed: q head h reads kv head h / (Hq / Hkv); o and lse
//     are written packed; partial (o, lse) states are merged.
//
// Design (ours, for CDNA4; the pages describe an FA2-derived kernel only by
// its tile rule):
//   * A work-group task is a tile of packed rows (query position x q head of
//     one GQA group, position-major) of one kv head.  Packing the group into
//     the MFMA M dimension reads each K/V row once per kv head.
//   * Keys are fetched straight through the page table: one 16-byte vector
//     load per (key, 8 head-dim elements), coalesced along head_dim, written
//     by the load itself into a double-buffered LDS tile (global->LDS direct
//     loads; FP8 caches are staged through registers and converted on the
//     way in).  Nothing is gathered into a contiguous copy.
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_{bf16,f16} with fp32
//     accumulation.  In that orientation each lane owns one query row (lane %
//     16) in every MFMA result, so the row statistics stay per lane and the P
//     fragment produced by the first MFMA is directly the B operand of the
//     second (no shuffles).  The exponentials are taken against a per-row
//     reference that moves only when a score exceeds it by more than 2^8
//     (lazy rescaling): then, and only then, the row max is reduced across
//     the 4 lane groups with two xor-shuffles; the row sum once at the end.
//   * Softmax runs in the log2 domain (scale * log2 e folded into one
//     multiply, hardware exp2); lse is converted to natural log on output.
//   * Tiles entirely inside every row's visible band skip the mask; tiles
//     outside the band are never visited (the scheduler clips key ranges).
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "pkv_attn.h"
#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {


// ---------------------------------------------------------------------------
// merge of split-KV partial states (N-way), work groups of rows of one split tile
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void split_merge_kernel(SplitMergeArgs a) {
  // TPR threads own one row (4 head-dim elements each); a work group covers
  // RPW rows of one split query tile.  Every thread sweeps the slots for its
  // 4 elements, U slots per step with all their loads (partial o and lse)
  // issued together (an index past the last slot re-reads the last one with
  // weight 0), keeping a running maximum of the slot lse values and
  // rescaling its sums when a step raises it; at most U slots take one
  // round trip to memory.
  constexpr int TPR = D / 4;
  constexpr int RPW = 256 / TPR;
  constexpr int U = 16;
  const MergeItem it = a.items[blockIdx.x];
  const int rl = blockIdx.y * RPW + (int)threadIdx.x / TPR;
  const int d4 = (int)threadIdx.x % TPR;
  if (rl >= it.nrows) return;
  const ReqInfo rq = a.reqs[it.b];
  const int G = a.group;
  const int64_t tr = a.tile_rows;
  const float* lse = a.part_lse + (int64_t)it.slot0 * tr + rl;   // slot c at lse[c * tr]
  const float* po = a.part_o + ((int64_t)it.slot0 * tr + rl) * D + d4 * 4;
  float mt = kNegInf, wt = 0.f;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int c0 = 0; c0 < it.nslots; c0 += U) {
    f32x4 v[U];
    float l[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int64_t c = min(c0 + j, it.nslots - 1);
      l[j] = lse[c * tr];
      v[j] = *reinterpret_cast<const f32x4*>(po + c * tr * D);
    }
    float mn = mt;
#pragma unroll
    for (int j = 0; j < U; ++j) mn = fmaxf(mn, l[j]);   // the re-read last slot changes nothing
    const float mu = (mn == kNegInf) ? 0.f : mn;
    const float sc = (mt == kNegInf) ? 0.f : fast_exp2(mt - mu);
    wt *= sc;
    acc *= sc;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const float w = c0 + j < it.nslots ? fast_exp2(l[j] - mu) : 0.f;
      wt += w;
      acc += w * v[j];
    }
    mt = mn;
  }
  const float inv = wt > 0.f ? 1.f / wt : 0.f;
  const int r = it.row0 + rl;
  const int pos = r / G;
  const int h = it.kvh * G + (r - pos * G);
  const int64_t orow = (int64_t)(rq.qo_start + pos) * a.num_qo_heads + h;
  T o4[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o4[i] = from_f32<T>(acc[i] * inv);
  T* __restrict__ op = static_cast<T*>(a.o);
  *reinterpret_cast<uint2*>(op + orow * D + d4 * 4) = *reinterpret_cast<uint2*>(o4);
  if (d4 == 0 && a.lse != nullptr)
    a.lse[orow] = (mt == kNegInf) ? kNegInf : (mt + fast_log2(wt)) * kLn2;
}

// ---------------------------------------------------------------------------
// merge_states: two partial states, natural-log lse
// ---------------------------------------------------------------------------
// In-place merges must not let one thread overwrite lse while another thread of
// the same row still needs the old value: split the lse update into its own pass.
__global__ __launch_bounds__(256) void merge_lse_kernel(const float* lse_a, const float* lse_b,
                                                        float* lse_out, int64_t rowheads) {
  constexpr float kLog2e = 1.44269504088896340736f;
  for (int64_t rh = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; rh < rowheads;
       rh += (int64_t)gridDim.x * blockDim.x) {
    const float la = lse_a[rh], lb = lse_b[rh];
    const float mt = fmaxf(la, lb);
    if (mt == kNegInf) {
      lse_out[rh] = kNegInf;
    } else {
      const float wt = fast_exp2((la - mt) * kLog2e) + fast_exp2((lb - mt) * kLog2e);
      lse_out[rh] = mt + fast_log2(wt) * kLn2;
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void merge_o_kernel(const T* o_a, const float* lse_a,
                                                      const T* o_b, const float* lse_b,
                                                      T* o_out, int64_t rowheads,
                                                      int32_t head_dim) {
  constexpr float kLog2e = 1.44269504088896340736f;
  const int64_t n = rowheads * head_dim;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t rh = idx / head_dim;
    const float la = lse_a[rh], lb = lse_b[rh];
    const float mt = fmaxf(la, lb);
    float out = 0.f;
    if (mt != kNegInf) {
      const float wa = fast_exp2((la - mt) * kLog2e);
      const float wb = fast_exp2((lb - mt) * kLog2e);
      // a side with no key carries weight 0 and must not poison the sum
      const float ta = wa > 0.f ? wa * to_f32(o_a[idx]) : 0.f;
      const float tb = wb > 0.f ? wb * to_f32(o_b[idx]) : 0.f;
      out = (ta + tb) / (wa + wb);
    }
    o_out[idx] = from_f32<T>(out);
  }
}

// ---------------------------------------------------------------------------
// plan upload: the task list from pinned host memory into the int workspace
// ---------------------------------------------------------------------------
// A kernel on the caller's stream rather than a DMA-engine copy: the next
// attention launch then follows it on the same queue with no cross-engine
// synchronisation.  16 bytes per thread; the host pads to a multiple of 16.
__global__ __launch_bounds__(256) void upload_kernel(uint4* __restrict__ dst,
                                                     const uint4* __restrict__ src, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

// ---------------------------------------------------------------------------
// append: new K/V rows into their pages
// ---------------------------------------------------------------------------
// One thread per (token, head, 16-byte chunk); every index is range-checked
// before it is used, so a bad token is counted and skipped.
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  const int chunks = a.head_dim / 8;
  const int64_t per_tok = (int64_t)a.heads * chunks;
  const int64_t total = a.num_tokens * per_tok;
  const char* ak = static_cast<const char*>(a.ak);
  const char* av = static_cast<const char*>(a.av);
  char* kp = static_cast<char*>(a.k);
  char* vp = static_cast<char*>(a.v);
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
       idx += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = idx / per_tok;
    const int rem = (int)(idx - t * per_tok);
    const int h = rem / chunks;
    const int c = rem - h * chunks;
    const int32_t b = a.batch_indices[t];
    const int32_t pos = a.positions[t];
    bool ok = b >= 0 && b < a.batch && pos >= 0;
    uint32_t page = 0, slot = 0;
    if (ok) {
      const int32_t first = a.kv_indptr[b];
      const int32_t n = a.kv_indptr[b + 1] - first;
      const uint32_t pidx = (uint32_t)(((uint64_t)(uint32_t)pos * a.page_magic) >> a.page_shift);
      ok = first >= 0 && (int64_t)pidx < (int64_t)n && (int64_t)first + pidx < a.num_indices;
      if (ok) {
        const int32_t pg = a.pages[first + pidx];
        ok = pg >= 0 && pg < a.num_pages;
        page = (uint32_t)pg;
        slot = (uint32_t)pos - pidx * (uint32_t)a.page_size;
      }
    }
    if (!ok) {
      if (h == 0 && c == 0 && a.err_count != nullptr) atomicAdd(a.err_count, 1);
      continue;
    }
    const KeyLoc loc{page, slot};
    const uint64_t ko = key_offset(loc, a.k_s_page, a.k_s_tok, (uint32_t)h * a.k_s_head + c * 8);
    const uint64_t vo = key_offset(loc, a.v_s_page, a.v_s_tok, (uint32_t)h * a.v_s_head + c * 8);
    const int64_t ks = (t * a.ak_s_tok + (int64_t)h * a.ak_s_head + c * 8) * 2;
    const int64_t vs = (t * a.av_s_tok + (int64_t)h * a.av_s_head + c * 8) * 2;
    *reinterpret_cast<uint4*>(kp + ko * 2) = *reinterpret_cast<const uint4*>(ak + ks);
    *reinterpret_cast<uint4*>(vp + vo * 2) = *reinterpret_cast<const uint4*>(av + vs);
  }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
hipError_t launch_attention(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                            hipStream_t s) {
  // the custom-mask and soft-cap variants live in their own files (compiled
  // in parallel); the plain kernel is instantiated here
  const bool mask = a.mask != nullptr, cap = a.cap_out != 0.f;
  if (a.kv_fp8) {
    if (mask && cap) return launch_attention_fp8_mask_cap(tile_kind, dtype, head_dim, a, s);
    if (mask) return launch_attention_fp8_mask(tile_kind, dtype, head_dim, a, s);
    if (cap) return launch_attention_fp8_cap(tile_kind, dtype, head_dim, a, s);
    return launch_attention_fp8(tile_kind, dtype, head_dim, a, s);
  }
  if (mask && cap) return launch_attention_mask_cap(tile_kind, dtype, head_dim, a, s);
  if (mask) return launch_attention_mask(tile_kind, dtype, head_dim, a, s);
  if (cap) return launch_attention_cap(tile_kind, dtype, head_dim, a, s);
  return launch_attention_var<0>(tile_kind, dtype, head_dim, a, s);
}

hipError_t launch_split_merge(int dtype, int head_dim, const SplitMergeArgs& a, hipStream_t s) {
  if (a.num_items == 0) return hipSuccess;
  const int rpw = 256 / (head_dim / 4);   // rows per work group
  dim3 grid(a.num_items, (a.tile_rows + rpw - 1) / rpw);
  if (dtype == 1 && head_dim == 128)
    hipLaunchKernelGGL((split_merge_kernel<__bf16, 128>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && head_dim == 64)
    hipLaunchKernelGGL((split_merge_kernel<__bf16, 64>), grid, dim3(256), 0, s, a);
  else if (dtype == 0 && head_dim == 128)
    hipLaunchKernelGGL((split_merge_kernel<_Float16, 128>), grid, dim3(256), 0, s, a);
  else if (dtype == 0 && head_dim == 64)
    hipLaunchKernelGGL((split_merge_kernel<_Float16, 64>), grid, dim3(256), 0, s, a);
  else if (dtype == 1 && head_dim == 256)
    hipLaunchKernelGGL((split_merge_kernel<__bf16, 256>), grid, dim3(256), 0, s, a);
  else if (dtype == 0 && head_dim == 256)
    hipLaunchKernelGGL((split_merge_kernel<_Float16, 256>), grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_merge_t(const void* o_a, const float* lse_a, const void* o_b,
                                 const float* lse_b, void* o_out, float* lse_out, int64_t rh,
                                 int32_t d, hipStream_t s) {
  const int64_t n = rh * d;
  const int64_t blocks_o = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
  const int64_t blocks_l = (rh + 255) / 256 < 65536 ? (rh + 255) / 256 : 65536;
  // o first (it reads the old lse), then lse: in-place merges stay correct.
  hipLaunchKernelGGL((merge_o_kernel<T>), dim3((unsigned)blocks_o), dim3(256), 0, s,
                     static_cast<const T*>(o_a), lse_a, static_cast<const T*>(o_b), lse_b,
                     static_cast<T*>(o_out), rh, d);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(merge_lse_kernel, dim3((unsigned)blocks_l), dim3(256), 0, s, lse_a, lse_b,
                     lse_out, rh);
  return hipGetLastError();
}

hipError_t launch_merge_states(int dtype, const void* o_a, const float* lse_a, const void* o_b,
                               const float* lse_b, void* o_out, float* lse_out, int64_t rows,
                               int32_t heads, int32_t head_dim, hipStream_t s) {
  const int64_t rh = rows * heads;
  if (rh == 0 || head_dim == 0) return hipSuccess;
  if (dtype == 1)
    return launch_merge_t<__bf16>(o_a, lse_a, o_b, lse_b, o_out, lse_out, rh, head_dim, s);
  if (dtype == 0)
    return launch_merge_t<_Float16>(o_a, lse_a, o_b, lse_b, o_out, lse_out, rh, head_dim, s);
  if (dtype == 2)
    return launch_merge_t<float>(o_a, lse_a, o_b, lse_b, o_out, lse_out, rh, head_dim, s);
  return hipErrorInvalidValue;
}

hipError_t launch_upload(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 == 0) return hipSuccess;
  const int64_t blocks = (n16 + 255) / 256 < 1024 ? (n16 + 255) / 256 : 1024;
  hipLaunchKernelGGL(upload_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                     static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16);
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, hipStream_t s) {
  const int64_t units = a.num_tokens * a.heads * (a.head_dim / 8);
  if (units == 0) return hipSuccess;
  const int64_t blocks = (units + 255) / 256 < 8192 ? (units + 255) / 256 : 8192;
  hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
