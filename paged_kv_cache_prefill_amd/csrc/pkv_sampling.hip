// Chain speculative-sampling acceptance on CDNA4 (gfx950).
//
// The step after verify (PR #362 "Support speculative-decode verify on ROCm,
// and stop auto routing short-query prefill to AITER", Summary and
// Architecture / design notes: the acceptance sampler runs over (batch_size,
// num_speculate_tokens), drafts are one chain per request).  Per request b:
// draft token x_t is accepted while u_t * q_t(x_t) < p_t(x_t); at the first
// rejection one token is drawn from the residual max(p_t - q_t, 0) (p_t
// itself if that is all zero) and the chain stops; if every draft is
// accepted a bonus token is drawn from p_n.  Draws are inverse-CDF with one
// uniform s per request: the smallest k whose running weight sum exceeds
// s * total, else the last k with a positive weight.
//
// One 1024-thread work group per request.  The accept loop reads two floats
// per position.  The selected row is read once in tiles of 1024 elements
// (lane-contiguous, so loads coalesce): each tile's weight sum goes to LDS;
// one wave then scans the tile sums, finds the tile holding the threshold,
// and the work group rescans that one tile to find the element.  HBM-bound:
// the bytes are the selected row(s), 4 or 8 bytes per vocabulary entry.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kSampThreads = 1024;
constexpr int kSampUnroll = 32;       // tiles whose loads are in flight together
constexpr int kSampMaxTiles = 1024;   // vocabulary up to 2^20 entries

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Weights of U entries k0, k0 + 1024, ... of the row: p, or the residual
// max(p - q, 0) when qrow is set; entries past the row are 0.  The reads are
// clamped into the row rather than guarded, so all of them are in flight at
// once (a guarded read would make the compiler wait for each in turn).
template <int U>
__device__ __forceinline__ void row_weights(const float* prow, const float* qrow, int k0, int V,
                                            float (&w)[U]) {
  if (qrow != nullptr) {
    float qv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kc = min(k0 + u * kSampThreads, V - 1);
      w[u] = prow[kc];
      qv[u] = qrow[kc];
    }
    // issue every read before using any (the compiler would otherwise start
    // subtracting, and waiting, after the first pair)
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = fmaxf(w[u] - qv[u], 0.f);
  } else {
#pragma unroll
    for (int u = 0; u < U; ++u) w[u] = prow[min(k0 + u * kSampThreads, V - 1)];
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int u = 0; u < U; ++u)
    if (k0 + u * kSampThreads >= V) w[u] = 0.f;
}

__global__ __launch_bounds__(kSampThreads) void spec_sample_kernel(SampleArgs a) {
  constexpr int NW = kSampThreads / 64;
  __shared__ float tile_sum[kSampMaxTiles];
  __shared__ float wsum[kSampUnroll][NW];
  __shared__ int lastpos, found, tile_last, tile_s;
  __shared__ float thr_s, excl_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.num_spec, V = a.vocab;
  const float* q_b = a.draft_probs + (int64_t)b * n * V;
  const float* p_b = a.target_probs + (int64_t)b * (n + 1) * V;
  int* out = a.out_ids + (int64_t)b * (n + 1);

  // ---- accept loop (every thread walks it; the reads are shared).  Eight
  // positions at a time: ids first, then their probabilities, so the loads
  // overlap instead of forming a chain.
  int t = 0;
  for (int t0 = 0; t0 < n; t0 += 8) {
    int xs[8];
    float ps[8], qs[8], us[8];
    // reads clamped into the arrays (see row_weights); invalid ones are masked after
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[i] = a.draft_ids[(int64_t)b * n + min(t0 + i, n - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ti = min(t0 + i, n - 1);
      const int xc = min(max(xs[i], 0), V - 1);
      ps[i] = p_b[(int64_t)ti * V + xc];
      qs[i] = q_b[(int64_t)ti * V + xc];
      us[i] = a.accept_u[(int64_t)b * n + ti];
      if (xs[i] < 0 || xs[i] >= V) ps[i] = 0.f;   // an id outside the vocabulary is rejected
    }
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (acc != i || t0 + i >= n || !(us[i] * qs[i] < ps[i])) continue;
      if (tid == 0) out[t0 + i] = xs[i];
      acc = i + 1;
    }
    t = t0 + acc;
    if (acc < 8) break;
  }
  if (tid == 0) a.num_accepted[b] = t;
  for (int k = t + 1 + tid; k <= n; k += kSampThreads) out[k] = -1;

  // ---- the row to draw from: the residual at the rejection (p_t itself if
  // the residual is all zero), else p_n
  const float* prow = p_b + (int64_t)t * V;
  const float* qrow = t < n ? q_b + (int64_t)t * V : nullptr;
  const int ntiles = (V + kSampThreads - 1) / kSampThreads;
  for (int pass = 0; pass < 2; ++pass) {
    if (pass == 1) qrow = nullptr;
    if (tid == 0) lastpos = -1;
    __syncthreads();
    int mylast = -1;
    for (int t0 = 0; t0 < ntiles; t0 += kSampUnroll) {
      float w[kSampUnroll];
      row_weights<kSampUnroll>(prow, qrow, t0 * kSampThreads + tid, V, w);
#pragma unroll
      for (int u = 0; u < kSampUnroll; ++u) {
        if (w[u] > 0.f) mylast = (t0 + u) * kSampThreads + tid;
        const float sw = wave_sum(w[u]);
        if (lane == 0) wsum[u][wave] = sw;
      }
      __syncthreads();
      if (tid < kSampUnroll && t0 + tid < ntiles) {   // fixed order over the waves
        float x = 0.f;
#pragma unroll
        for (int w2 = 0; w2 < NW; ++w2) x += wsum[tid][w2];
        tile_sum[t0 + tid] = x;
      }
      __syncthreads();
    }
    atomicMax(&lastpos, mylast);
    __syncthreads();
    if (lastpos < 0 && qrow != nullptr) continue;   // all-zero residual: draw from p_t
    break;
  }

  // ---- wave 0: inclusive prefix over the tiles; the first tile past s * total
  if (wave == 0) {
    float total = 0.f;
    for (int c = 0; c < ntiles; c += 64) {
      float x = c + lane < ntiles ? tile_sum[c + lane] : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (lane >= o) x += y;
      }
      if (c + lane < ntiles) tile_sum[c + lane] = total + x;
      total += __shfl(x, 63);
    }
    const float thr = a.sample_u[b] * total;
    int first = ntiles;
    for (int c = 0; c < ntiles; c += 64) {
      const uint64_t m = __ballot(c + lane < ntiles && tile_sum[c + lane] > thr);
      if (m) {
        first = c + __builtin_ctzll(m);
        break;
      }
    }
    if (lane == 0) {
      thr_s = thr;
      tile_s = first;
      excl_s = (first > 0 && first < ntiles) ? tile_sum[first - 1] : 0.f;
      found = 0x7fffffff;
      tile_last = -1;
    }
  }
  __syncthreads();
  // ---- rescan that tile: the first element whose running sum passes s * total
  const int tile = tile_s;
  if (tile < ntiles) {
    const int k = tile * kSampThreads + tid;
    float w1[1];
    row_weights<1>(prow, qrow, k, V, w1);
    const float w = w1[0];
    float x = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[0][wave] = x;
    __syncthreads();
    float off = excl_s;
    for (int w2 = 0; w2 < wave; ++w2) off += wsum[0][w2];
    if (w > 0.f) {
      atomicMax(&tile_last, k);
      if (off + x > thr_s) atomicMin(&found, k);
    }
    __syncthreads();
  }
  if (tid == 0) {
    // rounding can leave no element of the tile past the threshold: take its
    // last positive entry; no tile at all: the row's last positive entry
    int pick = lastpos;
    if (tile < ntiles) pick = found != 0x7fffffff ? found : (tile_last >= 0 ? tile_last : lastpos);
    out[t] = pick >= 0 ? pick : V - 1;
  }
}

hipError_t launch_spec_sample(const SampleArgs& a, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  hipLaunchKernelGGL(spec_sample_kernel, dim3(a.batch), dim3(kSampThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
