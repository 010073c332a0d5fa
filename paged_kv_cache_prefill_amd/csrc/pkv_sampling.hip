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
// Two kernels.  The first spreads each request's row over many work groups:
// each redoes the (cheap) accept loop, then sums its share of the row's
// 1024-entry tiles -- residual and plain weights, and the last positive
// entry of each -- into the workspace (work group 0 of a request also writes
// the accepted tokens).  The second, one 1024-thread work group per request,
// scans the tile sums in order, finds the tile holding s * total, rescans
// that tile and writes the drawn token.  HBM-bound: the bytes are the row(s)
// read once, 4 or 8 bytes per vocabulary entry.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

constexpr int kTile = 1024;           // entries per tile
constexpr int kSumThreads = 256;      // work group of the tile-sum kernel
constexpr int kSumUnroll = 8;         // tiles whose loads are in flight together
constexpr int kDrawThreads = 1024;    // work group of the draw kernel
constexpr int kSampMaxTiles = 1024;   // vocabulary up to 2^20 entries

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ int wave_max(int x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = max(x, __shfl_xor(x, o));
  return x;
}

// Accept loop of request b: the number of accepted drafts.  Eight positions
// at a time: ids first, then their probabilities, so the loads overlap.
// Reads are clamped into the arrays; an id outside the vocabulary is
// rejected.  With `write`, thread 0 stores the accepted ids.
__device__ int accept_chain(const SampleArgs& a, int b, bool write) {
  const int n = a.num_spec, V = a.vocab;
  const float* q_b = a.draft_probs + (int64_t)b * n * V;
  const float* p_b = a.target_probs + (int64_t)b * (n + 1) * V;
  int t = 0;
  for (int t0 = 0; t0 < n; t0 += 8) {
    int xs[8];
    float ps[8], qs[8], us[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) xs[i] = a.draft_ids[(int64_t)b * n + min(t0 + i, n - 1)];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ti = min(t0 + i, n - 1);
      const int xc = min(max(xs[i], 0), V - 1);
      ps[i] = p_b[(int64_t)ti * V + xc];
      qs[i] = q_b[(int64_t)ti * V + xc];
      us[i] = a.accept_u[(int64_t)b * n + ti];
      if (xs[i] < 0 || xs[i] >= V) ps[i] = 0.f;
    }
    int acc = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (acc != i || t0 + i >= n || !(us[i] * qs[i] < ps[i])) continue;
      if (write && threadIdx.x == 0) a.out_ids[(int64_t)b * (n + 1) + t0 + i] = xs[i];
      acc = i + 1;
    }
    t = t0 + acc;
    if (acc < 8) break;
  }
  return t;
}

// Tile sums: grid (chunks, batch).  ws[b][tile] = (residual sum, plain sum,
// last positive residual entry, last positive plain entry) of the row the
// draw reads; the residual fields are 0 / -1 when no draft was rejected.
__global__ __launch_bounds__(kSumThreads) void spec_tile_sums_kernel(SampleArgs a, float4* ws,
                                                                     int tiles_per_group) {
  constexpr int NW = kSumThreads / 64;
  __shared__ float part[kSumUnroll][2][NW];
  __shared__ int plast[kSumUnroll][2][NW];
  const int b = blockIdx.y, chunk = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.num_spec, V = a.vocab;
  const int t = accept_chain(a, b, chunk == 0);
  if (chunk == 0) {
    if (tid == 0) a.num_accepted[b] = t;
    for (int k = t + 1 + tid; k <= n; k += kSumThreads) a.out_ids[(int64_t)b * (n + 1) + k] = -1;
  }
  const float* prow = a.target_probs + ((int64_t)b * (n + 1) + t) * V;
  const bool resid = t < n;
  const float* qrow = resid ? a.draft_probs + ((int64_t)b * n + t) * V : nullptr;
  const int ntiles = (V + kTile - 1) / kTile;
  const int t_begin = chunk * tiles_per_group;
  const int t_end = min(ntiles, t_begin + tiles_per_group);
  for (int t0 = t_begin; t0 < t_end; t0 += kSumUnroll) {
    // all reads first (clamped into the row), then the sums
    float pv[kSumUnroll][kTile / kSumThreads], qv[kSumUnroll][kTile / kSumThreads];
    if (resid) {
#pragma unroll
      for (int u = 0; u < kSumUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kTile / kSumThreads; ++j) {
          const int k = min((t0 + u) * kTile + j * kSumThreads + tid, V - 1);
          pv[u][j] = prow[k];
          qv[u][j] = qrow[k];
        }
    } else {
#pragma unroll
      for (int u = 0; u < kSumUnroll; ++u)
#pragma unroll
        for (int j = 0; j < kTile / kSumThreads; ++j) {
          pv[u][j] = prow[min((t0 + u) * kTile + j * kSumThreads + tid, V - 1)];
          qv[u][j] = 0.f;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kSumUnroll; ++u) {
      float rs = 0.f, ps = 0.f;
      int rl = -1, pl = -1;
#pragma unroll
      for (int j = 0; j < kTile / kSumThreads; ++j) {
        const int k = (t0 + u) * kTile + j * kSumThreads + tid;
        const bool in = k < V && t0 + u < t_end;
        const float p = in ? pv[u][j] : 0.f;
        const float r = in && resid ? fmaxf(p - qv[u][j], 0.f) : 0.f;
        rs += r;
        ps += p;
        if (r > 0.f) rl = k;
        if (p > 0.f) pl = k;
      }
      rs = wave_sum(rs);
      ps = wave_sum(ps);
      rl = wave_max(rl);
      pl = wave_max(pl);
      if (lane == 0) {
        part[u][0][wave] = rs;
        part[u][1][wave] = ps;
        plast[u][0][wave] = rl;
        plast[u][1][wave] = pl;
      }
    }
    __syncthreads();
    if (tid < kSumUnroll && t0 + tid < t_end) {   // fixed order over the waves
      float rs = 0.f, ps = 0.f;
      int rl = -1, pl = -1;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        rs += part[tid][0][w];
        ps += part[tid][1][w];
        rl = max(rl, plast[tid][0][w]);
        pl = max(pl, plast[tid][1][w]);
      }
      ws[(int64_t)b * ntiles + t0 + tid] =
          make_float4(rs, ps, __int_as_float(rl), __int_as_float(pl));
    }
    __syncthreads();
  }
}

// Draw: one work group per request, after the tile sums.
__global__ __launch_bounds__(kDrawThreads) void spec_draw_kernel(SampleArgs a, const float4* ws) {
  __shared__ float tile_sum[kSampMaxTiles];
  __shared__ float wsum[kDrawThreads / 64];
  __shared__ int found, tile_last, tile_s, lastpos, use_plain;
  __shared__ float thr_s, excl_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.num_spec, V = a.vocab;
  const int t = a.num_accepted[b];
  const int ntiles = (V + kTile - 1) / kTile;
  const float4* wsb = ws + (int64_t)b * ntiles;
  // residual unless no draft was rejected or the residual is all zero
  if (wave == 0) {
    int last_r = -1;
    for (int c = lane; c < ntiles; c += 64) last_r = max(last_r, __float_as_int(wsb[c].z));
    last_r = wave_max(last_r);
    const int plain = (t >= n || last_r < 0) ? 1 : 0;
    int last = -1;
    for (int c = lane; c < ntiles; c += 64)
      last = max(last, __float_as_int(plain ? wsb[c].w : wsb[c].z));
    last = wave_max(last);
    if (lane == 0) {
      use_plain = plain;
      lastpos = last;
    }
  }
  __syncthreads();
  const bool plain = use_plain != 0;
  const float* prow = a.target_probs + ((int64_t)b * (n + 1) + t) * V;
  const float* qrow = plain ? nullptr : a.draft_probs + ((int64_t)b * n + t) * V;
  // wave 0: inclusive prefix over the tiles; the first tile past s * total
  if (wave == 0) {
    float total = 0.f;
    for (int c = 0; c < ntiles; c += 64) {
      float x = c + lane < ntiles ? (plain ? wsb[c + lane].y : wsb[c + lane].x) : 0.f;
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
  // rescan that tile: the first entry whose running sum passes s * total
  const int tile = tile_s;
  if (tile < ntiles) {
    const int k = tile * kTile + tid;
    const int kc = min(k, V - 1);
    float w = prow[kc];
    if (qrow != nullptr) w = fmaxf(w - qrow[kc], 0.f);
    if (k >= V) w = 0.f;
    float x = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    float off = excl_s;
    for (int w2 = 0; w2 < wave; ++w2) off += wsum[w2];
    if (w > 0.f) {
      atomicMax(&tile_last, k);
      if (off + x > thr_s) atomicMin(&found, k);
    }
    __syncthreads();
  }
  if (tid == 0) {
    // rounding can leave no entry of the tile past the threshold: take its
    // last positive entry; no tile at all: the row's last positive entry
    int pick = lastpos;
    if (tile < ntiles) pick = found != 0x7fffffff ? found : (tile_last >= 0 ? tile_last : lastpos);
    a.out_ids[(int64_t)b * (n + 1) + t] = pick >= 0 ? pick : V - 1;
  }
}

size_t spec_sample_workspace_bytes(int32_t batch, int32_t vocab) {
  return (size_t)batch * (size_t)((vocab + kTile - 1) / kTile) * sizeof(float4);
}

hipError_t launch_spec_sample(const SampleArgs& a, void* ws, hipStream_t s) {
  if (a.batch == 0) return hipSuccess;
  const int ntiles = (a.vocab + kTile - 1) / kTile;
  // about 1024 work groups in all, whole groups of kSumUnroll tiles each
  int groups = (1024 + a.batch - 1) / a.batch;
  int per = (ntiles + groups - 1) / groups;
  per = ((per + kSumUnroll - 1) / kSumUnroll) * kSumUnroll;
  groups = (ntiles + per - 1) / per;
  hipLaunchKernelGGL(spec_tile_sums_kernel, dim3(groups, a.batch), dim3(kSumThreads), 0, s, a,
                     static_cast<float4*>(ws), per);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(spec_draw_kernel, dim3(a.batch), dim3(kDrawThreads), 0, s, a,
                     static_cast<const float4*>(ws));
  return hipGetLastError();
}

}  // namespace pkv
