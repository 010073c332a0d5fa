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

#include <mutex>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

// Tile-sum storage of the allocation-free entry point: each GPU the library
// runs on holds one copy of this array until the process ends, shared by
// every such call on that GPU (calls that overlap on one GPU race).  Host
// code never names it directly: its device address comes from
// hipGetSymbolAddress, per device (spec_sample_scratch below).
static __device__ __align__(256) uint8_t scratch[pkv::kSpecScratchBytes];

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
  // Entry j of tile u for this thread: 4 consecutive entries per thread and
  // one 16-byte load per row when rows are 16-byte aligned (vocab a multiple
  // of 4), else entries j * kSumThreads + tid with 4-byte loads.
  constexpr int E = kTile / kSumThreads;   // entries per thread per tile
  static_assert(E == 4, "16-byte loads");
  const bool vec = (V & 3) == 0;
  auto entry = [&](int tile, int j) { return tile * kTile + (vec ? E * tid + j : j * kSumThreads + tid); };
  for (int t0 = t_begin; t0 < t_end; t0 += kSumUnroll) {
    // all reads first (clamped into the row), then the sums
    float pv[kSumUnroll][E], qv[kSumUnroll][E];
    if (vec) {
#pragma unroll
      for (int u = 0; u < kSumUnroll; ++u) {
        const int k4 = min((t0 + u) * kTile + E * tid, V - E);
        const float4 p4 = *reinterpret_cast<const float4*>(prow + k4);
        const float4 q4 = resid ? *reinterpret_cast<const float4*>(qrow + k4)
                                : make_float4(0.f, 0.f, 0.f, 0.f);
        pv[u][0] = p4.x; pv[u][1] = p4.y; pv[u][2] = p4.z; pv[u][3] = p4.w;
        qv[u][0] = q4.x; qv[u][1] = q4.y; qv[u][2] = q4.z; qv[u][3] = q4.w;
      }
    } else if (resid) {
#pragma unroll
      for (int u = 0; u < kSumUnroll; ++u)
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const int k = min(entry(t0 + u, j), V - 1);
          pv[u][j] = prow[k];
          qv[u][j] = qrow[k];
        }
    } else {
#pragma unroll
      for (int u = 0; u < kSumUnroll; ++u)
#pragma unroll
        for (int j = 0; j < E; ++j) {
          pv[u][j] = prow[min(entry(t0 + u, j), V - 1)];
          qv[u][j] = 0.f;
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < kSumUnroll; ++u) {
      float rs = 0.f, ps = 0.f;
      int rl = -1, pl = -1;
#pragma unroll
      for (int j = 0; j < E; ++j) {
        const int k = entry(t0 + u, j);
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

// Draw: one work group per request, after the tile sums.  Thread c holds
// tile c's sums (one load per thread, issued with the accepted count), so the
// choice of row, the prefix over the tiles and the tile to rescan need no
// further memory round trip; the rescan of that tile is the second.
__global__ __launch_bounds__(kDrawThreads) void spec_draw_kernel(SampleArgs a, const float4* ws) {
  constexpr int NWV = kDrawThreads / 64;
  static_assert(kSampMaxTiles <= kDrawThreads, "one tile per thread");
  __shared__ float wsum[NWV];
  __shared__ int wmax_r[NWV], wmax_p[NWV];
  __shared__ int found, tile_last, first_s;
  __shared__ float excl_s;
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = a.num_spec, V = a.vocab;
  const int ntiles = (V + kTile - 1) / kTile;
  const int t = a.num_accepted[b];
  float4 e = make_float4(0.f, 0.f, __int_as_float(-1), __int_as_float(-1));
  if (tid < ntiles) e = ws[(int64_t)b * ntiles + tid];
  if (tid == 0) {
    found = 0x7fffffff;
    tile_last = -1;
    first_s = ntiles;
  }
  // last positive residual / target entry of the row
  const int lr = wave_max(__float_as_int(e.z)), lp = wave_max(__float_as_int(e.w));
  if (lane == 0) {
    wmax_r[wave] = lr;
    wmax_p[wave] = lp;
  }
  __syncthreads();
  int last_r = -1, last_p = -1;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    last_r = max(last_r, wmax_r[w]);
    last_p = max(last_p, wmax_p[w]);
  }
  // residual unless no draft was rejected or the residual is all zero
  const bool plain = t >= n || last_r < 0;
  const int lastpos = plain ? last_p : last_r;
  // inclusive prefix of the tile sums (wave scans, then the wave totals in
  // order); the first tile whose prefix passes s * total
  const float x = tid < ntiles ? (plain ? e.y : e.x) : 0.f;
  float incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float y = __shfl_up(incl, o);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  float off = 0.f, total = 0.f;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    if (w < wave) off += wsum[w];
    total += wsum[w];
  }
  incl += off;
  const float thr = a.sample_u[b] * total;
  // one LDS atomic per wave (a same-address atomic from every lane would
  // serialize over the whole work group)
  {
    const uint64_t m = __ballot(tid < ntiles && incl > thr);
    if (lane == 0 && m) atomicMin(&first_s, wave * 64 + __builtin_ctzll(m));
  }
  __syncthreads();
  const int tile = first_s;
  if (tid == tile) excl_s = incl - x;
  __syncthreads();
  const float* prow = a.target_probs + ((int64_t)b * (n + 1) + t) * V;
  const float* qrow = plain ? nullptr : a.draft_probs + ((int64_t)b * n + t) * V;
  // rescan that tile: the first entry whose running sum passes s * total
  if (tile < ntiles) {
    const int k = tile * kTile + tid;
    const int kc = min(k, V - 1);
    float w = prow[kc];
    if (qrow != nullptr) w = fmaxf(w - qrow[kc], 0.f);
    if (k >= V) w = 0.f;
    float xs = w;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const float y = __shfl_up(xs, o);
      if (lane >= o) xs += y;
    }
    __syncthreads();   // every thread has read wsum above
    if (lane == 63) wsum[wave] = xs;
    __syncthreads();
    float off2 = excl_s;
    for (int w2 = 0; w2 < wave; ++w2) off2 += wsum[w2];
    const uint64_t pos = __ballot(w > 0.f);
    const uint64_t past = __ballot(w > 0.f && off2 + xs > thr);
    if (lane == 0) {
      const int kw = tile * kTile + wave * 64;
      if (pos) atomicMax(&tile_last, kw + 63 - __builtin_clzll(pos));
      if (past) atomicMin(&found, kw + __builtin_ctzll(past));
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

// Device address of `scratch` on the GPU that runs `stream` (the current
// device for the null stream): looked up once per device, with that device
// current (the caller's current device is restored), and kept.
hipError_t spec_sample_scratch(hipStream_t stream, void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  int dev = cur;
  if (stream != nullptr) {
    hipDevice_t d = 0;
    e = hipStreamGetDevice(stream, &d);
    if (e != hipSuccess) return e;
    dev = (int)d;
  }
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
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
