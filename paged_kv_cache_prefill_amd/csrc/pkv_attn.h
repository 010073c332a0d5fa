// The attention kernel template and its launchers, shared by the HIP files
// that instantiate its variants (plain, custom mask, soft-cap, both).  What
// it computes and how is described in pkv_kernels.hip.  Internal.
#pragma once

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include "pkv_device.h"
#include "pkv_internal.h"

namespace pkv {

// WM waves split the rows, WN waves split the keys of each LDS tile;
// each wave owns QB blocks of 16 rows and NW keys of the tile.  WPE is the
// number of waves per SIMD the register budget is sized for.  PM selects the
// page addressing: 0 any page size (per-key page-table lookup), 1 power-of-
// two pages shorter than one load instruction's rows (each lane's slot is
// fixed on complete tiles), 3 power-of-two pages of at least one load
// instruction's rows: each instruction stays on one page, so its page id is
// a scalar load and its address an SGPR base plus a per-lane 32-bit offset,
// issued from assembly (dma16), which the compiler does not track; explicit
// counter waits and barriers make those loads visible (see the loops below).
// With PM 0 and 1 the last, partial tile of a task takes the general path.
// VAR bit 0 adds the custom-mask test on edge tiles, bit 1 the logits
// soft-cap, bit 2 FP8 K/V (register-staged, PM 0 or 3); each combination is
// its own instantiation so the plain kernel carries none of them.  Bit 3 is
// the gather check: the same task list, page addressing, loads, waits and
// barriers, but instead of attending, every landed K/V tile is copied out of
// LDS (un-swizzled) to a [sum kv_len, Hkv, D] array.
template <typename T, int D, int WM, int WN, int QB, int NW, int WPE, int PM, int VAR>
__global__ __launch_bounds__(64 * WM * WN, WPE) void attn_kernel(AttnArgs a) {
  constexpr bool kMask = (VAR & 1) != 0;   // custom topology mask
  constexpr bool kCap = (VAR & 2) != 0;    // logits soft-cap
  constexpr bool kFp8 = (VAR & 4) != 0;    // FP8 E4M3 K/V (converted into LDS)
  constexpr bool kDump = (VAR & 8) != 0;   // copy the landed K/V tiles out instead
  // Short tiles on the scalar-page path bring Q in through LDS with the same
  // untracked direct loads as K and V, so the first key tiles load together
  // with it (the launcher takes this path only where Q's offsets within a
  // tile fit 32 bits).
  constexpr bool kQL = WN > 1 && PM == 3 && !kFp8;
  using Tr = Traits<T>;
  using frag = typename Tr::frag;
  constexpr int NWAVE = WM * WN;
  constexpr int MW = 16 * QB;           // rows per wave
  constexpr int NWG = NW * WN;          // keys per LDS tile
  constexpr int CH = D / 8;             // 16-byte chunks per key row
  constexpr int TCH = NWG * CH;         // chunks per tile (K or V)
  constexpr int NI = TCH / (64 * NWAVE);  // direct-load instructions per wave per tile
  constexpr int RPI = 64 / CH;          // key rows filled by one wave instruction
  constexpr int DK = D / 32;            // MFMA k-steps over head_dim
  constexpr int KB = NW / 16;           // 16-key blocks per wave
  constexpr int DB = D / 16;            // 16-wide head_dim blocks of the output
  constexpr int kReadAhead = 4;         // LDS fragment reads in flight ahead of the products
  static_assert(TCH % (64 * NWAVE) == 0, "tile not divisible among waves");
  static_assert(NW % 32 == 0 && CH >= 8, "shape");

  // Two K/V buffers as four separate LDS objects: the loop below is unrolled
  // by two so every access names one fixed buffer, which lets the compiler
  // see that the direct loads into one buffer cannot alias reads of the other
  // (it then keeps those loads in flight across the tile's compute).
  __shared__ uint4 lds_k0[TCH], lds_v0[TCH], lds_k1[TCH], lds_v1[TCH];
  __shared__ uint4 lds_q[kQL ? MW * WM * (D / 8) : 1];   // Q rows of the task (kQL)

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int wm = wave % WM;
  const int wn = wave / WM;
  const int l16 = lane & 15;
  const int g = lane >> 4;

  // The first dyn_base work groups (one per concurrent slot, all started at
  // once) take their own task; later ones, which start as slots free up, take
  // the next task of the longest-first list, whichever XCD they run on, so an
  // XCD that runs slower ends up with shorter tasks.  Each later group takes
  // exactly one index, so the one that gets the last index knows every other
  // group of this launch has taken its own and can put the counter back.
  // (short tiles only: the prefill tile's launches with more tasks than slots
  // keep each (request, kv head)'s tasks on one XCD, whose L2 then serves the
  // K/V tiles they share; taking tasks in start order across XCDs instead
  // measured slower there)
  int widx = blockIdx.x;
  if (WN > 1 && a.dyn_base > 0 && widx >= a.dyn_base) {
    __shared__ int lds_task;
    if (threadIdx.x == 0) {
      const int v = atomicAdd(a.dyn_next, 1);
      if (v == a.num_work - a.dyn_base - 1) atomicExch(a.dyn_next, 0);
      lds_task = a.dyn_base + v;
    }
    __syncthreads();
    widx = __builtin_amdgcn_readfirstlane(lds_task);
  }
  const WorkItem it = a.work[widx];
  if (it.nrows == 0) return;                    // padding task (whole work group)
  const ReqInfo rq = a.reqs[it.b];
  const int G = a.group;
  const int R = rq.qo_len * G;                  // packed rows of this (request, kv head)
  const int shift_q = rq.kv_len - rq.qo_len;    // bottom-right offset L - Q
  const int win = rq.window;

  const T* __restrict__ qp = static_cast<const T*>(a.q);
  const T* __restrict__ kp = static_cast<const T*>(a.k);
  const T* __restrict__ vp = static_cast<const T*>(a.v);

  // ---- Q fragments (B operand of S^T = K Q^T) and per-row visible ranges
  frag qf[QB][DK];
  int lo[QB], hi[QB];
  int mrow[QB];   // custom mask: bit index of (row, key 0)
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = it.row0 + wm * MW + qb * 16 + l16;
    const bool valid = (r - it.row0) < it.nrows && r < R;
    mrow[qb] = rq.mask_off * 8;
    if (valid) {
      const int pos = r / G;
      mrow[qb] += pos * rq.kv_len;
      const int h = it.kvh * G + (r - pos * G);
      if constexpr (!kQL && !kDump) {
        const T* src = qp + (int64_t)(rq.qo_start + pos) * a.q_s_tok + (int64_t)h * a.q_s_head;
#pragma unroll
        for (int dk = 0; dk < DK; ++dk)
          qf[qb][dk] =
              __builtin_bit_cast(frag, *reinterpret_cast<const uint4*>(src + dk * 32 + g * 8));
      }
      int l0 = 0;
      if (win >= 0) l0 = max(0, pos + shift_q - win);
      const int h0 = a.causal ? pos + shift_q : rq.kv_len - 1;
      lo[qb] = max(l0, it.key_lo);
      hi[qb] = min(h0, it.kv_end - 1);
    } else {
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) qf[qb][dk] = __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0));
      lo[qb] = 1;
      hi[qb] = 0;
    }
  }

  // Keys every valid row of the task sees: tiles inside need no mask.
  int full_lo, full_hi;
  {
    const int rmax = min(it.row0 + it.nrows, R) - 1;
    const int pmin = it.row0 / G;
    const int pmax = rmax / G;
    full_lo = (win >= 0) ? max(0, pmax + shift_q - win) : 0;
    full_lo = max(full_lo, it.key_lo);
    full_hi = a.causal ? pmin + shift_q : rq.kv_len - 1;
    full_hi = min(full_hi, it.kv_end - 1);
    if constexpr (kMask) full_hi = min(full_hi, rq.mask_full - 1);
  }

  f32x4 oacc[DB][QB];
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = kNegInf;
    l_run[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) oacc[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int ntiles = it.kv_end > it.tile_begin ? (it.kv_end - it.tile_begin + NWG - 1) / NWG : 0;
  const int last_key = it.kv_end - 1;

  // Direct global->LDS loads: wave instruction m fills tile slots
  // [(m * NWAVE + wave) * 64, +64); lane i writes slot +i, which is key row
  // (m * NWAVE + wave) * RPI + i / CH at position i % CH, i.e. logical chunk
  // swz_k / swz_v of it.  Keys at or past kv_end read the last key instead
  // (finite data, masked to zero weight), so no read leaves the request.
  uint32_t koff[NI], voff[NI];   // element offsets of this lane's chunks within a key row
  uint32_t kin[NI], vin[NI];     // ... plus the lane's fixed slot on complete tiles (PM 1)
  int lrow[NI];
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    lrow[m] = (m * NWAVE + wave) * RPI + lane / CH;
    koff[m] = (uint32_t)swz_k<CH>(lrow[m], lane % CH) * 8 + (uint32_t)it.kvh * a.k_s_head;
    voff[m] = (uint32_t)swz_v<CH>(lrow[m], lane % CH) * 8 + (uint32_t)it.kvh * a.v_s_head;
    const uint32_t lslot = (uint32_t)lrow[m] & (uint32_t)(a.page_size - 1);
    kin[m] = lslot * a.k_s_tok + koff[m];
    vin[m] = lslot * a.v_s_tok + voff[m];
  }
  // PM 3 on complete tiles (j0 is a multiple of NWG): instruction m covers
  // tile rows r0 .. r0 + RPI - 1, r0 = (m * NWAVE + wave) * RPI, all on page
  // table entry (j0 >> shift) + (r0 >> shift) at slots (j0 & pmask) +
  // (r0 & pmask) + i.  kfull / vfull hold the lane's byte offset from that
  // page's slot j0 & pmask (which is 0 when pages are not longer than a tile).
  const uint32_t pmask = (uint32_t)a.page_size - 1;
  uint32_t kfull[NI], vfull[NI];
  int32_t pidx[NI];   // page-table entry of instruction m, relative to j0 >> shift
#pragma unroll
  for (int m = 0; m < NI; ++m) {
    const uint32_t r0 = (uint32_t)((m * NWAVE + wave) * RPI);
    const uint32_t sl = (r0 & pmask) + (uint32_t)(lane / CH);
    kfull[m] = (sl * a.k_s_tok + koff[m]) * (uint32_t)sizeof(T);
    vfull[m] = (sl * a.v_s_tok + voff[m]) * (uint32_t)sizeof(T);
    pidx[m] = (int32_t)(r0 >> a.page_shift);
  }
  // page strides in bytes: PM 3 is launched only where they fit 32 bits
  const uint32_t kpage_b = a.k_s_page * (uint32_t)sizeof(T), vpage_b = a.v_s_page * (uint32_t)sizeof(T);
  const uint32_t ktok_b = a.k_s_tok * (uint32_t)sizeof(T), vtok_b = a.v_s_tok * (uint32_t)sizeof(T);
  // page (and, on the general path, slot) of each lane row of the next tile
  uint32_t lpage[NI], lslot[NI];
  uint32_t spage[NI];       // PM 3: page of each load instruction's rows (scalar)
  const int32_t* ptab = a.pages + rq.page_off;
  const const_i32* ptab_s = (const const_i32*)ptab;   // scalar loads
  auto fetch_pages = [&](int j0) __attribute__((always_inline)) {
    if constexpr (PM == 3) {
      if (j0 + NWG <= it.kv_end) {
        const const_i32* pt = ptab_s + (j0 >> a.page_shift);
#pragma unroll
        for (int m = 0; m < NI; ++m) spage[m] = (uint32_t)pt[pidx[m]];
      } else {
#pragma unroll
        for (int m = 0; m < NI; ++m)
          spage[m] = (uint32_t)ptab_s[(uint32_t)min(j0 + (m * NWAVE + wave) * RPI, last_key) >>
                                      a.page_shift];
      }
      return;
    }
    if (PM == 1 && j0 + NWG <= it.kv_end) {
      const int32_t* pt = ptab + (j0 >> a.page_shift);
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        lpage[m] = (uint32_t)pt[lrow[m] >> a.page_shift];
        lslot[m] = (uint32_t)lrow[m] & (uint32_t)(a.page_size - 1);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const KeyLoc l = locate_key(ptab, (uint32_t)min(j0 + lrow[m], last_key), a.page_magic,
                                    a.page_shift, (uint32_t)a.page_size);
        lpage[m] = l.page;
        lslot[m] = l.slot;
      }
    }
  };
  // Direct loads of the K (is_k) or the V half of tile j0 into dst.
  auto issue_part = [&](auto is_k, int j0, uint4* dst) __attribute__((always_inline)) {
    constexpr bool IK = decltype(is_k)::value;
    const T* pool = IK ? kp : vp;
    const int full = j0 + NWG <= it.kv_end;
    if constexpr (PM == 3) {
      // one page per instruction: SGPR base + per-lane 32-bit byte offset
      const char* pb = reinterpret_cast<const char*>(pool);
      const uint32_t ld = (uint32_t)(uintptr_t)dst;
      const uint32_t page_b = IK ? kpage_b : vpage_b, tok_b = IK ? ktok_b : vtok_b;
      if (full) {
        // complete tile: per instruction one 64-bit page base (SGPRs)
        const char* b0 = pb + ((uint32_t)j0 & pmask) * tok_b;
#pragma unroll
        for (int m = 0; m < NI; ++m)
          dma16(b0 + (uint64_t)spage[m] * page_b, IK ? kfull[m] : vfull[m],
                ld + (uint32_t)((m * NWAVE + wave) * 64 * 16));
      } else {
        // last, partial tile: rows past the end read the last key; the
        // lane's offset is kfull / vfull moved from slot sl to its clamped slot
#pragma unroll
        for (int m = 0; m < NI; ++m) {
          const int r0 = (m * NWAVE + wave) * RPI;
          const uint32_t slot = (uint32_t)min(j0 + r0 + lane / CH, last_key) & pmask;
          const uint32_t sl = ((uint32_t)r0 & pmask) + (uint32_t)(lane / CH);
          dma16(pb + (uint64_t)spage[m] * page_b, (IK ? kfull[m] : vfull[m]) + (slot - sl) * tok_b,
                ld + (uint32_t)((m * NWAVE + wave) * 64 * 16));
        }
      }
    } else if (PM == 1 && full) {
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const uint64_t o = (uint64_t)lpage[m] * (IK ? a.k_s_page : a.v_s_page) + (IK ? kin[m] : vin[m]);
        load_lds16(pool + o, dst + (m * NWAVE + wave) * 64);
      }
    } else {
#pragma unroll
      for (int m = 0; m < NI; ++m) {
        const KeyLoc l{lpage[m], lslot[m]};
        const uint64_t o = IK ? key_offset(l, a.k_s_page, a.k_s_tok, koff[m])
                              : key_offset(l, a.v_s_page, a.v_s_tok, voff[m]);
        load_lds16(pool + o, dst + (m * NWAVE + wave) * 64);
      }
    }
  };

  // Scores of the current tile, turned into probabilities P in place.
  f32x4 s[KB][QB];
  // S^T = K Q^T, mask, online softmax: s becomes P.
  auto tile_s = [&](auto masked, const uint4* kt, int j0) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
    // The score products and the softmax run at raised wave priority (back
    // to normal as the PV products start): the other wave on the SIMD then
    // fills the gaps with its PV work instead of interleaving its own matrix
    // products into this chain, whose results gate everything after it in
    // this wave.
    {
      // K fragments are read kReadAhead products ahead of use; the scheduling
      // barriers (only scalar and vector ALU work may cross them) keep the
      // compiler from sinking the reads next to their products, where each
      // would wait out the LDS latency.
      constexpr int NF = DK * KB, PFK = kReadAhead < NF ? kReadAhead : NF;
      frag kf[NF];
      auto ldk = [&](int f) __attribute__((always_inline)) {
        const int dk = f / KB, kb = f % KB;
        const int row = wn * NW + kb * 16 + l16;
        kf[f] = __builtin_bit_cast(frag, kt[row * CH + swz_k<CH>(row, dk * 4 + g)]);
      };
#pragma unroll
      for (int f = 0; f < PFK; ++f) ldk(f);
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        if (f + PFK < NF) ldk(f + PFK);
        const int dk = f / KB, kb = f % KB;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[kb][qb] = Tr::mfma(kf[f], qf[qb][dk], s[kb][qb]);
        __builtin_amdgcn_sched_barrier(0x6);   // SALU and VALU may cross
      }
    }

    // lane owns row l16 of each qb block and keys kb*16 + 4g + i of the slice
    const int jl = j0 + wn * NW + 4 * g;
    // logits soft-cap: scores become cap * log2(e) * tanh(sm_scale * s / cap),
    // already in log2 units; masked scores are set to -inf after this, below.
    // tanh(y) = 1 - 2 / (1 + e^{2y}) (exp2 and a reciprocal) is within a few
    // ulp of 1 of tanh, so the capped logit is within ~2e-7 * cap of its
    // value: caps up to 1024 use this form alone.  Larger caps (cap_series)
    // would turn that into a visible error for logits far below the cap, so
    // there |y| < 1/4 takes the Taylor series y (1 - y^2/3 + 2y^4/15 -
    // 17y^6/315) instead, where the first form would lose the small value to
    // cancellation (relative error of either below 1e-6, so a huge cap
    // reproduces the plain logit).
    const float mul = kCap ? 1.f : a.scale_log2;
    if constexpr (kCap) {
      if (a.cap_series) {
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float y = s[kb][qb][i] * a.cap_in;
              const float y2 = y * y;
              const float series =
                  y * __builtin_fmaf(y2, __builtin_fmaf(y2, __builtin_fmaf(y2, -17.f / 315.f,
                                                                           2.f / 15.f),
                                                        -1.f / 3.f),
                                     1.f);
              const float e = fast_exp2(y * 2.8853900817779268f);   // e^{2y}
              const float big = __builtin_fmaf(-2.f, __builtin_amdgcn_rcpf(1.f + e), 1.f);
              s[kb][qb][i] = (fabsf(y) < 0.25f ? series : big) * a.cap_out;
            }
      } else {
        // 2 log2(e) * cap_in folded into one multiplier, and cap_out * (1 - 2r)
        // into one fused multiply-add
        const float c2 = a.cap_in * 2.8853900817779268f;
        const float m2 = -2.f * a.cap_out;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float e = fast_exp2(s[kb][qb][i] * c2);   // e^{2y}
              s[kb][qb][i] = __builtin_fmaf(m2, __builtin_amdgcn_rcpf(1.f + e), a.cap_out);
            }
      }
    }
    // Lazy rescaling: exponents are taken against a reference m_run per row
    // that moves only when a score exceeds it by more than kTau (log2 units),
    // so every p stays <= 2^kTau; the reference cancels in o = sum p v / sum p
    // and is added back into lse.  The common case needs no cross-lane work:
    // each lane tests its own scores against the (row-uniform) reference, and
    // only when some lane of the wave fails does the wave reduce the row
    // maxima over the four lane groups of a row and rescale.
    float mloc[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float x = s[kb][qb][i];
          if constexpr (MASKED) {
            const int j = jl + kb * 16 + i;
            bool ok = j >= lo[qb] && j <= hi[qb];
            if constexpr (kMask) {
              // the key index is clamped into the request so the byte read
              // stays inside its mask whatever ok is
              const int bit = mrow[qb] + min(max(j, 0), rq.kv_len - 1);
              ok = ok && ((a.mask[bit >> 3] >> (bit & 7)) & 1);
            }
            x = ok ? x : kNegInf;
            s[kb][qb][i] = x;
          }
          mx = fmaxf(mx, x);
        }
      }
      mloc[qb] = mx * mul;
      grow = grow || (mloc[qb] > m_run[qb] + kTau);
    }
    if (wave_any(grow)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = fmaxf(mloc[qb], __shfl_xor(mloc[qb], 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run[qb], mx);
        const float alpha = m_new == kNegInf ? 1.f : fast_exp2(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) oacc[db][qb] *= alpha;
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float m_use = (m_run[qb] == kNegInf) ? 0.f : m_run[qb];
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float p = fast_exp2(__builtin_fmaf(s[kb][qb][i], mul, -m_use));
          s[kb][qb][i] = p;
          rs += p;
        }
      }
      l_run[qb] += rs;
    }
  };

  // Gather check: tile keys [j0, j0 + NWG) below kv_end (the rest were
  // clamped re-reads of the last key) from LDS to out[kv_out_start + j][kvh].
  auto dump_tile = [&](auto is_k, const uint4* t, int j0) __attribute__((always_inline)) {
    constexpr bool IK = decltype(is_k)::value;
    uint4* out = static_cast<uint4*>(IK ? a.gather_k : a.gather_v);
    const int hkv = a.num_qo_heads / a.group;
    for (int idx = tid; idx < NWG * CH; idx += 64 * NWAVE) {
      const int r = idx / CH, c = idx % CH;
      const int j = j0 + r;
      if (j >= it.kv_end) continue;
      const int pos = IK ? swz_k<CH>(r, c) : swz_v<CH>(r, c);
      out[((int64_t)(rq.kv_out_start + j) * hkv + it.kvh) * CH + c] = t[r * CH + pos];
    }
  };

  auto tile_pv_hook = [&](const char* vt, int j0, auto&& hook) __attribute__((always_inline)) {
    if constexpr (kDump) {
      dump_tile(Flag<false>{}, reinterpret_cast<const uint4*>(vt), j0);
      hook();
      return;
    }
    // O^T += V^T P^T, 32 keys per MFMA.  B operand element e of lane
    // (g, l16) is key 4g+e (e < 4) or 16+4g+(e-4) of the 32-key step, where
    // S^T left them.  The A operand (V^T) comes from two transposing LDS
    // reads: lane r of each 16-lane group points at 4 head-dim elements
    // d0 + 4(r%4) of key 4g + r/4 (+16); the read hands lane t element
    // V[4g + k][d0 + t] as its element k.
    // V^T fragments read kReadAhead products ahead, as the K fragments above
    constexpr int NS = NW / 32, NF = NS * DB, PFV = kReadAhead < NF ? kReadAhead : NF;
    frag vf[NF];
    auto ldv = [&](int f) __attribute__((always_inline)) {
      const int st = f / DB, db = f % DB;
      const int key0 = wn * NW + st * 32 + 4 * g + (l16 >> 2);
      const int key1 = key0 + 16;
      const int d = db * 16 + 4 * (l16 & 3);        // first of 4 elements this lane points at
      const int c = d >> 3, off = (d & 7) * 2;      // chunk and byte offset inside it
      const int a0 = (key0 * CH + swz_v<CH>(key0, c)) * 16 + off;
      const int a1 = (key1 * CH + swz_v<CH>(key1, c)) * 16 + off;
      vf[f] = __builtin_bit_cast(frag, lds_read_tr16_x2(vt + a0, vt + a1));
    };
#pragma unroll
    for (int f = 0; f < PFV; ++f) ldv(f);
    frag pb[NS][QB];
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[st][qb][i] = from_f32<T>(s[2 * st][qb][i]);
          pb[st][qb][4 + i] = from_f32<T>(s[2 * st + 1][qb][i]);
        }
      }
    hook();   // runs once the first V^T reads and the conversion of P are issued
    __builtin_amdgcn_s_setprio(0);   // raised by tile_s, kept over the conversion of P
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      if (f + PFV < NF) ldv(f + PFV);
      const int st = f / DB, db = f % DB;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) oacc[db][qb] = Tr::mfma(vf[f], pb[st][qb], oacc[db][qb]);
      __builtin_amdgcn_sched_barrier(0x6);   // SALU and VALU may cross
    }
  };
  auto tile_pv = [&](const char* vt, int j0) __attribute__((always_inline)) {
    tile_pv_hook(vt, j0, [] {});
  };

  auto run_s = [&](const uint4* kt, int j0) __attribute__((always_inline)) {
    if constexpr (kDump) {
      dump_tile(Flag<true>{}, kt, j0);
      return;
    }
    if (j0 >= full_lo && j0 + NWG - 1 <= full_hi)
      tile_s(Flag<false>{}, kt, j0);
    else
      tile_s(Flag<true>{}, kt, j0);
  };
  // One LDS tile: S^T = K Q^T, online softmax, O^T += V^T P^T.
  auto run_tile = [&](const uint4* kt, const uint4* vt, int j0) __attribute__((always_inline)) {
    run_s(kt, j0);
    tile_pv(reinterpret_cast<const char*>(vt), j0);
  };

  if constexpr (kFp8) {
    // FP8 caches: each thread loads whole 16-byte key-row chunks (16 codes)
    // through the page table into registers while the current tile runs,
    // then converts them into the other LDS buffer (two bf16/fp16 chunks,
    // same swizzled layout), before the barrier that closes the tile.  The
    // short-query tiles (one work group per CU, bound by load latency) keep
    // two tiles of codes in flight in two register sets.
    constexpr int C16 = D / 16;                     // 16-byte FP8 chunks per key row
    constexpr int M8 = NWG * C16 / (64 * NWAVE);    // chunks per thread per tile
    constexpr int NS = WN > 1 ? 2 : 1;              // register staging sets
    static_assert(M8 >= 1 && NWG * C16 % (64 * NWAVE) == 0, "fp8 tile split");
    const uint8_t* kb8 = static_cast<const uint8_t*>(a.k);
    const uint8_t* vb8 = static_cast<const uint8_t*>(a.v);
    uint4 kst[NS][M8], vst[NS][M8];
    // PM 3 (power-of-two pages of at least RPW8 keys): wave instruction m
    // reads key rows r0 .. r0 + RPW8 - 1 of the tile, r0 = RPW8 * (wave +
    // NWAVE * m), all on one page, so on complete tiles its page id is a
    // scalar load and each lane adds a fixed byte offset (its row in the
    // group and its 16-byte chunk) to a scalar base: the data loads never
    // wait on per-lane page-id loads, which would hold back (in-order
    // completion) the loads of the tiles still in flight.
    constexpr int RPW8 = 64 / C16;
    const uint32_t f8k = (uint32_t)(lane / C16) * a.k_s_tok + (uint32_t)it.kvh * a.k_s_head +
                         (uint32_t)(lane % C16) * 16;
    const uint32_t f8v = (uint32_t)(lane / C16) * a.v_s_tok + (uint32_t)it.kvh * a.v_s_head +
                         (uint32_t)(lane % C16) * 16;
    auto load8 = [&](auto set, int j0) __attribute__((always_inline)) {
      constexpr int S = decltype(set)::value;
      if (PM == 3 && j0 + NWG <= it.kv_end) {
        uint32_t pg[M8];   // all page ids first: one wait for the scalar loads
#pragma unroll
        for (int m = 0; m < M8; ++m)
          pg[m] = (uint32_t)ptab_s[(uint32_t)(j0 + RPW8 * (wave + NWAVE * m)) >> a.page_shift];
#pragma unroll
        for (int m = 0; m < M8; ++m) {
          const int r0 = RPW8 * (wave + NWAVE * m);
          const uint32_t sl = (uint32_t)(j0 + r0) & (uint32_t)(a.page_size - 1);
          const uint8_t* kr = kb8 + (uint64_t)pg[m] * a.k_s_page + sl * a.k_s_tok;
          const uint8_t* vr = vb8 + (uint64_t)pg[m] * a.v_s_page + sl * a.v_s_tok;
          kst[S][m] = *reinterpret_cast<const uint4*>(kr + f8k);
          vst[S][m] = *reinterpret_cast<const uint4*>(vr + f8v);
        }
        // keeps the compiler from sinking these loads towards their use
        asm volatile("" ::: "memory");
        return;
      }
#pragma unroll
      for (int m = 0; m < M8; ++m) {
        const int gc = tid + m * 64 * NWAVE;
        const int row = gc / C16, c16 = gc - (gc / C16) * C16;
        const KeyLoc l = locate_key(ptab, (uint32_t)min(j0 + row, last_key), a.page_magic,
                                    a.page_shift, (uint32_t)a.page_size);
        kst[S][m] = *reinterpret_cast<const uint4*>(
            kb8 + key_offset(l, a.k_s_page, a.k_s_tok, (uint32_t)it.kvh * a.k_s_head + c16 * 16));
        vst[S][m] = *reinterpret_cast<const uint4*>(
            vb8 + key_offset(l, a.v_s_page, a.v_s_tok, (uint32_t)it.kvh * a.v_s_head + c16 * 16));
      }
    };
    auto store8 = [&](auto set, uint4* kdst, uint4* vdst) __attribute__((always_inline)) {
      constexpr int S = decltype(set)::value;
#pragma unroll
      for (int m = 0; m < M8; ++m) {
        const int gc = tid + m * 64 * NWAVE;
        const int row = gc / C16, c = 2 * (gc - (gc / C16) * C16);
        uint4 lo, hi;
        e4m3x16_to<T>(kst[S][m], lo, hi);
        kdst[row * CH + swz_k<CH>(row, c)] = lo;
        kdst[row * CH + swz_k<CH>(row, c + 1)] = hi;
        e4m3x16_to<T>(vst[S][m], lo, hi);
        vdst[row * CH + swz_v<CH>(row, c)] = lo;
        vdst[row * CH + swz_v<CH>(row, c + 1)] = hi;
      }
    };
    using S0 = Flag<false>;
    using S1 = Flag<(NS > 1)>;   // the second set, or the first again
    const int tb = it.tile_begin;
    if (ntiles > 0) {
      load8(S0{}, tb);
      store8(S0{}, lds_k0, lds_v0);
    }
    // Q must have landed before the loop: the compiler may issue the Q loads
    // late, and a wait for them inside the loop would also wait for the
    // staging loads in flight (in-order completion).
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int dk = 0; dk < DK; ++dk) asm volatile("" ::"v"(qf[qb][dk]));
    if (NS > 1 && ntiles > 0) load8(S1{}, tb + NWG);
    __syncthreads();
    // With two sets, raw tile u sits in set u % 2 from two tiles ahead; with
    // one, tile u + 1 is loaded as tile u starts.  With two sets the loads
    // and conversions run unconditionally (tiles past the end read the last
    // key and fill a buffer no one reads): a skipped conversion would leave
    // the compiler assuming that set's loads may still be pending, and its
    // waits before reusing the registers would then hold back the loads of
    // the other set (in-order completion).
    for (int t = 0; t < ntiles; t += 2) {
      const int j0 = tb + t * NWG;
      if constexpr (NS > 1) {
        load8(S0{}, j0 + 2 * NWG);
      } else {
        if (t + 1 < ntiles) load8(S0{}, j0 + NWG);
      }
      run_tile(lds_k0, lds_v0, j0);
      if (NS > 1 || t + 1 < ntiles) store8(S1{}, lds_k1, lds_v1);
      __syncthreads();
      if (t + 1 >= ntiles) break;
      if constexpr (NS > 1) {
        load8(S1{}, j0 + 3 * NWG);
      } else {
        if (t + 2 < ntiles) load8(S0{}, j0 + 2 * NWG);
      }
      run_tile(lds_k1, lds_v1, j0 + NWG);
      if (NS > 1 || t + 2 < ntiles) store8(S0{}, lds_k0, lds_v0);
      __syncthreads();
    }
  } else if constexpr (WN == 1) {
    // One barrier per tile: K and V of tile t + 1 are issued together once
    // the softmax of tile t is done and its first V^T reads are on their way
    // (tile_pv_hook), and waited for as it ends.  Issued as the tile starts,
    // their LDS writes slowed the score products, which gate the rest of the
    // tile (3-4% on the prefill launches); issued after the first V^T reads
    // they no longer delay those either (another ~2%).
    if (ntiles > 0) {
      fetch_pages(it.tile_begin);
      issue_part(Flag<true>{}, it.tile_begin, lds_k0);
      issue_part(Flag<false>{}, it.tile_begin, lds_v0);
      if (ntiles > 1) fetch_pages(it.tile_begin + NWG);
    }
    wait_all();
    __syncthreads();
    if (!kDump && (wm * MW >= it.nrows || it.row0 + wm * MW >= R)) {
      // a wave holding only padding rows of the task's last row tile: it
      // issues its share of the loads and meets every barrier of the loop
      // below (one per tile), computes nothing, and has no row to write
      for (int t = 0; t + 1 < ntiles; ++t) {
        const int j0 = it.tile_begin + t * NWG;
        issue_part(Flag<true>{}, j0 + NWG, (t & 1) ? lds_k0 : lds_k1);
        issue_part(Flag<false>{}, j0 + NWG, (t & 1) ? lds_v0 : lds_v1);
        if (t + 2 < ntiles) fetch_pages(j0 + 2 * NWG);
        wait_all();
        __syncthreads();
      }
      if (ntiles > 0) {
        wait_all();
        __syncthreads();
      }
      return;
    }
    for (int t = 0; t < ntiles; t += 2) {
      const int j0 = it.tile_begin + t * NWG;
      // even tile: compute from buffer 0 while buffer 1 fills
      run_s(lds_k0, j0);
      tile_pv_hook(reinterpret_cast<const char*>(lds_v0), j0, [&] {
        if (t + 1 < ntiles) {
          issue_part(Flag<true>{}, j0 + NWG, lds_k1);
          issue_part(Flag<false>{}, j0 + NWG, lds_v1);
          if (t + 2 < ntiles) fetch_pages(j0 + 2 * NWG);
        }
      });
      wait_all();
      __syncthreads();
      if (t + 1 >= ntiles) break;
      // odd tile: compute from buffer 1 while buffer 0 fills
      run_s(lds_k1, j0 + NWG);
      tile_pv_hook(reinterpret_cast<const char*>(lds_v1), j0 + NWG, [&] {
        if (t + 2 < ntiles) {
          issue_part(Flag<true>{}, j0 + 2 * NWG, lds_k0);
          issue_part(Flag<false>{}, j0 + 2 * NWG, lds_v0);
          if (t + 3 < ntiles) fetch_pages(j0 + 3 * NWG);
        }
      });
      wait_all();
      __syncthreads();
    }
  } else {
  // Short tiles: direct loads, K and V staggered by half a tile.  Tile t's
  // keys go to lds_k[t % 2] and its values to lds_v[t % 2]; V(t + 1) is
  // issued as tile t starts and K(t + 2) once every wave has finished S(t),
  // so each load has about one and a half tiles of compute to land.  The
  // per-wave counter waits below rely on these loads completing in issue
  // order (K0 V0 | K1 | V1 K2 | V2 K3 ...): the wait before S(t + 1) leaves
  // V(t + 1) and K(t + 2) in flight, the one before PV(t) leaves K(t + 1)
  // and V(t + 1); the barrier after each wait makes every wave's loads
  // visible.  Other vector memory accesses issued in between (page-id
  // loads) only make the waits stricter.  The first wait is a full one: it
  // also covers the Q loads, which the compiler tracks (it then knows they
  // are done inside the loop).
  const int tb = it.tile_begin;
  if constexpr (kQL) {
    // Q rows first (row rr of the task: packed row row0 + rr, rows past the
    // task re-read its last row), then K0, V0 and K1 before the first wait,
    // which leaves V0 and K1 in flight.  SGPR base: the task's first position; lane
    // offsets: (position - first) * s_tok + head * s_head + chunk, in bytes.
    // LDS slot c of row rr holds chunk c ^ (rr % 8) (rows are a multiple of
    // the bank width apart: the fragment reads below would otherwise take
    // 16 rows from the same banks).
    constexpr int QCH = MW * WM * CH;               // 16-byte chunks of the Q rows
    static_assert(QCH % 64 == 0, "Q rows per wave instruction");
    const int pos0 = it.row0 / G;
    const char* qbase = reinterpret_cast<const char*>(qp) +
                        ((int64_t)(rq.qo_start + pos0) * a.q_s_tok) * (int64_t)sizeof(T);
    const int rlast = min(it.row0 + it.nrows, R) - 1;
#pragma unroll
    for (int i = wave * 64; i < (kDump ? 0 : QCH); i += 64 * NWAVE) {   // no Q when gathering
      const int rr = (i + lane) / CH, c = ((i + lane) % CH) ^ (rr & 7);
      const int r = min(it.row0 + rr, rlast);
      const int pos = r / G;
      const int h = it.kvh * G + (r - pos * G);
      const uint32_t off = ((uint32_t)(pos - pos0) * (uint32_t)a.q_s_tok +
                            (uint32_t)h * (uint32_t)a.q_s_head + (uint32_t)c * 8) *
                           (uint32_t)sizeof(T);
      dma16(qbase, off, (uint32_t)(uintptr_t)lds_q + (uint32_t)i * 16);
    }
    if (ntiles > 0) {
      fetch_pages(tb);
      issue_part(Flag<true>{}, tb, lds_k0);
      issue_part(Flag<false>{}, tb, lds_v0);
      if (ntiles > 1) {
        fetch_pages(tb + NWG);
        issue_part(Flag<true>{}, tb + NWG, lds_k1);
      }
    }
    // Q and K0 landed; V0 (and K1) may still be in flight: the first tile's
    // score products need only Q and K0, and the first step's wait before its
    // PV products covers V0 (in-order completion)
    if (ntiles > 1) wait_vm_lgkm0<2 * NI>(); else if (ntiles == 1) wait_vm_lgkm0<NI>(); else wait_vm_lgkm0<0>();
    __syncthreads();
#pragma unroll
    for (int qb = 0; qb < (kDump ? 0 : QB); ++qb) {
      const int rl = wm * MW + qb * 16 + l16;
      const bool valid = rl < it.nrows && it.row0 + rl < R;
#pragma unroll
      for (int dk = 0; dk < DK; ++dk)
        qf[qb][dk] = valid ? __builtin_bit_cast(frag, lds_q[rl * CH + ((dk * 4 + g) ^ (rl & 7))])
                           : __builtin_bit_cast(frag, make_uint4(0, 0, 0, 0));
    }
  } else {
    if (ntiles > 0) {
      fetch_pages(tb);
      issue_part(Flag<true>{}, tb, lds_k0);
      issue_part(Flag<false>{}, tb, lds_v0);
      if (ntiles > 1) fetch_pages(tb + NWG);
    }
    wait_all();
    __syncthreads();
    if (ntiles > 1) issue_part(Flag<true>{}, tb + NWG, lds_k1);
  }

  // one tile; BUF is t % 2
  auto step = [&](auto buf, int t) __attribute__((always_inline)) {
    constexpr int BUF = decltype(buf)::value;
    uint4* kc = BUF ? lds_k1 : lds_k0;
    uint4* vc = BUF ? lds_v1 : lds_v0;
    uint4* vn = BUF ? lds_v0 : lds_v1;
    const int j0 = tb + t * NWG;
    if (t + 1 < ntiles) {
      issue_part(Flag<false>{}, j0 + NWG, vn);          // V(t + 1)
      if (t + 2 < ntiles) fetch_pages(j0 + 2 * NWG);
    }
    run_s(kc, j0);
    if (t + 1 < ntiles) wait_vm_lgkm0<2 * NI>(); else wait_vm_lgkm0<0>();   // V(t) landed
    __syncthreads();
    if (t + 2 < ntiles) issue_part(Flag<true>{}, j0 + 2 * NWG, kc);        // K(t + 2)
    tile_pv(reinterpret_cast<const char*>(vc), j0);
    if (t + 1 < ntiles) {
      if (t + 2 < ntiles) wait_vm_lgkm0<2 * NI>(); else wait_vm_lgkm0<NI>();  // K(t + 1) landed
      __syncthreads();
    }
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(Flag<0>{}, t);
    if (t + 1 >= ntiles) break;
    step(Flag<1>{}, t + 1);
  }
  __syncthreads();   // the epilogue below reuses the buffers
  }   // FP8 / direct-load paths

  if constexpr (kDump) return;   // the gather check writes no attention output

  // ---- epilogue
  // Row sums were kept per lane; reduce over the 4 lane groups sharing a row.
  float l_tot[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float x = l_run[qb] + __shfl_xor(l_run[qb], 16);
    l_tot[qb] = x + __shfl_xor(x, 32);
  }

  T* __restrict__ op = static_cast<T*>(a.o);
  const bool to_partial = it.slot >= 0;

  if constexpr (WN == 1) {
    if (to_partial) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int rl = wm * MW + qb * 16 + l16;  // row within the task
        const int r = it.row0 + rl;
        if (rl >= it.nrows || r >= R) continue;
        float inv = l_tot[qb] > 0.f ? 1.f / l_tot[qb] : 0.f;
        if constexpr (kFp8) inv *= a.v_scale;   // V = codes * v_scale
        const float lse2 = l_tot[qb] > 0.f ? m_run[qb] + fast_log2(l_tot[qb]) : kNegInf;
        float* dst = a.part_o + ((int64_t)it.slot * (WM * MW) + rl) * D;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          f32x4 v = oacc[db][qb] * inv;
          *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * g) = v;
        }
        if (g == 0) a.part_lse[(int64_t)it.slot * (WM * MW) + rl] = lse2;
      }
    } else {
      // O in the q dtype, staged through LDS (the K/V buffers are free once
      // the key loop has ended).  A lane holds 4-element pieces of 16 rows, so
      // storing from registers writes 32-byte pieces of 16 rows per
      // instruction; from LDS each lane stores a whole 16-byte chunk and one
      // instruction covers 64 / CH consecutive rows (whole output rows of
      // consecutive heads).  Wave w's region: its MW rows of CH chunks, chunk
      // c of row r at position swz_k(r, c); orow_w[r] is row r's output row,
      // or -1 past the task.  Each wave reads back only what its own lanes
      // wrote, and LDS completes one wave's accesses in order.
      static_assert((WM / 2) * MW * D * (int)sizeof(T) <= (int)sizeof(lds_k0), "LDS too small");
      static_assert(WM * MW * 8 <= (int)sizeof(lds_k1), "LDS too small");
      char* stage = reinterpret_cast<char*>(wm < WM / 2 ? lds_k0 : lds_v0) +
                    (wm % (WM / 2)) * MW * D * (int)sizeof(T);
      int64_t* orow_w = reinterpret_cast<int64_t*>(lds_k1) + wm * MW;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int rw = qb * 16 + l16;           // row within the wave
        const int rl = wm * MW + rw;            // row within the task
        const int r = it.row0 + rl;
        const bool valid = rl < it.nrows && r < R;
        float inv = l_tot[qb] > 0.f ? 1.f / l_tot[qb] : 0.f;
        if constexpr (kFp8) inv *= a.v_scale;   // V = codes * v_scale
        int64_t orow = -1;
        if (valid) {
          const int pos = r / G;
          const int h = it.kvh * G + (r - pos * G);
          orow = (int64_t)(rq.qo_start + pos) * a.num_qo_heads + h;
        }
        if (g == 0) {
          orow_w[rw] = orow;
          if (valid && a.lse != nullptr)
            a.lse[orow] = l_tot[qb] > 0.f ? (m_run[qb] + fast_log2(l_tot[qb])) * kLn2 : kNegInf;
        }
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          T o4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) o4[i] = from_f32<T>(oacc[db][qb][i] * inv);
          const int c = db * 2 + (g >> 1);      // chunk of elements db * 16 + 4g .. + 3
          *reinterpret_cast<uint2*>(stage + (rw * CH + swz_k<CH>(rw, c)) * 16 + (g & 1) * 8) =
              *reinterpret_cast<uint2*>(o4);
        }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int i = lane; i < MW * CH; i += 64) {
        const int rw = i / CH, c = i % CH;
        const int64_t orow = orow_w[rw];
        const uint4 v = *reinterpret_cast<const uint4*>(stage + (rw * CH + swz_k<CH>(rw, c)) * 16);
        if (orow >= 0) *reinterpret_cast<uint4*>(op + orow * D + c * 8) = v;
      }
    }
  } else {
    // Waves along keys hold partial states of the same rows: combine in LDS.
    static_assert(WM == 1, "key-split tiles use one row block");
    // per-wave [MW][D] fp32 slices: waves 0..WN/2-1 in lds_k0, the rest in lds_k1.
    // The 16-byte chunk c of row r sits at chunk c ^ (r % 8) of the row: rows
    // are a multiple of the 128-byte bank width apart, so the plain layout
    // would put the 16 rows a wave writes at once in the same banks.
    auto red_o_of = [&](int w) -> float* {
      float* base = reinterpret_cast<float*>(w < WN / 2 ? lds_k0 : lds_k1);
      return base + (w % (WN / 2)) * MW * D;
    };
    float* red_m = reinterpret_cast<float*>(lds_v0);     // [WN][MW]
    float* red_l = red_m + WN * MW;                      // [WN][MW]
    static_assert(WN % 2 == 0 && (WN / 2) * MW * D * 4 <= (int)sizeof(lds_k0), "LDS too small");
    // orow_t[r]: output row of row r (any value >= 0 for a partial tile), -1 past the task
    int64_t* orow_t = reinterpret_cast<int64_t*>(red_l + WN * MW);
    static_assert(2 * WN * MW * 4 + MW * 8 <= (int)sizeof(lds_v0), "LDS too small");
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (g == 0) {
        red_m[wn * MW + qb * 16 + l16] = m_run[qb];
        red_l[wn * MW + qb * 16 + l16] = l_tot[qb];
      }
    }
    __syncthreads();
    // Each wave folds the whole row normalisation into its own slice,
    // o_w 2^(m_w - mt) / lt with mt = max_w m_w and lt = sum_w l_w 2^(m_w - mt),
    // so the slices only need adding up; wave 0 writes each row's lse and
    // output row.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int rl = qb * 16 + l16;
      float mt = kNegInf;
#pragma unroll
      for (int w = 0; w < WN; ++w) mt = fmaxf(mt, red_m[w * MW + rl]);
      const float mu = (mt == kNegInf) ? 0.f : mt;
      float lt = 0.f;
#pragma unroll
      for (int w = 0; w < WN; ++w) lt += red_l[w * MW + rl] * fast_exp2(red_m[w * MW + rl] - mu);
      float inv = lt > 0.f ? 1.f / lt : 0.f;
      if constexpr (kFp8) inv *= a.v_scale;   // V = codes * v_scale
      const float sc = fast_exp2(m_run[qb] - mu) * inv;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        f32x4 v = oacc[db][qb] * sc;
        *reinterpret_cast<f32x4*>(red_o_of(wn) + rl * D + ((db * 4 + g) ^ (rl & 7)) * 4) = v;
      }
      if (wn == 0 && g == 0) {
        const int r = it.row0 + rl;
        const float lse2 = lt > 0.f ? mt + fast_log2(lt) : kNegInf;
        int64_t orow = -1;
        if (rl < it.nrows && r < R) {
          if (to_partial) {
            orow = 0;
            a.part_lse[(int64_t)it.slot * MW + rl] = lse2;
          } else {
            const int pos = r / G;
            const int h = it.kvh * G + (r - pos * G);
            orow = (int64_t)(rq.qo_start + pos) * a.num_qo_heads + h;
            if (a.lse != nullptr) a.lse[orow] = lse2 == kNegInf ? kNegInf : lse2 * kLn2;
          }
        }
        orow_t[rl] = orow;
      }
    }
    __syncthreads();
    // Every thread adds up the slices for 4 consecutive head-dim elements of some rows.
    for (int idx = tid; idx < MW * (D / 4); idx += 64 * NWAVE) {
      const int rl = idx / (D / 4);
      const int d4 = idx - rl * (D / 4);
      const int64_t orow = orow_t[rl];
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int w = 0; w < WN; ++w)
        acc += *reinterpret_cast<const f32x4*>(red_o_of(w) + rl * D + (d4 ^ (rl & 7)) * 4);
      if (orow < 0) continue;
      if (to_partial) {
        *reinterpret_cast<f32x4*>(a.part_o + ((int64_t)it.slot * MW + rl) * D + d4 * 4) = acc;
      } else {
        T o4[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) o4[i] = from_f32<T>(acc[i]);
        *reinterpret_cast<uint2*>(op + orow * D + d4 * 4) = *reinterpret_cast<uint2*>(o4);
      }
    }
  }
}

template <typename T, int D, int PM, int VAR>
static hipError_t launch_attention_pm(int tile_kind, const AttnArgs& a, hipStream_t s) {
  dim3 grid(a.num_work);
  if constexpr (D == 256) {   // one shape: 4 waves x 16 rows, 32-key tiles, one wave per SIMD
    if (tile_kind != TILE_PREFILL) return hipErrorInvalidValue;
    hipLaunchKernelGGL((attn_kernel<T, D, 4, 1, 1, 32, 1, PM, VAR>), grid, dim3(256), 0, s, a);
  } else {
    switch (tile_kind) {
      case TILE_PREFILL:
        hipLaunchKernelGGL((attn_kernel<T, D, 4, 1, 2, 64, 2, PM, VAR>), grid, dim3(256), 0, s, a);
        break;
      case TILE_SHORT16:
        hipLaunchKernelGGL((attn_kernel<T, D, 1, 4, 1, 32, 2, PM, VAR>), grid, dim3(256), 0, s, a);
        break;
      case TILE_SHORT32:
        hipLaunchKernelGGL((attn_kernel<T, D, 1, 4, 2, 32, 2, PM, VAR>), grid, dim3(256), 0, s, a);
        break;
      default:
        return hipErrorInvalidValue;
    }
  }
  return hipGetLastError();
}

template <typename T, int D, int VAR>
static hipError_t launch_attention_t(int tile_kind, const AttnArgs& a, hipStream_t s) {
  if (a.num_work == 0) return hipSuccess;
  const bool pow2 = (a.page_size & (a.page_size - 1)) == 0;
  if constexpr ((VAR & 4) != 0) {
    // FP8: scalar page ids when a page holds a whole wave instruction's rows
    if (pow2 && a.page_size >= 64 / (D / 16))
      return launch_attention_pm<T, D, 3, VAR>(tile_kind, a, s);
    return launch_attention_pm<T, D, 0, VAR>(tile_kind, a, s);
  } else {
    // 32-bit byte offsets: page strides, and (short tiles, Q through LDS)
    // a tile's Q rows from its first position
    const bool page_b32 =
        (uint64_t)a.k_s_page * sizeof(T) < (1ull << 32) &&
        (uint64_t)a.v_s_page * sizeof(T) < (1ull << 32) &&
        ((uint64_t)a.q_s_tok * 33 + (uint64_t)a.q_s_head * a.num_qo_heads + D) * sizeof(T) <
            (1ull << 32);
    if (pow2 && a.page_size >= 512 / D) {
      if (page_b32) return launch_attention_pm<T, D, 3, VAR>(tile_kind, a, s);
      return launch_attention_pm<T, D, 0, VAR>(tile_kind, a, s);   // pages of 4 GiB or more
    }
    if (pow2) return launch_attention_pm<T, D, 1, VAR>(tile_kind, a, s);
    return launch_attention_pm<T, D, 0, VAR>(tile_kind, a, s);
  }
}

template <int VAR>
hipError_t launch_attention_var(int tile_kind, int dtype, int head_dim, const AttnArgs& a,
                                hipStream_t s) {
  if (dtype == 1 && head_dim == 128) return launch_attention_t<__bf16, 128, VAR>(tile_kind, a, s);
  if (dtype == 1 && head_dim == 64) return launch_attention_t<__bf16, 64, VAR>(tile_kind, a, s);
  if (dtype == 0 && head_dim == 128) return launch_attention_t<_Float16, 128, VAR>(tile_kind, a, s);
  if (dtype == 0 && head_dim == 64) return launch_attention_t<_Float16, 64, VAR>(tile_kind, a, s);
  if (dtype == 1 && head_dim == 256) return launch_attention_t<__bf16, 256, VAR>(tile_kind, a, s);
  if (dtype == 0 && head_dim == 256) return launch_attention_t<_Float16, 256, VAR>(tile_kind, a, s);
  return hipErrorInvalidValue;
}

}  // namespace pkv
