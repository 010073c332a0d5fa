// Device helpers shared by the HIP kernel files: operand types and MFMA
// wrappers, the page-table address path, LDS swizzles, direct global->LDS
// loads and transposing LDS reads.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

#include "pkv_internal.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kTau = 8.f;   // lazy-rescale threshold, log2 units
constexpr float kNegInf = -__builtin_inff();

template <typename T>
struct Traits;

template <>
struct Traits<__bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x4 mfma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Traits<_Float16> {
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x4 mfma(frag a, frag b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

template <typename T>
__device__ __forceinline__ float to_f32(T x) {
  return static_cast<float>(x);
}

template <typename T>
__device__ __forceinline__ T from_f32(float x) {
  return static_cast<T>(x);  // round to nearest even
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }


// Page-table address path, shared by the attention and debug-gather kernels:
// logical key j of a request lives on page ptab[j / P] at slot j % P, and
// element e of head h of that key at page * s_page + slot * s_tok + h * s_head + e.
struct KeyLoc {
  uint32_t page, slot;
};
__device__ __forceinline__ KeyLoc locate_key(const int32_t* ptab, uint32_t j, uint32_t magic,
                                             uint32_t shift, uint32_t page_size) {
  const uint32_t pidx = (uint32_t)(((uint64_t)j * magic) >> shift);
  return KeyLoc{(uint32_t)ptab[pidx], j - pidx * page_size};
}
__device__ __forceinline__ uint64_t key_offset(KeyLoc k, uint32_t s_page, uint32_t s_tok,
                                               uint32_t in_page) {
  return (uint64_t)k.page * s_page + (k.slot * s_tok + in_page);
}

// ---------------------------------------------------------------------------
// attention
// ---------------------------------------------------------------------------
// LDS tiles hold key rows of D elements as CH = D/8 16-byte chunks,
// row-major and unpadded, with the chunk order permuted per row so that the
// reads of one MFMA fragment spread over all banks:
//  * K (16-byte reads, consecutive lanes on consecutive rows, same chunk):
//    chunk c of row r sits at position c ^ (r & 15) (r & 7 when CH = 8);
//  * V (transposing 8-byte reads: 16 lanes cover 4 consecutive keys x 2
//    adjacent chunks): chunk c of key k sits at c ^ ((2k) & (CH - 1)), which
//    keeps those 8 chunks, and 32 lanes' 16, on distinct positions.
template <int CH>
__device__ __forceinline__ int swz_k(int row, int chunk) {
  return chunk ^ (row & (CH >= 16 ? 15 : 7));
}
template <int CH>
__device__ __forceinline__ int swz_v(int key, int chunk) {
  return chunk ^ ((2 * key) & (CH - 1));
}

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// 16 bytes from global memory straight into LDS: lane i of the wave writes
// dst + 16 * i (dst is wave-uniform).
__device__ __forceinline__ void load_lds16(const void* src, void* dst) {
  __builtin_amdgcn_global_load_lds(src, dst, 16, 0, 0);
}
// The same load in its saddr form, issued from assembly: 16 bytes per lane
// from sbase + voff (sbase wave-uniform, voff a per-lane 32-bit byte offset)
// into LDS at lds + 16 * lane.  The compiler neither tracks nor waits for it:
// the caller waits (s_waitcnt vmcnt) and synchronises before any wave reads
// the destination.  M0 carries the LDS base; nothing else in these kernels
// uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"   // M0 is listed as clobbered on purpose
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, uint32_t lds) {
  // sbase and lds are uniform over the wave; readfirstlane makes that
  // explicit so the "s" operands get SGPRs even where the compiler's
  // uniformity analysis cannot prove it (it is free when they already are).
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t bs = ((uint64_t)__builtin_amdgcn_readfirstlane((uint32_t)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t ls = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(reinterpret_cast<const char*>(bs)), "s"(ls)
               : "memory", "m0");
}
#pragma clang diagnostic pop
// 16 FP8 E4M3 codes (16 bytes, lowest first) to 16 values of T, returned as
// two 8-element chunks.  Every E4M3 value is exact in bf16 and fp16.
template <typename T>
__device__ __forceinline__ void e4m3x16_to(uint4 in, uint4& lo, uint4& hi) {
  // One instruction per two codes, straight to the 16-bit type (scale 1).
  const uint32_t w[4] = {in.x, in.y, in.z, in.w};
  uint32_t out[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (__is_same(T, __bf16)) {
      out[2 * i] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, false));  // bytes 0, 1
      out[2 * i + 1] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)w[i], 1.0f, true));   // bytes 2, 3
    } else {
      out[2 * i] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[i], 1.0f, false));
      out[2 * i + 1] = __builtin_bit_cast(
          uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((int)w[i], 1.0f, true));
    }
  }
  lo = make_uint4(out[0], out[1], out[2], out[3]);
  hi = make_uint4(out[4], out[5], out[6], out[7]);
}
// Loads through this pointer type are scalar (constant address space).
typedef __attribute__((address_space(4))) const int32_t const_i32;
// Wait for every outstanding memory operation of this wave.
__device__ __forceinline__ void wait_all() { __builtin_amdgcn_s_waitcnt(0); }
// Wait until at most N vector memory loads of this wave are outstanding and
// every LDS / scalar memory access has completed (gfx9 s_waitcnt encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// Two transposing 8-byte LDS reads joined into one 8-element fragment.
__device__ __forceinline__ i16x8 lds_read_tr16_x2(const char* p0, const char* p1) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p0);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p1);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ bool wave_any(bool x) { return __any(x); }

template <bool B>
struct Flag {
  static constexpr bool value = B;
};

}  // namespace pkv
