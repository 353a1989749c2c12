// Internal helpers shared by the libsvlm kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string>

#include "svlm.h"

namespace svlm {

// ---------------------------------------------------------------------------
// host side: status reporting
// ---------------------------------------------------------------------------
int fail(int status, const char* fmt, ...);        // records svlm_last_error(), returns status
int check_launch(const char* what);                // hipGetLastError() -> SVLM_E_HIP / SVLM_OK
int num_cus();                                     // compute units of the current device (cached)

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// ---------------------------------------------------------------------------
// device side: vector types for the bf16 matrix-core builtins
// ---------------------------------------------------------------------------
typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short bf16x4;
typedef __attribute__((__vector_size__(2 * sizeof(unsigned)))) unsigned u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

// v_mfma_f32_16x16x32_bf16.  Lane l (c = l % 16, g = l / 16):
//   a holds A[m = c][k = 8g .. 8g+7], b holds B[k = 8g .. 8g+7][n = c],
//   acc holds C[m = 4g .. 4g+3][n = c].
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x16_bf16.  Lane l (c = l % 16, g = l / 16):
//   a holds A[m = c][k = 4g .. 4g+3], b holds B[k = 4g .. 4g+3][n = c],
//   acc holds C[m = 4g .. 4g+3][n = c].
__device__ __forceinline__ f32x4 mfma16k16(const bf16x4& a, const bf16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 as_bf16x4(const u32x2& v) {
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

// Select two 16-bit halves: result.lo = lo_src half, result.hi = hi_src half.
// sel 0x05040100 takes the low halves, 0x07060302 the high halves.
__device__ __forceinline__ unsigned perm(unsigned hi_src, unsigned lo_src, unsigned sel) {
  return __builtin_amdgcn_perm(hi_src, lo_src, sel);
}
constexpr unsigned kPermLo = 0x05040100u;
constexpr unsigned kPermHi = 0x07060302u;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float bits_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f_bits(float f) { return __builtin_bit_cast(unsigned, f); }

// max(a, b) for non-NaN operands as one v_max_f32: fmaxf would first quiet
// possible NaNs in every operand it cannot prove canonical (cross-lane
// results, for one), which doubles the instruction count of a max tree.
__device__ __forceinline__ float fmax_nn(float a, float b) {
  float r;
  __asm__("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

// Cross-lane butterflies on the VALU (gfx950 v_permlane16/32_swap): after the
// swap the two results hold the values of lanes l and l ^ 16 (or l ^ 32).
// The max forms take non-NaN operands.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  return fmax_nn(bits_f(r[0]), bits_f(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return fmax_nn(bits_f(r[0]), bits_f(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(r[0]) + bits_f(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(f_bits(x), f_bits(x), false, false);
  return bits_f(r[0]) + bits_f(r[1]);
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace svlm
