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

// a * b for non-negative operands, saturated at INT64_MAX
inline int64_t mul_sat(int64_t a, int64_t b) { return (a != 0 && b > INT64_MAX / a) ? INT64_MAX : a * b; }

// Dispatch limits that every launch here stays within: the x dimension counts
// work-items (workgroups x threads) below 2^31, y and z count workgroups below
// 2^16.  Callers form the workgroup counts in 64 bits, before any narrowing.
inline bool grid_fits(int64_t x_blocks, int threads, int64_t y = 1, int64_t z = 1) {
  return x_blocks >= 1 && x_blocks <= INT32_MAX / threads && y >= 1 && y < 65536 && z >= 1 && z < 65536;
}

// ---------------------------------------------------------------------------
// debug builds (-DSVLM_DEBUG): kernels record violated device preconditions.
// Device variables are not shared between the library's code objects, so
// each source file holds its own flag word and a host function that takes
// (reads and clears) it; svlm_debug_flags() collects them.
// ---------------------------------------------------------------------------
#ifdef SVLM_DEBUG
static __device__ unsigned g_debug_flags;
__device__ __forceinline__ void debug_check(bool ok, unsigned bit) {
  if (!ok) __hip_atomic_fetch_or(&g_debug_flags, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// this file's flags, cleared; false on a HIP error
static inline bool debug_take_here(unsigned* out) {
  unsigned v = 0;
  const unsigned zero = 0;
  if (hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_debug_flags), sizeof v) != hipSuccess) return false;
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_debug_flags), &zero, sizeof zero) != hipSuccess) return false;
  *out = v;
  return true;
}
bool debug_take_decode_attn(unsigned* out);
bool debug_take_f32_path(unsigned* out);
bool debug_take_gather(unsigned* out);
bool debug_take_select(unsigned* out);
bool debug_take_verify(unsigned* out);
#else
__device__ __forceinline__ void debug_check(bool, unsigned) {}
#endif

// ---------------------------------------------------------------------------
// fp32 operands (SVLM_F32): plain vector-ALU kernels in f32_path.hip
// ---------------------------------------------------------------------------
struct AttnF32Args {
  const float* q;
  int64_t q_sb;
  const float* k;
  const float* v;
  int64_t kv_sb, kv_sh, kv_sn;
  const int32_t* kv_len;  // key count of (b, g) at kv_len[b * len_sb + g * len_sh]
  int64_t len_sb, len_sh;
  int max_kv_len;
  const int32_t* kv_idx;  // nullptr: keys are cache rows 0 .. n - 1
  int64_t idx_sb, idx_sh;
  int kv_rows;
  int batch, nq, Hq, Hkv, D;
  float scale;
  int causal;
  float* out;
  float* lse;
};
void launch_attn_f32(const AttnF32Args& a, hipStream_t st);

struct ScoreF32Args {
  const float* q;
  int64_t q_st, q_sh;
  const float* k;
  int64_t k_sh, k_sn;
  int T, q_pos0, vis_start, n_vis, Hq, Hkv, D;
  float scale;
  float* lse;  // workspace [Hq][T], natural log
  int agg;
  float alpha, beta;
  float* out;
};
void launch_score_f32(const ScoreF32Args& a, int rows, hipStream_t st);

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
__device__ __forceinline__ float fmax3_nn(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
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


// ---------------------------------------------------------------------------
// device side: buffer loads, LDS-DMA staging and their waits
// ---------------------------------------------------------------------------
// buffer descriptor word 3 for gfx9-family raw buffer loads (no swizzle, no stride)
constexpr int kBufferFlags = 0x00020000;
// cache policy of the streaming KV loads: nontemporal
constexpr int kNT = 2;

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int enc = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  __builtin_amdgcn_s_waitcnt(enc);
  __asm__ volatile("" ::: "memory");
}

// LDS reads of one staged key block, issued together and waited for inside
// the same asm block, so no read is in flight when the outputs are used.  The
// staging ring is written by LDS-DMA transfers whose completion the kernel
// tracks with its own vmcnt waits; reads that the compiler cannot see keep it
// from adding waits on every transfer in flight.  Outputs are early-clobber:
// a read may complete while later reads of the block are still queued.
__device__ __forceinline__ void lds_read_b128x8(u32x4 (&d)[8], const unsigned (&a)[8]) {
  __asm__ volatile(
      "ds_read_b128 %0, %8\n\t"
      "ds_read_b128 %1, %9\n\t"
      "ds_read_b128 %2, %10\n\t"
      "ds_read_b128 %3, %11\n\t"
      "ds_read_b128 %4, %12\n\t"
      "ds_read_b128 %5, %13\n\t"
      "ds_read_b128 %6, %14\n\t"
      "ds_read_b128 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3]), "=&v"(d[4]), "=&v"(d[5]), "=&v"(d[6]), "=&v"(d[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}
__device__ __forceinline__ void lds_read_b128x2(u32x4 (&d)[2], const unsigned (&a)[2]) {
  __asm__ volatile(
      "ds_read_b128 %0, %2\n\t"
      "ds_read_b128 %1, %3\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1])
      : "v"(a[0]), "v"(a[1])
      : "memory");
}
__device__ __forceinline__ void lds_read_b128x4(u32x4 (&d)[4], const unsigned (&a)[4]) {
  __asm__ volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %5\n\t"
      "ds_read_b128 %2, %6\n\t"
      "ds_read_b128 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d[0]), "=&v"(d[1]), "=&v"(d[2]), "=&v"(d[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}
__device__ __forceinline__ void lds_read_b128x2_b64x4(u32x4 (&k)[2], u32x2 (&v)[4], const unsigned (&a)[6]) {
  __asm__ volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b64 %2, %8\n\t"
      "ds_read_b64 %3, %9\n\t"
      "ds_read_b64 %4, %10\n\t"
      "ds_read_b64 %5, %11\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(k[0]), "=&v"(k[1]), "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5])
      : "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  __asm__ volatile("" ::: "memory");
}

// Workgroup-wide execution barrier without a memory fence: LDS-DMA staging
// slots are handed over by each wave's own vmcnt waits before it, so the
// barrier must not drain the transfers still in flight (a fenced barrier
// waits for every outstanding vector-memory operation).
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return (unsigned)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

}  // namespace svlm
