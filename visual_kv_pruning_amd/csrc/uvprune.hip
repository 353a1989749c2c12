// svlm_uvprune_score: UV-Prune score of every video token.
//
// ParallelVLM notes, method section 1 ("UV-Prune"): with S^l_ij the cosine
// similarity of video token i and text token j at target layer l, the score
// is dS_i = sum_j sum_l (S^l_ij - S^(l-1)_ij), and the kept tokens are the
// top-K of dS.  The sum over l telescopes to S^L_ij - S^0_ij, and the sum
// over j of a cosine is one dot product with the sum of the normalised text
// vectors:
//   dS_i = <V^L_i, xbar^L> / |V^L_i| - <V^0_i, xbar^0> / |V^0_i|,
//   xbar^l = sum_j X^l_j / |X^l_j|,
// so the work is one streaming pass over the video hidden states of the two
// layers (HBM-bound), after two small passes over the text.
//
// Three launches: text row norms (one workgroup per text row and layer), the
// normalised text sums (64 dimensions per workgroup, rows split over its four
// waves and added in a fixed order), and
// the video rows (one wave per row, the two text sums staged in LDS, the
// rows read with nontemporal loads since each byte is read once).  All
// reductions run in a fixed order, so results are deterministic.  A zero
// vector's similarities are 0.
#include <algorithm>
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr int kThreads = 256;
constexpr int kMaxDim = 16384;  // the two fp32 text sums (2 x 64 KB) fit in LDS
constexpr int kLoadBatch = 4;   // text-row chunks per thread in flight (text norms)

struct UvArgs {
  const uint16_t* v0;
  const uint16_t* vL;
  int64_t v_sn;
  int n_vis;
  const uint16_t* x0;
  const uint16_t* xL;
  int64_t x_sn;
  int n_text, d;
  float out_scale, out_offset;
  float* out;
  float* inv_x;  // [2][n_text]
  float* xbar;   // [2][d]
};

__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float inv_norm(float sumsq) { return sumsq > 0.f ? 1.f / sqrtf(sumsq) : 0.f; }

// 1 / |X^l_j| for every text row j and layer l (blockIdx.y)
__global__ __launch_bounds__(kThreads) void text_norms(UvArgs a) {
  const int j = blockIdx.x, layer = blockIdx.y;
  const uint16_t* row = (layer ? a.xL : a.x0) + (int64_t)j * a.x_sn;
  // kLoadBatch chunks per thread in flight, summed in the order of a plain loop
  const int nc = a.d / 8;
  float ss = 0.f;
  for (int c0 = threadIdx.x; c0 < nc; c0 += kThreads * kLoadBatch) {
    u32x4 w[kLoadBatch];
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) {
      const int c = c0 + u * kThreads;
      w[u] = (c < nc) ? *(const u32x4*)(row + 8 * c) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kLoadBatch; ++u) {
      if (c0 + u * kThreads >= nc) break;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float lo = bf16_lo(w[u][e]), hi = bf16_hi(w[u][e]);
        ss = fmaf(lo, lo, ss);
        ss = fmaf(hi, hi, ss);
      }
    }
  }
  ss = wave_sum(ss);
  __shared__ float sm[kThreads / 64];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += sm[w];
    a.inv_x[layer * a.n_text + j] = inv_norm(t);
  }
}

// xbar^l[k] = sum_j X^l_j[k] / |X^l_j|: a workgroup takes 64 dimensions; its
// four waves sum the rows j = w, w + 4, ... (many loads in flight), and the
// four partial sums are added in wave order
__global__ __launch_bounds__(kThreads) void text_sums(UvArgs a) {
  const int layer = blockIdx.y;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int k = blockIdx.x * 64 + lane;
  const uint16_t* x = layer ? a.xL : a.x0;
  const float* inv = a.inv_x + layer * a.n_text;
  float acc = 0.f;
  if (k < a.d) {
#pragma unroll 8
    for (int j = wv; j < a.n_text; j += kThreads / 64)
      acc = fmaf(__uint_as_float((unsigned)x[(int64_t)j * a.x_sn + k] << 16), inv[j], acc);
  }
  __shared__ float part[kThreads / 64][64];
  part[wv][lane] = acc;
  __syncthreads();
  if (wv == 0 && k < a.d) {
    float t = 0.f;
#pragma unroll
    for (int w = 0; w < kThreads / 64; ++w) t += part[w][lane];
    a.xbar[layer * a.d + k] = t;
  }
}

// one wave per video row: |V^0_i|^2, <V^0_i, xbar^0>, |V^L_i|^2, <V^L_i, xbar^L>
constexpr int kRowUnroll = 8;  // 16-byte chunks per lane in flight per layer
constexpr int kXbarBatch = 16; // text-sum loads per thread in flight when LDS is filled

__device__ __forceinline__ void row_chunk(const u32x4& w0, const u32x4& wL, const float4* xb, int d4, int c,
                                          float& ss0, float& dt0, float& ssL, float& dtL) {
  const float4 b0 = xb[2 * c], b1 = xb[2 * c + 1];
  const float4 c0 = xb[d4 + 2 * c], c1 = xb[d4 + 2 * c + 1];
  const float xb0[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
  const float xbL[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float p = bf16_lo(w0[e]), q = bf16_hi(w0[e]);
    ss0 = fmaf(p, p, ss0);
    ss0 = fmaf(q, q, ss0);
    dt0 = fmaf(p, xb0[2 * e], dt0);
    dt0 = fmaf(q, xb0[2 * e + 1], dt0);
    const float s = bf16_lo(wL[e]), t = bf16_hi(wL[e]);
    ssL = fmaf(s, s, ssL);
    ssL = fmaf(t, t, ssL);
    dtL = fmaf(s, xbL[2 * e], dtL);
    dtL = fmaf(t, xbL[2 * e + 1], dtL);
  }
}

__global__ __launch_bounds__(kThreads) void video_scores(UvArgs a) {
  extern __shared__ float4 sm_xbar[];  // [2][d / 4]
  const int d4 = a.d / 4;
  // the text sums into LDS, kXbarBatch loads per thread in flight
  for (int k0 = threadIdx.x; k0 < 2 * d4; k0 += kThreads * kXbarBatch) {
    float4 t[kXbarBatch];
#pragma unroll
    for (int u = 0; u < kXbarBatch; ++u) {
      const int k = k0 + u * kThreads;
      t[u] = (k < 2 * d4) ? ((const float4*)a.xbar)[k] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < kXbarBatch; ++u) {
      const int k = k0 + u * kThreads;
      if (k < 2 * d4) sm_xbar[k] = t[u];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int waves = gridDim.x * (kThreads / 64);
  const int chunks = a.d / 8;
  const int full = chunks / (64 * kRowUnroll) * (64 * kRowUnroll);  // chunks covered by whole groups
  for (int i = blockIdx.x * (kThreads / 64) + wave; i < a.n_vis; i += waves) {
    const u32x4* r0 = (const u32x4*)(a.v0 + (int64_t)i * a.v_sn);
    const u32x4* rL = (const u32x4*)(a.vL + (int64_t)i * a.v_sn);
    float ss0 = 0.f, dt0 = 0.f, ssL = 0.f, dtL = 0.f;
    for (int c0 = 0; c0 < full; c0 += 64 * kRowUnroll) {
      u32x4 w0[kRowUnroll], wL[kRowUnroll];
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) {  // every load of the group first; nontemporal: read once
        w0[u] = __builtin_nontemporal_load(&r0[c0 + 64 * u + lane]);
        wL[u] = __builtin_nontemporal_load(&rL[c0 + 64 * u + lane]);
      }
#pragma unroll
      for (int u = 0; u < kRowUnroll; ++u) row_chunk(w0[u], wL[u], sm_xbar, d4, c0 + 64 * u + lane, ss0, dt0, ssL, dtL);
    }
    for (int c = full + lane; c < chunks; c += 64)
      row_chunk(__builtin_nontemporal_load(&r0[c]), __builtin_nontemporal_load(&rL[c]), sm_xbar, d4, c, ss0, dt0,
                ssL, dtL);
    ss0 = wave_sum(ss0);
    dt0 = wave_sum(dt0);
    ssL = wave_sum(ssL);
    dtL = wave_sum(dtL);
    if (lane == 0) {
      const float ds = dtL * inv_norm(ssL) - dt0 * inv_norm(ss0);
      a.out[i] = fmaf(a.out_scale, ds, a.out_offset);
    }
  }
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" size_t svlm_uvprune_workspace(int n_text, int d) {
  if (n_text < 1 || d < 1) return 0;
  return ((size_t)2 * n_text * sizeof(float) + 255) / 256 * 256 + (size_t)2 * d * sizeof(float);
}

extern "C" int svlm_uvprune_score(const void* v0, const void* vL, int64_t v_sn, int n_vis, const void* x0,
                                  const void* xL, int64_t x_sn, int n_text, int d, int dtype, float out_scale,
                                  float out_offset, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != SVLM_BF16) return fail(SVLM_E_UNSUPPORTED, "svlm_uvprune_score: only SVLM_BF16 hidden states");
  if (n_vis < 1 || n_text < 1 || d < 1) return fail(SVLM_E_INVALID, "svlm_uvprune_score: n_vis, n_text, d must be >= 1");
  if (d % 8 || d > kMaxDim)
    return fail(SVLM_E_UNSUPPORTED, "svlm_uvprune_score: d must be a multiple of 8 and <= %d (got %d)", kMaxDim, d);
  if (!v0 || !vL || !x0 || !xL || !out) return fail(SVLM_E_INVALID, "svlm_uvprune_score: null pointer");
  if (v_sn < d || x_sn < d || v_sn % 8 || x_sn % 8)
    return fail(SVLM_E_INVALID, "svlm_uvprune_score: row strides must be multiples of 8 elements and >= d");
  if (!aligned16(v0) || !aligned16(vL) || !aligned16(x0) || !aligned16(xL))
    return fail(SVLM_E_INVALID, "svlm_uvprune_score: hidden-state pointers must be 16-byte aligned");
  if (!std::isfinite(out_scale) || !std::isfinite(out_offset))
    return fail(SVLM_E_INVALID, "svlm_uvprune_score: out_scale and out_offset must be finite");
  if (!grid_fits(n_text, kThreads, 2))
    return fail(SVLM_E_UNSUPPORTED, "svlm_uvprune_score: %d text tokens exceed the launch limit", n_text);
  const size_t need = svlm_uvprune_workspace(n_text, d);
  if (!ws || ws_bytes < need)
    return fail(SVLM_E_WORKSPACE, "svlm_uvprune_score: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return fail(SVLM_E_INVALID, "svlm_uvprune_score: workspace must be 16-byte aligned");
  UvArgs a;
  a.v0 = (const uint16_t*)v0;
  a.vL = (const uint16_t*)vL;
  a.v_sn = v_sn;
  a.n_vis = n_vis;
  a.x0 = (const uint16_t*)x0;
  a.xL = (const uint16_t*)xL;
  a.x_sn = x_sn;
  a.n_text = n_text;
  a.d = d;
  a.out_scale = out_scale;
  a.out_offset = out_offset;
  a.out = out;
  a.inv_x = (float*)ws;
  a.xbar = (float*)((char*)ws + ((size_t)2 * n_text * sizeof(float) + 255) / 256 * 256);
  hipStream_t st = (hipStream_t)stream;
  text_norms<<<dim3((unsigned)n_text, 2), kThreads, 0, st>>>(a);
  text_sums<<<dim3((unsigned)((d + 63) / 64), 2), kThreads, 0, st>>>(a);
  const int blocks = (int)std::min<int64_t>(((int64_t)n_vis + kThreads / 64 - 1) / (kThreads / 64), 1024);
  const size_t lds = (size_t)2 * d * sizeof(float);
  if (lds > 64 * 1024) {
    const hipError_t e =
        hipFuncSetAttribute((const void*)video_scores, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return fail(SVLM_E_HIP, "svlm_uvprune_score: %s", hipGetErrorString(e));
  }
  video_scores<<<blocks, kThreads, lds, st>>>(a);
  return check_launch("svlm_uvprune_score");
}
