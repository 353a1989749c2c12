// fp32 operands (SVLM_F32) for svlm_score, svlm_decode_attn and
// svlm_decode_attn_indexed: the tiny reference configuration keeps its q, k
// and v in fp32, and these kernels take them as given (no rounding to bf16).
//
// Plain vector-ALU fp32 arithmetic with natural-base exp/log, no matrix cores:
// the operations are the same as the bf16 kernels' (SpecVLM listing,
// section 5, for the mean text-to-visual attention; Sparse-to-Dense
// explainer, "decoding process", for draft and verify attention), written for
// clarity at small sizes.  The bf16 kernels are the tuned path.
//
//  * attention: one wave per output row (batch, query, q head).  Lanes take
//    64 keys at a time (one key each, the whole dot product), the wave keeps
//    an online (max, sum), and the weights go through LDS to the lanes that
//    own the output columns (D / 64 each).
//  * score pass 1: one wave per (q head, text query) forms the row's
//    log-sum-exp over its causal keys.
//  * score pass 2: one thread per (output row, visual token) sums the
//    normalised weights over the text queries and the row's q heads, then
//    applies out = alpha * mean + beta * out.
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

__device__ __forceinline__ float wave_max_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_sum_f(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

template <int D>
__global__ __launch_bounds__(64) void attn_f32_rows(AttnF32Args a) {
  constexpr int PER = D / 64;  // output columns per lane
  __shared__ float qs[D];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // ((b * nq) + i) * Hq + h
  const int h = row % a.Hq;
  const int i = (row / a.Hq) % a.nq;
  const int b = row / (a.Hq * a.nq);
  const int g = h / (a.Hq / a.Hkv);
  const int n_raw = a.kv_len[(int64_t)b * a.len_sb + (int64_t)g * a.len_sh];
  if (threadIdx.x == 0) debug_check(n_raw >= a.nq && n_raw <= a.max_kv_len, SVLM_DBG_KV_LEN);
  const int n_kv = min(max(n_raw, 0), a.max_kv_len);
  const int lim = a.causal ? n_kv - a.nq + i + 1 : n_kv;
  const float* qrow = a.q + (int64_t)b * a.q_sb + ((int64_t)i * a.Hq + h) * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) qs[lane + 64 * e] = qrow[lane + 64 * e];
  __syncthreads();
  const float* kb = a.k + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const float* vb = a.v + (int64_t)b * a.kv_sb + (int64_t)g * a.kv_sh;
  const int32_t* idx = a.kv_idx ? a.kv_idx + (int64_t)b * a.idx_sb + (int64_t)g * a.idx_sh : nullptr;
  // cache row of key position p, or -1 for an index outside the cache (a zero row)
  auto key_row = [&](int p) -> int {
    if (!idx) return p;
    const int r = idx[p];
    debug_check(r >= 0 && r < a.kv_rows, SVLM_DBG_KV_INDEX);
    return (r >= 0 && r < a.kv_rows) ? r : -1;
  };
  float m = -INFINITY, l = 0.f;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int base = 0; base < lim; base += 64) {
    const int p = base + lane;
    float s = -INFINITY;
    if (p < lim) {
      const int r = key_row(p);
      float dot = 0.f;
      if (r >= 0) {
        const float* kr = kb + (int64_t)r * a.kv_sn;
        for (int d = 0; d < D; ++d) dot = fmaf(qs[d], kr[d], dot);
      }
      s = dot * a.scale;
    }
    const float m_new = fmaxf(m, wave_max_f(s));
    const float alpha = (m == -INFINITY) ? 0.f : expf(m - m_new);
    const float w = (p < lim) ? expf(s - m_new) : 0.f;
    l = l * alpha + wave_sum_f(w);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] *= alpha;
    m = m_new;
    ps[lane] = w;
    __syncthreads();
    const int cnt = min(64, lim - base);
    for (int j = 0; j < cnt; ++j) {
      const int r = key_row(base + j);
      if (r < 0) continue;
      const float* vr = vb + (int64_t)r * a.kv_sn;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] = fmaf(ps[j], vr[lane + 64 * e], acc[e]);
    }
    __syncthreads();
  }
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
  float* orow = a.out + (int64_t)row * D;
#pragma unroll
  for (int e = 0; e < PER; ++e) orow[lane + 64 * e] = acc[e] * inv;
  if (a.lse && lane == 0) a.lse[row] = (l > 0.f) ? m + logf(l) : -INFINITY;
}

// pass 1: lse[h][t] over keys 0 .. q_pos0 + t
template <int D>
__global__ __launch_bounds__(64) void score_f32_lse(ScoreF32Args a) {
  const int lane = threadIdx.x;
  const int h = blockIdx.x / a.T;
  const int t = blockIdx.x % a.T;
  const int g = h / (a.Hq / a.Hkv);
  const float* qrow = a.q + (int64_t)t * a.q_st + (int64_t)h * a.q_sh;
  const float* kb = a.k + (int64_t)g * a.k_sh;
  const int lim = a.q_pos0 + t + 1;
  float m = -INFINITY, l = 0.f;
  for (int n = lane; n < lim; n += 64) {
    const float* kr = kb + (int64_t)n * a.k_sn;
    float dot = 0.f;
    for (int d = 0; d < D; ++d) dot = fmaf(qrow[d], kr[d], dot);
    const float s = dot * a.scale;
    const float m_new = fmaxf(m, s);
    l = l * ((m == -INFINITY) ? 0.f : expf(m - m_new)) + expf(s - m_new);
    m = m_new;
  }
  const float M = wave_max_f(m);
  const float L = wave_sum_f((m == -INFINITY) ? 0.f : l * expf(m - M));
  if (lane == 0) a.lse[(int64_t)h * a.T + t] = M + logf(L);
}

// pass 2: out[r][i] = alpha * (mean over the row's q heads and the text
// queries of the weight on visual key vis_start + i) + beta * out[r][i]
template <int D>
__global__ __launch_bounds__(256) void score_f32_cols(ScoreF32Args a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  if (i >= a.n_vis) return;
  const int G = a.Hq / a.Hkv;
  int h0, nh;
  if (a.agg == SVLM_AGG_QHEAD) { h0 = r; nh = 1; }
  else if (a.agg == SVLM_AGG_KVHEAD) { h0 = r * G; nh = G; }
  else { h0 = 0; nh = a.Hq; }
  float acc = 0.f;
  for (int h = h0; h < h0 + nh; ++h) {
    const float* kr = a.k + (int64_t)(h / G) * a.k_sh + (int64_t)(a.vis_start + i) * a.k_sn;
    float hs = 0.f;
    for (int t = 0; t < a.T; ++t) {
      const float* qrow = a.q + (int64_t)t * a.q_st + (int64_t)h * a.q_sh;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot = fmaf(qrow[d], kr[d], dot);
      hs += expf(dot * a.scale - a.lse[(int64_t)h * a.T + t]);
    }
    acc += hs / (float)a.T;
  }
  const float v = acc / (float)nh;
  float* o = a.out + (int64_t)r * a.n_vis + i;
  *o = (a.beta == 0.f) ? a.alpha * v : a.alpha * v + a.beta * (*o);
}

}  // namespace

void launch_attn_f32(const AttnF32Args& a, hipStream_t st) {
  const unsigned rows = (unsigned)((int64_t)a.batch * a.nq * a.Hq);
  if (a.D == 128) attn_f32_rows<128><<<rows, 64, 0, st>>>(a);
  else attn_f32_rows<64><<<rows, 64, 0, st>>>(a);
}

void launch_score_f32(const ScoreF32Args& a, int rows, hipStream_t st) {
  const dim3 cols((unsigned)((a.n_vis + 255) / 256), (unsigned)rows);
  if (a.D == 128) {
    score_f32_lse<128><<<(unsigned)((int64_t)a.Hq * a.T), 64, 0, st>>>(a);
    score_f32_cols<128><<<cols, 256, 0, st>>>(a);
  } else {
    score_f32_lse<64><<<(unsigned)((int64_t)a.Hq * a.T), 64, 0, st>>>(a);
    score_f32_cols<64><<<cols, 256, 0, st>>>(a);
  }
}

}  // namespace svlm

#ifdef SVLM_DEBUG
bool svlm::debug_take_f32_path(unsigned* out) { return debug_take_here(out); }
#endif
