// svlm_score: mean text-to-visual attention per visual token.
//
// SpecVLM technology-transfer listing, section 5 ("solution"): from the target
// model's attention matrix, the average attention the text tokens give each
// visual token.  Sparse-to-Dense explainer, "KV cache selection": the same
// signal at prefill, per layer and head.  The attention matrix itself is
// never stored (a block-wise attention kernel cannot expose it; two passes
// can):
//   pass 1: per (q head, text row) log-sum-exp over the causal key range,
//           split over key ranges; partial (max, sum) per split;
//   pass 2: per (q head, visual key range) recompute QK^T, form
//           P = exp2(c*s - lse2) and sum it over the text rows;
//   agg:    mean over heads as requested, out = alpha*agg + beta*out.
// Both passes use v_mfma_f32_16x16x32_bf16 with fp32 accumulation.  Pass 1
// computes S^T (lane = one text row x 4 keys), so row statistics stay in the
// lane; pass 2 computes S (lane = 4 rows x one key), so column sums need
// only two cross-lane steps.  The workgroups of the G q heads that share a KV
// head and key range are placed on one XCD so the K tile is read from HBM
// once and served from that XCD's L2 to the others.
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr float kNegInf = -INFINITY;

struct ScoreArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  const uint16_t* k;
  int64_t k_sh, k_sn;
  int T, n_ctx, q_pos0, vis_start, n_vis, Hq, Hkv, G;
  float c;  // scale * log2(e), > 0
  int S1, kps1, S2, kps2;
  int remap1, remap2;
  float* ml;    // [Hq][T][S1][2] raw (max, sum)
  float* head;  // [Hq][n_vis]
  int agg;
  float alpha, beta;
  float* out;
};

// block id -> (q head, split); with remap the G q heads of a (split, KV head)
// group share id % 8, i.e. one XCD
__device__ __forceinline__ void decode_block(int id, int S, int Hkv, int G, int remap, int& h, int& s) {
  if (remap) {
    const int x = id & 7, slot = id >> 3;
    const int hl = slot % G;
    const int q = (slot / G) * 8 + x;  // group = s * Hkv + g
    s = q / Hkv;
    h = (q % Hkv) * G + hl;
  } else {
    h = id % (Hkv * G);
    s = id / (Hkv * G);
  }
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2, float c) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;
  const float a1 = (m == kNegInf) ? 0.f : l * exp2f((m - M) * c);
  const float a2 = (m2 == kNegInf) ? 0.f : l2 * exp2f((m2 - M) * c);
  m = M;
  l = a1 + a2;
}

template <int D, int RB>
__device__ __forceinline__ void load_q(const ScoreArgs& a, int h, bf16x8 (&qop)[RB][D / 32]) {
  const int lane = threadIdx.x & 63, c = lane & 15, g4 = lane >> 4;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = rb * 16 + c;
    if (t < a.T) {
      const uint16_t* qr = a.q + (int64_t)t * a.q_st + (int64_t)h * a.q_sh + g4 * 8;
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qop[rb][kk] = as_bf16x8(*(const u32x4*)(qr + kk * 32));
    } else {
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) qop[rb][kk] = bf16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }
}

// K operand of a 16-key block: lane holds K[key t0 + c][32 kk + 8 g4 .. +8]
template <int D>
__device__ __forceinline__ void load_k(const uint16_t* kb, int64_t k_sn, int key, u32x4 (&kop)[D / 32]) {
  const int g4 = (threadIdx.x & 63) >> 4;
  const uint16_t* kr = kb + (int64_t)key * k_sn + g4 * 8;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) kop[kk] = *(const u32x4*)(kr + kk * 32);
}

template <int D, int RB, int NW>
__global__ __launch_bounds__(64 * NW, (RB >= 8 ? 1 : 2)) void score_pass1(ScoreArgs a) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g4 = lane >> 4;
  int h, s;
  decode_block(blockIdx.x, a.S1, a.Hkv, a.G, a.remap1, h, s);
  const int g = h / a.G;
  bf16x8 qop[RB][KK];
  load_q<D, RB>(a, h, qop);
  int lim[RB];  // keys < lim visible to the lane's row
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = rb * 16 + c;
    lim[rb] = (t < a.T) ? a.q_pos0 + t + 1 : 0;
  }
  const int k_begin = s * a.kps1;
  const int k_end = min(k_begin + a.kps1, a.q_pos0 + a.T);
  const int all_vis_end = min(k_end, a.q_pos0 + 1);  // keys every text row sees
  const uint16_t* kb = a.k + (int64_t)g * a.k_sh;
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
  }

  auto step = [&](const u32x4 (&k0)[KK], const u32x4 (&k1)[KK], int t0) {
    f32x4 sacc[2][RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        x0 = mfma16(as_bf16x8(k0[kk]), qop[rb][kk], x0);
        x1 = mfma16(as_bf16x8(k1[kk]), qop[rb][kk], x1);
      }
      sacc[0][rb] = x0;
      sacc[1][rb] = x1;
    }
    const bool masked = (t0 + 32 > all_vis_end);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float raw[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        raw[e] = sacc[e >> 2][rb][e & 3];
        if (masked) {
          const int key = t0 + 16 * (e >> 2) + 4 * g4 + (e & 3);
          if (key >= lim[rb] || key >= k_end) raw[e] = kNegInf;
        }
      }
      float lmax = raw[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) lmax = fmaxf(lmax, raw[e]);
      const float m_new = fmaxf(m[rb], lmax);
      const float mc = (m_new == kNegInf) ? 0.f : m_new * a.c;
      const float alpha = fast_exp2(m[rb] * a.c - mc);
      float sum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += fast_exp2(fmaf(raw[e], a.c, -mc));
      l[rb] = l[rb] * alpha + sum;
      m[rb] = m_new;
    }
  };

  {
    const int stride = 32 * NW;
    int t0 = k_begin + 32 * wave;
    u32x4 a0[KK], a1[KK], b0[KK], b1[KK];
    if (t0 < k_end) {
      load_k<D>(kb, a.k_sn, min(t0 + c, k_end - 1), a0);
      load_k<D>(kb, a.k_sn, min(t0 + 16 + c, k_end - 1), a1);
    }
    while (t0 < k_end) {
      int tn = t0 + stride;
      if (tn < k_end) {
        load_k<D>(kb, a.k_sn, min(tn + c, k_end - 1), b0);
        load_k<D>(kb, a.k_sn, min(tn + 16 + c, k_end - 1), b1);
      }
      step(a0, a1, t0);
      t0 = tn;
      if (t0 >= k_end) break;
      tn = t0 + stride;
      if (tn < k_end) {
        load_k<D>(kb, a.k_sn, min(tn + c, k_end - 1), a0);
        load_k<D>(kb, a.k_sn, min(tn + 16 + c, k_end - 1), a1);
      }
      step(b0, b1, t0);
      t0 = tn;
    }
  }

  // merge the four lane groups, then the waves (fixed order)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    merge_ml(m[rb], l[rb], __shfl_xor(m[rb], 16), __shfl_xor(l[rb], 16), a.c);
    merge_ml(m[rb], l[rb], __shfl_xor(m[rb], 32), __shfl_xor(l[rb], 32), a.c);
  }
  __shared__ float sm[NW][RB * 16][2];
  if (g4 == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      sm[wave][rb * 16 + c][0] = m[rb];
      sm[wave][rb * 16 + c][1] = l[rb];
    }
  }
  __syncthreads();
  for (int t = threadIdx.x; t < a.T; t += 64 * NW) {
    float M = sm[0][t][0], L = sm[0][t][1];
    for (int w = 1; w < NW; ++w) merge_ml(M, L, sm[w][t][0], sm[w][t][1], a.c);
    *(float2*)(a.ml + (((int64_t)h * a.T + t) * a.S1 + s) * 2) = make_float2(M, L);
  }
}

template <int D, int RB, int NW>
__global__ __launch_bounds__(64 * NW, (RB >= 8 ? 1 : 2)) void score_pass2(ScoreArgs a) {
  constexpr int KK = D / 32;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane & 15, g4 = lane >> 4;
  int h, s;
  decode_block(blockIdx.x, a.S2, a.Hkv, a.G, a.remap2, h, s);
  const int g = h / a.G;

  // row log-sum-exp (log2 units, scaled) from the pass-1 partials, in split order
  __shared__ float sm_lse[RB * 16];
  for (int t = threadIdx.x; t < RB * 16; t += 64 * NW) {
    float v = INFINITY;  // padded rows contribute exp2(-inf) = 0
    if (t < a.T) {
      const float* p = a.ml + ((int64_t)h * a.T + t) * a.S1 * 2;
      float M = p[0], L = p[1];
      for (int sp = 1; sp < a.S1; ++sp) merge_ml(M, L, p[2 * sp], p[2 * sp + 1], a.c);
      v = M * a.c + log2f(L);
    }
    sm_lse[t] = v;
  }
  bf16x8 qop[RB][KK];
  load_q<D, RB>(a, h, qop);
  __syncthreads();
  float lse[RB][4];  // rows 16 rb + 4 g4 + ii
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) lse[rb][ii] = sm_lse[rb * 16 + 4 * g4 + ii];

  const float invT = 1.f / (float)a.T;
  const int v_begin = a.vis_start + s * a.kps2;
  const int v_end = min(v_begin + a.kps2, a.vis_start + a.n_vis);
  const uint16_t* kb = a.k + (int64_t)g * a.k_sh;
  float* hrow = a.head + (int64_t)h * a.n_vis - a.vis_start;

  auto step = [&](const u32x4 (&k0)[KK], const u32x4 (&k1)[KK], int t0) {
    float col0 = 0.f, col1 = 0.f;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        x0 = mfma16(qop[rb][kk], as_bf16x8(k0[kk]), x0);
        x1 = mfma16(qop[rb][kk], as_bf16x8(k1[kk]), x1);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        col0 += fast_exp2(fmaf(x0[ii], a.c, -lse[rb][ii]));
        col1 += fast_exp2(fmaf(x1[ii], a.c, -lse[rb][ii]));
      }
    }
    col0 += __shfl_xor(col0, 16);
    col1 += __shfl_xor(col1, 16);
    col0 += __shfl_xor(col0, 32);
    col1 += __shfl_xor(col1, 32);
    if (g4 == 0) {
      if (t0 + c < v_end) hrow[t0 + c] = col0 * invT;
      if (t0 + 16 + c < v_end) hrow[t0 + 16 + c] = col1 * invT;
    }
  };

  {
    const int stride = 32 * NW;
    int t0 = v_begin + 32 * wave;
    u32x4 a0[KK], a1[KK], b0[KK], b1[KK];
    if (t0 < v_end) {
      load_k<D>(kb, a.k_sn, min(t0 + c, v_end - 1), a0);
      load_k<D>(kb, a.k_sn, min(t0 + 16 + c, v_end - 1), a1);
    }
    while (t0 < v_end) {
      int tn = t0 + stride;
      if (tn < v_end) {
        load_k<D>(kb, a.k_sn, min(tn + c, v_end - 1), b0);
        load_k<D>(kb, a.k_sn, min(tn + 16 + c, v_end - 1), b1);
      }
      step(a0, a1, t0);
      t0 = tn;
      if (t0 >= v_end) break;
      tn = t0 + stride;
      if (tn < v_end) {
        load_k<D>(kb, a.k_sn, min(tn + c, v_end - 1), a0);
        load_k<D>(kb, a.k_sn, min(tn + 16 + c, v_end - 1), a1);
      }
      step(b0, b1, t0);
      t0 = tn;
    }
  }
}

__global__ __launch_bounds__(256) void score_agg(ScoreArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  if (i >= a.n_vis) return;
  int h0, nh;
  if (a.agg == SVLM_AGG_QHEAD) { h0 = r; nh = 1; }
  else if (a.agg == SVLM_AGG_KVHEAD) { h0 = r * a.G; nh = a.G; }
  else { h0 = 0; nh = a.Hq; }
  float acc = 0.f;
  for (int hh = 0; hh < nh; ++hh) acc += a.head[(int64_t)(h0 + hh) * a.n_vis + i];
  const float v = acc / (float)nh;
  float* o = a.out + (int64_t)r * a.n_vis + i;
  *o = (a.beta == 0.f) ? a.alpha * v : a.alpha * v + a.beta * (*o);
}

template <int D, int RB>
void launch_passes(const ScoreArgs& a, hipStream_t st) {
  constexpr int NW = 4;
  score_pass1<D, RB, NW><<<a.Hq * a.S1, 64 * NW, 0, st>>>(a);
  score_pass2<D, RB, NW><<<a.Hq * a.S2, 64 * NW, 0, st>>>(a);
}

template <int D>
void launch_d(const ScoreArgs& a, int rb, hipStream_t st) {
  switch (rb) {
    case 1: launch_passes<D, 1>(a, st); break;
    case 2: launch_passes<D, 2>(a, st); break;
    case 4: launch_passes<D, 4>(a, st); break;
    case 6: launch_passes<D, 6>(a, st); break;
    default: launch_passes<D, 8>(a, st); break;
  }
}

int pick_rb(int T) {
  if (T <= 16) return 1;
  if (T <= 32) return 2;
  if (T <= 64) return 4;
  if (T <= 96) return 6;
  return 8;
}

// splits so that Hq * S is about 2 workgroups per CU, each with >= 8 key blocks per wave
int pick_splits(int Hq, int Hkv, int keys, int* kps, int* remap) {
  const int target = 2 * num_cus();
  int S = std::max(1, (target + Hq - 1) / Hq);
  const int max_s = std::max(1, keys / (4 * 32 * 2));
  S = std::min(S, max_s);
  // make the (split, KV head) group count a multiple of 8 for the XCD placement
  while ((S * Hkv) % 8 != 0 && S < 8 * max_s) ++S;
  int per = (keys + S - 1) / S;
  per = (per + 31) / 32 * 32;
  S = (keys + per - 1) / per;
  *kps = per;
  *remap = ((S * Hkv) % 8 == 0) ? 1 : 0;
  return S;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" size_t svlm_score_workspace(int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  if (T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || q_pos0 < 0 || n_vis < 1) return 0;
  int kps, remap;
  const int S1 = pick_splits(Hq, Hkv, q_pos0 + T, &kps, &remap);
  return (size_t)Hq * T * S1 * 2 * sizeof(float) + (size_t)Hq * n_vis * sizeof(float);
}

extern "C" int svlm_score(const void* q_text, int64_t q_st, int64_t q_sh, const void* k, int64_t k_sh, int64_t k_sn,
                          int dtype, int T, int n_ctx, int q_pos0, int vis_start, int n_vis, int Hq, int Hkv, int D,
                          float scale, int agg, float alpha, float beta, float* out, void* ws, size_t ws_bytes,
                          void* stream) {
  if (dtype != SVLM_BF16) return fail(SVLM_E_UNSUPPORTED, "svlm_score: only SVLM_BF16 operands are supported");
  if (D != 64 && D != 128) return fail(SVLM_E_UNSUPPORTED, "svlm_score: D must be 64 or 128 (got %d)", D);
  if (T < 1 || T > 128) return fail(SVLM_E_UNSUPPORTED, "svlm_score: 1 <= T <= 128 text queries supported (got %d)", T);
  if (!q_text || !k || !out) return fail(SVLM_E_INVALID, "svlm_score: null pointer");
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(SVLM_E_INVALID, "svlm_score: Hq must be a positive multiple of Hkv");
  if (n_ctx < 1 || q_pos0 < 0 || (int64_t)q_pos0 + T > n_ctx)
    return fail(SVLM_E_INVALID, "svlm_score: need 0 <= q_pos0 and q_pos0 + T <= n_ctx");
  if (n_vis < 1 || n_vis > (1 << 18) || vis_start < 0 || (int64_t)vis_start + n_vis > (int64_t)q_pos0 + 1)
    return fail(SVLM_E_INVALID, "svlm_score: visual range must lie in [0, q_pos0] (every text query sees it)");
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVLM_E_INVALID, "svlm_score: scale must be finite and > 0");
  if (agg != SVLM_AGG_QHEAD && agg != SVLM_AGG_KVHEAD && agg != SVLM_AGG_ALL)
    return fail(SVLM_E_INVALID, "svlm_score: unknown aggregation %d", agg);
  if (!std::isfinite(alpha) || !std::isfinite(beta)) return fail(SVLM_E_INVALID, "svlm_score: alpha, beta must be finite");
  if (!aligned16(q_text) || !aligned16(k)) return fail(SVLM_E_INVALID, "svlm_score: q_text and k must be 16-byte aligned");
  if (q_st % 8 || q_sh % 8 || k_sh % 8 || k_sn % 8 || k_sn < D || q_st < 0 || q_sh < 0 || k_sh < 0)
    return fail(SVLM_E_INVALID, "svlm_score: strides must be non-negative multiples of 8 elements, k_sn >= D");
  ScoreArgs a;
  a.q = (const uint16_t*)q_text;
  a.q_st = q_st;
  a.q_sh = q_sh;
  a.k = (const uint16_t*)k;
  a.k_sh = k_sh;
  a.k_sn = k_sn;
  a.T = T;
  a.n_ctx = n_ctx;
  a.q_pos0 = q_pos0;
  a.vis_start = vis_start;
  a.n_vis = n_vis;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.c = scale * kLog2e;
  // pass 1 covers keys [0, q_pos0 + T): everything any text row sees
  a.S1 = pick_splits(Hq, Hkv, q_pos0 + T, &a.kps1, &a.remap1);
  a.S2 = pick_splits(Hq, Hkv, n_vis, &a.kps2, &a.remap2);
  if (a.S1 > 1024) return fail(SVLM_E_UNSUPPORTED, "svlm_score: too many key splits");
  const size_t ml_bytes = (size_t)Hq * T * a.S1 * 2 * sizeof(float);
  const size_t need = svlm_score_workspace(T, Hq, Hkv, q_pos0, n_vis);
  if (!ws || ws_bytes < need)
    return fail(SVLM_E_WORKSPACE, "svlm_score: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return fail(SVLM_E_INVALID, "svlm_score: workspace must be 16-byte aligned");
  a.ml = (float*)ws;
  a.head = (float*)((char*)ws + ml_bytes);
  a.agg = agg;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  hipStream_t st = (hipStream_t)stream;
  const int rb = pick_rb(T);
  if (D == 128) launch_d<128>(a, rb, st);
  else launch_d<64>(a, rb, st);
  const int rows = (agg == SVLM_AGG_QHEAD) ? Hq : (agg == SVLM_AGG_KVHEAD ? Hkv : 1);
  score_agg<<<dim3((unsigned)((n_vis + 255) / 256), (unsigned)rows), 256, 0, st>>>(a);
  return check_launch("svlm_score");
}
