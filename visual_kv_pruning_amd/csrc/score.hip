// svlm_score: mean text-to-visual attention per visual token.
//
// SpecVLM technology-transfer listing, section 5 ("solution"): from the target
// model's attention matrix, the average attention the text tokens give each
// visual token.  Sparse-to-Dense explainer, "KV cache selection": the same
// signal at prefill, per layer and head.  The attention matrix itself is
// never stored (a block-wise attention kernel cannot expose it; two passes
// can):
//   pass 1: per (q head, text row) log-sum-exp over the causal key range,
//           split over key ranges; partial (reference max, sum) per split;
//   pass 2: per (q head, visual key range) recompute QK^T, form
//           P = exp2(c*s - lse2) and sum it over the text rows;
//   agg:    mean over heads as requested, out = alpha*agg + beta*out.
//
// A workgroup owns one KV head and one key range, with one wave per q head of
// the KV group (up to 8).  The key tile (64 keys) is staged HBM -> LDS once by
// LDS-DMA transfers that all waves share (one barrier per tile), so K is read
// from memory once per workgroup; the text queries of a wave's head sit in
// registers.  Both passes use v_mfma_f32_16x16x32_bf16 with fp32 accumulation:
// pass 1 computes S^T (lane = one text row x 4 keys per 16-key block) and keeps
// a lazily raised reference maximum per lane group, so a key costs one fma,
// one exp2 and one add; pass 2 computes S (lane = 4 text rows x one key), so a
// column sum over the rows needs two cross-lane steps per tile, and the waves
// add their heads through LDS.  Exp throughput bounds both passes.
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr float kNegInf = -INFINITY;
constexpr int kTileKeys = 64;      // keys per staged K tile
constexpr float kRescaleSum = 256.f;  // a lane's 4-key weight sum above this raises its reference maximum
constexpr int kLseBatch = 16;      // pass-1 partials loaded at once when a row's log-sum-exp is formed

struct ScoreArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  const uint16_t* k;
  int64_t k_sh, k_sn;
  int T, n_ctx, q_pos0, vis_start, n_vis, Hq, Hkv, G;
  int HG1, HG2;  // head groups (workgroups) per KV head, pass 1 and pass 2
  float c;  // scale * log2(e), > 0
  int S1, kps1, S2, kps2;
  float* ml;   // [Hq][T][S1][2]: per split, (reference maximum in raw-score units, sum)
  float* grp;  // [Hkv * HG][n_vis]: per head group, the sum over its heads of the column means
  int agg;
  float alpha, beta;
  float* out;
};

// block id -> (KV head g, head group hg, key split s).  Workgroups are handed
// to the eight XCDs round-robin by id, so the HG head groups of one (KV head,
// split) take ids 8 apart: they run on one XCD, and the K tiles one of them
// fetches reach the others from that XCD's L2.  Ids past the last (g, s) pair
// of a partial group of eight are idle.
__device__ __forceinline__ bool decode_block(int S, int Hkv, int HG, int& g, int& hg, int& s) {
  const int bid = blockIdx.x;
  const int rest = bid >> 3;
  hg = rest % HG;
  const int pair = (rest / HG) * 8 + (bid & 7);
  if (pair >= Hkv * S) return false;
  s = pair % S;
  g = pair / S;
  return true;
}

__device__ __forceinline__ void merge_ml(float& m, float& l, float m2, float l2, float c) {
  const float M = fmaxf(m, m2);
  if (M == kNegInf) return;
  const float a1 = (m == kNegInf) ? 0.f : l * fast_exp2((m - M) * c);
  const float a2 = (m2 == kNegInf) ? 0.f : l2 * fast_exp2((m2 - M) * c);
  m = M;
  l = a1 + a2;
}

// Ring depth of the shared K tiles: a wave issues PW transfers per tile and
// at most NS - 1 tiles are outstanding (6-bit wait counter); LDS holds NS tiles.
template <int D, int W>
constexpr int score_ring_depth() {
  constexpr int TB = kTileKeys * D * 2;
  constexpr int PW = (TB / 1024) / W;
  int ns = 2;
  while (ns < 8 && ns * PW <= 63 && (size_t)(ns + 1) * TB <= 128 * 1024) ++ns;
  return ns;
}

// Staging of the K tiles of one (KV head, key range) through a ring of NS
// slots in LDS: every wave issues its share (PW transfers of 1 KB) of each
// tile; rows are XOR-swizzled by 16-byte chunk (chunk p of row r holds source
// chunk p ^ (r % CH)).  Tiles past the range deliver zeros.
template <int D, int W, int NS>
struct KRing {
  static constexpr int ROWB = D * 2, CH = ROWB / 16;
  static constexpr int TB = kTileKeys * ROWB;
  static constexpr int NI = TB / 1024;
  static constexpr int PW = NI / W;
  static_assert(PW >= 1 && NI % W == 0, "tile transfers must split evenly over the waves");
  static_assert((NS - 1) * PW <= 63, "ring depth");
  static constexpr int kMaxPW = 16;  // one wave staging a whole D = 128 tile
  static_assert(PW <= kMaxPW, "transfers per wave");
  __amdgpu_buffer_rsrc_t rs;
  unsigned char* lds;
  int wave, row_bytes;
  // per-lane source offset of each of this wave's PW transfers (set by init;
  // a fixed bound: sized by PW, the host pass of this compiler dropped the
  // kernels' launch stubs)
  int src_lane[kMaxPW];

  __device__ void init(const uint16_t* k_rows, int n_rows, int64_t k_sn, unsigned char* ring, int w) {
    const int lane = threadIdx.x & 63;
    row_bytes = (int)(k_sn * 2);
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)k_rows, (short)0, n_rows * row_bytes, kBufferFlags);
    lds = ring;
    wave = w;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int r = (wave * PW + i) * (1024 / ROWB) + lane / CH;
      const int p = lane % CH;
      src_lane[i] = r * row_bytes + ((p ^ (r % CH)) * 16);
    }
  }
  __device__ void stage(int slot, int tile) const {
    const int soff = tile * kTileKeys * row_bytes;
#pragma unroll
    for (int i = 0; i < PW; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(lds + slot * TB + (wave * PW + i) * 1024), 16, src_lane[i],
          soff, 0, kNT);
  }
  // LDS byte offset (within a slot) of the lane's K operand chunk: key row r, d chunk kk*4 + g4
  static __device__ unsigned koff(int r, int kk, int g4) { return r * ROWB + (((kk * 4 + g4) ^ (r % CH)) * 16); }
};

// the KK K-operand chunks of one 16-key block of a staged tile
template <int KK>
__device__ __forceinline__ void read_k_block(unsigned base, const unsigned (&ko)[KK], u32x4 (&kq)[KK]) {
  unsigned ad[KK];
#pragma unroll
  for (int e = 0; e < KK; ++e) ad[e] = base + ko[e];
  if constexpr (KK == 4) lds_read_b128x4(kq, ad);
  else lds_read_b128x2(kq, ad);
}

// S = Q K^T for two 16-key blocks and every text row block (lane: rows
// 16 rb + 4 g4 + i, key c of each block)
template <int RB, int KK>
__device__ __forceinline__ void qk_half(const u32x4 (&q)[RB][KK], const u32x4 (&kq)[2][KK], f32x4 (&S)[RB][2]) {
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      s0 = mfma16(as_bf16x8(q[rb][kk]), as_bf16x8(kq[0][kk]), s0);
      s1 = mfma16(as_bf16x8(q[rb][kk]), as_bf16x8(kq[1][kk]), s1);
    }
    S[rb][0] = s0;
    S[rb][1] = s1;
  }
}

// the lane's part of the column sums of P = exp2(c s - lse) for the two key blocks
template <int RB>
__device__ __forceinline__ void colsum_half(const f32x4 (&S)[RB][2], const float (&lse)[RB][4], float c, float& c0,
                                            float& c1) {
  c0 = 0.f;
  c1 = 0.f;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c0 += fast_exp2(fmaf(S[rb][0][i], c, -lse[rb][i]));
      c1 += fast_exp2(fmaf(S[rb][1][i], c, -lse[rb][i]));
    }
}

// the lane's part of the column sum of P = exp2(c s - lse) for one 16-key
// block (lane: rows 16 rb + 4 g4 + i, key c).  One block at a time keeps the
// score accumulators few enough to live in ordinary VGPRs next to the query
// registers, so the exponentials read them without accumulator moves.
template <int RB, int KK>
__device__ __forceinline__ float qk_colsum_block(const u32x4 (&q)[RB][KK], const u32x4 (&kq)[KK],
                                                 const float (&lse)[RB][4], float c) {
  f32x4 S[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    S[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) S[rb] = mfma16(as_bf16x8(q[rb][kk]), as_bf16x8(kq[kk]), S[rb]);
  }
  // pairwise sums (a fixed tree, not one serial chain of RB * 4 dependent adds)
  float r[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float e[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) e[i] = fast_exp2(fmaf(S[rb][i], c, -lse[rb][i]));
    r[rb] = (e[0] + e[1]) + (e[2] + e[3]);
  }
#pragma unroll
  for (int w = 1; w < RB; w *= 2)
#pragma unroll
    for (int rb = 0; rb + w < RB; rb += 2 * w) r[rb] += r[rb + w];
  return r[0];
}

// the 2 * KK K-operand chunks of key blocks kb0, kb0 + 1 of a staged tile
template <int KK, int BLOCK_BYTES>
__device__ __forceinline__ void read_k_pair(unsigned base, const unsigned (&ko)[KK], u32x4 (&kq)[2][KK]) {
  if constexpr (KK == 4) {
    unsigned ad[8];
    u32x4 d[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ad[e] = base + ko[e % 4] + (e / 4) * BLOCK_BYTES;
    lds_read_b128x8(d, ad);
#pragma unroll
    for (int e = 0; e < 8; ++e) kq[e / 4][e % 4] = d[e];
  } else {
    unsigned ad[4];
    u32x4 d[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ad[e] = base + ko[e % 2] + (e / 2) * BLOCK_BYTES;
    lds_read_b128x4(d, ad);
#pragma unroll
    for (int e = 0; e < 4; ++e) kq[e / 2][e % 2] = d[e];
  }
}

// this wave's head's text queries: lane (c, g4) holds row 16 rb + c, d = 32 kk + 8 g4 .. + 7
// (rows past T read zeros)
template <int D, int RB>
__device__ __forceinline__ void load_q(const ScoreArgs& a, int h, u32x4 (&q)[RB][D / 32]) {
  const int lane = threadIdx.x & 63, c = lane & 15, g4 = lane >> 4;
  const int bytes = (int)(((int64_t)(a.T - 1) * a.q_st + D) * 2);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + (int64_t)h * a.q_sh), (short)0, bytes, kBufferFlags);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int t = rb * 16 + c;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
      const int off = (t < a.T) ? (int)(((int64_t)t * a.q_st + 32 * kk + 8 * g4) * 2) : bytes;
      q[rb][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
    }
  }
}

template <int D, int RB, int W, int NS>
__global__ __launch_bounds__(64 * W, 1) void score_pass1(ScoreArgs a) {
  constexpr int KK = D / 32;
  using Ring = KRing<D, W, NS>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  int g, hg, s;
  if (!decode_block(a.S1, a.Hkv, a.HG1, g, hg, s)) return;
  const int hl = hg * W + wave;  // head within the KV group; waves past the group compute but do not write
  const int h = g * a.G + min(hl, a.G - 1);

  const int k_begin = s * a.kps1;
  const int k_end = min(k_begin + a.kps1, a.q_pos0 + a.T);
  const int n_tiles = (k_end > k_begin) ? (k_end - k_begin + kTileKeys - 1) / kTileKeys : 0;

  __shared__ __align__(16) unsigned char ring[NS * Ring::TB];
  Ring kr;
  kr.init(a.k + (int64_t)g * a.k_sh + (int64_t)k_begin * a.k_sn, max(k_end - k_begin, 0), a.k_sn, ring, wave);

  u32x4 qreg[RB][KK];
  load_q<D, RB>(a, h, qreg);
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) kr.stage(u, u);
  wait_vmcnt<(NS - 1) * Ring::PW>();  // the query loads, issued first, have landed

  // tiles below n_full are visible to every row and lie inside the range
  const int vis_all = min(k_end, a.q_pos0 + 1) - k_begin;
  const int n_full = min(n_tiles, vis_all > 0 ? vis_all / kTileKeys : 0);
  // LDS offsets of the lane's K chunks in key block 0 (block 1 is 16 rows on)
  unsigned ko[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) ko[kk] = Ring::koff(c, kk, g4);
  const unsigned ring0 = lds_addr(ring);

  // per lane group: reference maximum in log2 units of the scaled score, sum
  float mc[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    mc[rb] = kNegInf;
    l[rb] = 0.f;
  }

  auto tile = [&](int t, bool masked) {
    wait_vmcnt<(NS - 2) * Ring::PW>();  // this wave's share of tile t has landed
    wg_barrier();                       // every share of tile t has landed; tile t-1 is retired
    kr.stage((t + NS - 1) % NS, t + NS - 1);
    const unsigned base = ring0 + (unsigned)((t % NS) * Ring::TB);
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {  // one 16-key block at a time keeps the live registers low
      u32x4 kq[KK];
      read_k_block<KK>(base + (unsigned)(kb * 16 * Ring::ROWB), ko, kq);
      const int key0 = k_begin + t * kTileKeys + 16 * kb;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) s0 = mfma16(as_bf16x8(kq[kk]), as_bf16x8(qreg[rb][kk]), s0);
        float x[4];
        if (masked) {
          const int tq = rb * 16 + c;
          const int lim = min(k_end, (tq < a.T) ? a.q_pos0 + tq + 1 : 0);  // keys < lim visible to the row
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (key0 + 4 * g4 + e < lim) ? s0[e] : kNegInf;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = s0[e];
        }
        // weights against the current reference: the 4-key sum exceeds
        // kRescaleSum = 2^8 (or is inf / NaN: no reference yet) only when a
        // score passes the reference by about 8 (log2 units); the reference is
        // then raised to the block maximum and the weights recomputed.  The
        // maximum is taken only on that rare path, so the hot path is one
        // fma, one exp2 and one add per score.
        float p[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(x[e], a.c, -mc[rb]));
        float s4 = (p[0] + p[1]) + (p[2] + p[3]);
        if (!(s4 <= kRescaleSum)) {
          const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])) * a.c;
          const float m_new = fmaxf(mc[rb], lmax);
          l[rb] *= (mc[rb] == kNegInf) ? 0.f : fast_exp2(mc[rb] - m_new);
          mc[rb] = m_new;
          const float mneg = (m_new == kNegInf) ? 0.f : -m_new;
#pragma unroll
          for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(x[e], a.c, mneg));
          s4 = (p[0] + p[1]) + (p[2] + p[3]);
        }
        l[rb] += s4;
      }
    }
  };
  int t = 0;
  for (; t < n_full; ++t) tile(t, false);
  for (; t < n_tiles; ++t) tile(t, true);
  wait_vmcnt<0>();

  // merge the four lane groups (fixed order) and write this split's row state
  // (maximum back in raw-score units)
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    float m = (mc[rb] == kNegInf) ? kNegInf : mc[rb] / a.c, ll = l[rb];
    {
      const auto mr = __builtin_amdgcn_permlane16_swap(f_bits(m), f_bits(m), false, false);
      const auto lr = __builtin_amdgcn_permlane16_swap(f_bits(ll), f_bits(ll), false, false);
      float m0 = bits_f(mr[0]), l0 = bits_f(lr[0]);
      merge_ml(m0, l0, bits_f(mr[1]), bits_f(lr[1]), a.c);
      m = m0;
      ll = l0;
    }
    {
      const auto mr = __builtin_amdgcn_permlane32_swap(f_bits(m), f_bits(m), false, false);
      const auto lr = __builtin_amdgcn_permlane32_swap(f_bits(ll), f_bits(ll), false, false);
      float m0 = bits_f(mr[0]), l0 = bits_f(lr[0]);
      merge_ml(m0, l0, bits_f(mr[1]), bits_f(lr[1]), a.c);
      m = m0;
      ll = l0;
    }
    const int tq = rb * 16 + c;
    if (g4 == 0 && hl < a.G && tq < a.T)
      *(float2*)(a.ml + (((int64_t)h * a.T + tq) * a.S1 + s) * 2) = make_float2(m, ll);
  }
}

template <int D, int RB, int W, int NS>
__global__ __launch_bounds__(64 * W, 1) void score_pass2(ScoreArgs a) {
  constexpr int KK = D / 32;
  using Ring = KRing<D, W, NS>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  int g, hg, s;
  if (!decode_block(a.S2, a.Hkv, a.HG2, g, hg, s)) return;
  const int hl = hg * W + wave;
  const bool active = hl < a.G;
  const int h = g * a.G + min(hl, a.G - 1);

  const int v_begin = a.vis_start + s * a.kps2;
  const int v_end = min(v_begin + a.kps2, a.vis_start + a.n_vis);
  const int n_tiles = (v_end > v_begin) ? (v_end - v_begin + kTileKeys - 1) / kTileKeys : 0;

  __shared__ __align__(16) unsigned char ring[NS * Ring::TB];
  __shared__ float sm_lse[W][RB * 16];
  __shared__ float xch[2][W][kTileKeys];
  Ring kr;
  kr.init(a.k + (int64_t)g * a.k_sh + (int64_t)v_begin * a.k_sn, max(v_end - v_begin, 0), a.k_sn, ring, wave);

  u32x4 qreg[RB][KK];
  load_q<D, RB>(a, h, qreg);
#pragma unroll
  for (int u = 0; u < NS - 1; ++u) kr.stage(u, u);

  // row log-sum-exp (log2 units of the scaled score) from the pass-1 partials,
  // in split order; padded rows get +inf and so contribute exp2(-inf) = 0
  // (the partials are loaded kLseBatch splits at a time, so a row costs
  // ceil(S1 / kLseBatch) memory round trips rather than S1)
  for (int tq = lane; tq < RB * 16; tq += 64) {
    float v = INFINITY;
    if (tq < a.T) {
      const float2* p = (const float2*)(a.ml + ((int64_t)h * a.T + tq) * a.S1 * 2);
      float M = kNegInf, L = 0.f;
      for (int s0 = 0; s0 < a.S1; s0 += kLseBatch) {
        float2 part[kLseBatch];
#pragma unroll
        for (int j = 0; j < kLseBatch; ++j) part[j] = (s0 + j < a.S1) ? p[s0 + j] : make_float2(kNegInf, 0.f);
#pragma unroll
        for (int j = 0; j < kLseBatch; ++j) merge_ml(M, L, part[j].x, part[j].y, a.c);
      }
      v = (L > 0.f) ? M * a.c + log2f(L) : INFINITY;
    }
    sm_lse[wave][tq] = v;
  }
  wait_lgkmcnt0();
  float lse[RB][4];  // rows 16 rb + 4 g4 + i
#pragma unroll
  for (int rb = 0; rb < RB; ++rb)
#pragma unroll
    for (int i = 0; i < 4; ++i) lse[rb][i] = sm_lse[wave][rb * 16 + 4 * g4 + i];

  unsigned ko[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) ko[kk] = Ring::koff(c, kk, g4);
  const unsigned ring0 = lds_addr(ring);
  const float invT = 1.f / (float)a.T;
  const bool direct = (a.agg == SVLM_AGG_QHEAD) || (a.agg == SVLM_AGG_KVHEAD && a.HG2 == 1);
  // the KV-head mean is taken here when one workgroup holds the whole group, else by score_agg
  const float grp_scale = (direct && a.agg == SVLM_AGG_KVHEAD) ? 1.f / (float)a.G : 1.f;

  // writes one output element: the head row (q-head aggregation), the KV-head row
  // when one workgroup holds the whole group, else the group sum for the final mean
  auto emit = [&](int row, int key, float v) {
    const int i = key - a.vis_start;
    if (direct) {
      float* o = a.out + (int64_t)row * a.n_vis + i;
      *o = (a.beta == 0.f) ? a.alpha * v : a.alpha * v + a.beta * (*o);
    } else {
      a.grp[(int64_t)row * a.n_vis + i] = v;
    }
  };
  // wave 0 adds the waves' column means of tile tt (published in xch[tt % 2])
  auto flush = [&](int tt) {
    if (wave != 0) return;
    const int key = v_begin + tt * kTileKeys + lane;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += xch[tt & 1][w][lane];
    if (key < v_end) emit(direct ? g : g * a.HG2 + hg, key, v * grp_scale);
  };

  wait_vmcnt<(NS - 1) * Ring::PW>();  // the query loads, issued first, have landed
  for (int t = 0; t < n_tiles; ++t) {
    wait_vmcnt<(NS - 2) * Ring::PW>();
    wait_lgkmcnt0();  // this wave's column means of tile t-1 are in LDS
    wg_barrier();
    kr.stage((t + NS - 1) % NS, t + NS - 1);
    if (a.agg != SVLM_AGG_QHEAD && t > 0) flush(t - 1);
    const unsigned base = ring0 + (unsigned)((t % NS) * Ring::TB);
    float col[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4 kq[KK];
      read_k_block<KK>(base + (unsigned)(kb * 16 * Ring::ROWB), ko, kq);
      col[kb] = qk_colsum_block<RB, KK>(qreg, kq, lse, a.c);
    }
    // column sums over the rows held by the four lane groups; lane (c, g4) then
    // keeps key 16 g4 + c of the tile
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) col[kb] = sum_xor32(sum_xor16(col[kb]));
    const float v = ((g4 == 0) ? col[0] : (g4 == 1) ? col[1] : (g4 == 2) ? col[2] : col[3]) * invT;
    const int key = v_begin + t * kTileKeys + 16 * g4 + c;
    if (a.agg == SVLM_AGG_QHEAD) {
      if (active && key < v_end) emit(h, key, v);
    } else {
      xch[t & 1][wave][16 * g4 + c] = active ? v : 0.f;
    }
  }
  wait_vmcnt<0>();
  if (a.agg != SVLM_AGG_QHEAD && n_tiles > 0) {
    wait_lgkmcnt0();
    wg_barrier();
    flush(n_tiles - 1);
  }
}

// final mean over the group sums (KV-head rows split over several workgroups,
// or the single all-head row), out = alpha * mean + beta * out
__global__ __launch_bounds__(256) void score_agg(ScoreArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int r = blockIdx.y;
  if (i >= a.n_vis) return;
  int r0, nr;
  float div;
  if (a.agg == SVLM_AGG_KVHEAD) {
    r0 = r * a.HG2;
    nr = a.HG2;
    div = (float)a.G;
  } else {
    r0 = 0;
    nr = a.Hkv * a.HG2;
    div = (float)a.Hq;
  }
  float acc = 0.f;
  for (int k = 0; k < nr; ++k) acc += a.grp[(int64_t)(r0 + k) * a.n_vis + i];
  const float v = acc / div;
  float* o = a.out + (int64_t)r * a.n_vis + i;
  *o = (a.beta == 0.f) ? a.alpha * v : a.alpha * v + a.beta * (*o);
}

// (g, s) pairs in groups of 8 (one per XCD), times the head groups
inline unsigned pass_blocks(int Hkv, int S, int HG) { return (unsigned)((Hkv * S + 7) / 8 * 8 * HG); }

template <int D, int RB, int W>
void launch_pass1(const ScoreArgs& a, hipStream_t st) {
  score_pass1<D, RB, W, score_ring_depth<D, W>()><<<pass_blocks(a.Hkv, a.S1, a.HG1), 64 * W, 0, st>>>(a);
}
template <int D, int RB, int W>
void launch_pass2(const ScoreArgs& a, hipStream_t st) {
  score_pass2<D, RB, W, score_ring_depth<D, W>()><<<pass_blocks(a.Hkv, a.S2, a.HG2), 64 * W, 0, st>>>(a);
}

template <int D, int RB>
void launch_rb(const ScoreArgs& a, int w1, int w2, hipStream_t st) {
  switch (w1) {
    case 1: launch_pass1<D, RB, 1>(a, st); break;
    case 2: launch_pass1<D, RB, 2>(a, st); break;
    case 4: launch_pass1<D, RB, 4>(a, st); break;
    default: launch_pass1<D, RB, 8>(a, st); break;
  }
  switch (w2) {
    case 1: launch_pass2<D, RB, 1>(a, st); break;
    case 2: launch_pass2<D, RB, 2>(a, st); break;
    default: launch_pass2<D, RB, 4>(a, st); break;
  }
}

template <int D>
void launch_d(const ScoreArgs& a, int rb, int w1, int w2, hipStream_t st) {
  switch (rb) {
    case 1: launch_rb<D, 1>(a, w1, w2, st); break;
    case 2: launch_rb<D, 2>(a, w1, w2, st); break;
    case 4: launch_rb<D, 4>(a, w1, w2, st); break;
    case 6: launch_rb<D, 6>(a, w1, w2, st); break;
    default: launch_rb<D, 8>(a, w1, w2, st); break;
  }
}

int pick_rb(int T) {
  if (T <= 16) return 1;
  if (T <= 32) return 2;
  if (T <= 64) return 4;
  if (T <= 96) return 6;
  return 8;
}

// waves per workgroup: the q heads of a KV group, rounded up to a power of two,
// at most `cap`.  Pass 1 takes up to 8 (two waves per SIMD hide each other's
// waits); pass 2 up to 4 (it is bound by exp throughput, and one wave per SIMD
// spares the barrier across eight)
int pick_waves(int G, int cap) {
  int w = 1;
  while (w < G && w < cap) w *= 2;
  return w;
}

// key splits so that there is about one workgroup per compute unit, with at
// least 2 tiles per split; the split length is a whole number of tiles
int pick_splits(int groups, int w, int keys, int* kps) {
  (void)w;
  const int target = std::max(1, num_cus());
  int S = std::max(1, (target + groups - 1) / groups);
  const int tiles = (keys + kTileKeys - 1) / kTileKeys;
  S = std::max(1, std::min(S, tiles / 2));
  const int per_tiles = (tiles + S - 1) / S;
  *kps = per_tiles * kTileKeys;
  return (keys + *kps - 1) / *kps;
}

struct Geometry {
  int W1, HG1, S1, kps1, W2, HG2, S2, kps2;
};
Geometry geometry(int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  Geometry gm;
  const int G = Hq / Hkv;
  gm.W1 = pick_waves(G, 8);
  gm.HG1 = (G + gm.W1 - 1) / gm.W1;
  gm.S1 = pick_splits(Hkv * gm.HG1, gm.W1, q_pos0 + T, &gm.kps1);
  gm.W2 = pick_waves(G, 4);
  gm.HG2 = (G + gm.W2 - 1) / gm.W2;
  gm.S2 = pick_splits(Hkv * gm.HG2, gm.W2, n_vis, &gm.kps2);
  return gm;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" size_t svlm_score_workspace(int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  if (T < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || q_pos0 < 0 || n_vis < 1) return 0;
  const Geometry gm = geometry(T, Hq, Hkv, q_pos0, n_vis);
  const size_t ml = ((size_t)Hq * T * gm.S1 * 2 * sizeof(float) + 255) / 256 * 256;
  return ml + (size_t)Hkv * gm.HG2 * n_vis * sizeof(float);
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
  // buffer-descriptor ranges and offsets are 32-bit: one head's text queries,
  // and one KV head's keys (plus the tiles staged past a split's end)
  if (((int64_t)(T - 1) * q_st + D) * 2 > INT32_MAX || ((int64_t)n_ctx + 1024) * k_sn * 2 > INT32_MAX)
    return fail(SVLM_E_UNSUPPORTED, "svlm_score: (T-1) * q_st + D and (n_ctx + 1024) * k_sn must stay below 2^30 elements");
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
  const Geometry gm = geometry(T, Hq, Hkv, q_pos0, n_vis);
  a.HG1 = gm.HG1;
  a.HG2 = gm.HG2;
  a.S1 = gm.S1;
  a.kps1 = gm.kps1;
  a.S2 = gm.S2;
  a.kps2 = gm.kps2;
  const size_t ml_bytes = ((size_t)Hq * T * a.S1 * 2 * sizeof(float) + 255) / 256 * 256;
  const size_t need = svlm_score_workspace(T, Hq, Hkv, q_pos0, n_vis);
  if (!ws || ws_bytes < need)
    return fail(SVLM_E_WORKSPACE, "svlm_score: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return fail(SVLM_E_INVALID, "svlm_score: workspace must be 16-byte aligned");
  a.ml = (float*)ws;
  a.grp = (float*)((char*)ws + ml_bytes);
  a.agg = agg;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  hipStream_t st = (hipStream_t)stream;
  const int rb = pick_rb(T);
  if (D == 128) launch_d<128>(a, rb, gm.W1, gm.W2, st);
  else launch_d<64>(a, rb, gm.W1, gm.W2, st);
  const bool direct = (agg == SVLM_AGG_QHEAD) || (agg == SVLM_AGG_KVHEAD && gm.HG2 == 1);
  if (!direct) {
    const int rows = (agg == SVLM_AGG_KVHEAD) ? Hkv : 1;
    score_agg<<<dim3((unsigned)((n_vis + 255) / 256), (unsigned)rows), 256, 0, st>>>(a);
  }
  return check_launch("svlm_score");
}
