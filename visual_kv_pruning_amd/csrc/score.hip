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
// A workgroup owns one KV head and one key range.  Its waves (up to 8) share
// the group's (q head, 16-row text block) units: round-robin over the waves
// where a wave per head would leave waves idle, else one head per wave.  The
// key tile (64 keys) is staged HBM -> LDS once by
// LDS-DMA transfers that all waves share (one barrier per tile), so K is read
// from memory once per workgroup; the text queries of a wave's units sit in
// registers.  Both passes use v_mfma_f32_16x16x32_bf16 with fp32 accumulation
// and compute S^T (lane = one text row x 4 keys per 16-key block, so a lane
// needs one log-sum-exp per row block).  Pass 1 keeps a lazily raised
// reference maximum per lane group, so a key costs one fma, one exp2 and one
// add; pass 2 adds a lane's row blocks in registers and the 16 row lanes of
// each key through LDS, and the waves add their units through LDS.  Several
// layers can share one launch of each pass.
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr float kNegInf = -INFINITY;
constexpr int kTileKeys = 64;      // keys per staged K tile
constexpr float kRescaleSum = 256.f;  // a lane's 4-key weight sum above this raises its reference maximum
constexpr int kLseBatch = 32;      // pass-1 partials per row loaded at once when a row's log-sum-exp is formed
constexpr int kUnits2Max8 = 4;     // pass 2 with eight waves: most units per wave in the unit form

struct ScoreArgs {
  const uint16_t* q;
  int64_t q_st, q_sh;
  const uint16_t* k;
  int64_t k_sh, k_sn;
  int T, n_ctx, q_pos0, vis_start, n_vis, Hq, Hkv, G;
  int HG1, HG2;  // head groups (workgroups) per KV head, pass 1 and pass 2
  float c;  // scale * log2(e), > 0
  int S1, kps1, S2, kps2;
  float* ml;   // [Hq][S1][T][2]: per split, (reference maximum in raw-score units, sum); split-major,
               // so one split's rows are contiguous for the loads that merge them
  float* grp;  // [Hkv * HG][n_vis]: per head group, the sum over its heads of the column means
  int agg;
  float alpha, beta;
  float* out;
  // several layers per call: workgroups of layer l follow those of layer l-1
  int layers;             // 1 for svlm_score
  int64_t q_sl, k_sl;     // per-layer element strides of q and k
  int64_t ws_sl;          // per-layer float stride of both workspace parts (ml and grp)
  int layer_mean;         // 1: the layers are averaged into one row set (score_agg_layers)
  int rows;               // output rows per layer (by agg)
};

// the arguments as seen by one layer's workgroups: inputs, workspace and (one
// row set per layer) output moved to that layer
__device__ __forceinline__ ScoreArgs layer_args(const ScoreArgs& a0, int layer) {
  ScoreArgs a = a0;
  a.q += layer * a0.q_sl;
  a.k += layer * a0.k_sl;
  a.ml += layer * a0.ws_sl;
  a.grp += layer * a0.ws_sl;
  if (!a0.layer_mean) a.out += (int64_t)layer * a0.rows * a0.n_vis;
  return a;
}

// block id -> (layer, KV head g, head group hg, key split s).  Workgroups are
// handed to the eight XCDs round-robin by id, so the HG head groups of one
// (layer, KV head, split) take ids 8 apart: they run on one XCD, and the K
// tiles one of them fetches reach the others from that XCD's L2.  The
// (layer, g, s) triples are numbered across layers, so only the last group
// of eight can be partial (its missing ids are idle) and every XCD gets an
// equal share.
__device__ __forceinline__ bool decode_block(int bid, int S, int Hkv, int HG, int layers, int& layer, int& g,
                                             int& hg, int& s) {
  const int rest = bid >> 3;
  hg = rest % HG;
  const int trip = (rest / HG) * 8 + (bid & 7);
  const int per_layer = Hkv * S;
  if (trip >= layers * per_layer) return false;
  layer = trip / per_layer;
  const int pair = trip - layer * per_layer;
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
// at most NS - 1 tiles are outstanding (6-bit wait counter); LDS holds NS
// tiles, at most MAXNS.  A tile's arithmetic takes several microseconds, far
// longer than staging one, so a shallow ring keeps the key loop fed; deeper
// rings only add to the burst of loads every workgroup issues at once when
// the kernel starts.  Measured per 72B-shape layer: pass 1 best at 4 slots,
// pass 2 at 3.
#ifndef SVLM_SCORE_RING1
#define SVLM_SCORE_RING1 4
#endif
#ifndef SVLM_SCORE_RING2
#define SVLM_SCORE_RING2 3
#endif
template <int D, int W, int MAXNS>
constexpr int score_ring_depth() {
  constexpr int TB = kTileKeys * D * 2;
  constexpr int PW = (TB / 1024) / W;
  int ns = 2;
  while (ns < MAXNS && ns * PW <= 63 && (size_t)(ns + 1) * TB <= 128 * 1024) ++ns;
  return ns;
}

// Staging of the K tiles of one (KV head, key range) through a ring of NS
// slots in LDS: every wave issues its share (PW transfers of 1 KB) of each
// tile; rows are XOR-swizzled by 16-byte chunk (chunk p of row r holds source
// chunk p ^ (r % CH)).  Tiles past the range deliver zeros.  Transfer i of
// wave w moves the tile's 1 KB piece i W + w.  When W is a multiple of 4 (or
// at D = 64, where a piece spans whole swizzle periods) every piece a lane
// moves has the same row phase, so one per-lane source offset serves all of
// them and the piece's first row enters as the scalar offset (no per-transfer
// offset registers to keep live through the key loop).
template <int D, int W, int NS>
struct KRing {
  static constexpr int ROWB = D * 2, CH = ROWB / 16;
  static constexpr int TB = kTileKeys * ROWB;
  static constexpr int NI = TB / 1024;
  static constexpr int PW = NI / W;
  static constexpr int RPT = 1024 / ROWB;  // rows per transfer
  static constexpr bool kOneOffset = (CH <= RPT) || (W % (CH / RPT) == 0);
  static_assert(PW >= 1 && NI % W == 0, "tile transfers must split evenly over the waves");
  static_assert((NS - 1) * PW <= 63, "ring depth");
  static constexpr int kMaxPW = 16;  // one wave staging a whole D = 128 tile
  static_assert(PW <= kMaxPW, "transfers per wave");
  __amdgpu_buffer_rsrc_t rs;
  unsigned char* lds;
  int wave, row_bytes;
  // per-lane source offset of each of this wave's PW transfers (only the
  // first when kOneOffset; a fixed bound: sized by the template parameters,
  // the host pass of this compiler dropped the kernels' launch stubs)
  int src_lane[kMaxPW];

  __device__ void init(const uint16_t* k_rows, int n_rows, int64_t k_sn, unsigned char* ring, int w) {
    const int lane = threadIdx.x & 63;
    row_bytes = (int)(k_sn * 2);
    rs = __builtin_amdgcn_make_buffer_rsrc((void*)k_rows, (short)0, n_rows * row_bytes, kBufferFlags);
    lds = ring;
    wave = w;
#pragma unroll
    for (int i = 0; i < (kOneOffset ? 1 : PW); ++i) {
      const int r = (i * W + wave) * RPT + lane / CH;
      const int p = lane % CH;
      src_lane[i] = (kOneOffset ? lane / CH : r) * row_bytes + ((p ^ (r % CH)) * 16);
    }
  }
  __device__ __forceinline__ void stage_to(unsigned char* dst, int tile) const {
    const int soff = tile * kTileKeys * row_bytes;
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int piece = i * W + wave;
      if constexpr (kOneOffset)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + piece * 1024), 16,
                                                 src_lane[0], soff + piece * RPT * row_bytes, 0, kNT);
      else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(dst + piece * 1024), 16,
                                                 src_lane[i], soff, 0, kNT);
    }
  }
  __device__ __forceinline__ void stage(int slot, int tile) const { stage_to(lds + slot * TB, tile); }
  // LDS byte offset (within a slot) of the lane's K operand chunk: key row r, d chunk kk*4 + g4
  static __device__ unsigned koff(int r, int kk, int g4) { return r * ROWB + (((kk * 4 + g4) ^ (r % CH)) * 16); }
};

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

// Work units of a KV group: (q head, 16-row block of the text).
//  - Unit form: unit u (head u / RBT, row block u % RBT, RBT = row blocks of
//    T) goes to wave slot u mod (HG W) of the group's HG workgroups of W
//    waves, so every wave holds U or U - 1 units, U = ceil(G RBT / (HG W)).
//    With a wave per head, five heads per KV head left three of eight waves
//    idle and two SIMDs carrying two heads each; seven left one SIMD at half
//    the load of the others.
//  - Head form (pass 2 with one output row per q head): wave hl = hg W + w
//    holds the U row blocks of head hl (none past the group).
// A unit's text queries sit in registers as the B operand of S^T = K Q^T.
template <bool UNITS>
struct WaveUnits {
  int n;                       // units of this wave (wave-uniform)
  int slot, stride, total, rbt, g0, G;
  __device__ WaveUnits(const ScoreArgs& a, int g, int hg, int HG, int W, int wave, int U) {
    G = a.G;
    g0 = g * a.G;
    slot = hg * W + wave;
    rbt = (a.T + 15) / 16;
    if constexpr (UNITS) {
      stride = HG * W;
      total = a.G * rbt;
      n = (total > slot) ? (total - slot + stride - 1) / stride : 0;
    } else {
      stride = 0;
      total = 0;
      n = (slot < a.G) ? U : 0;
    }
  }
  // q head (global index) and first text row of unit i of this wave; units
  // past n repeat the wave's last one (their results are never used)
  __device__ __forceinline__ void at(int i, int& head, int& row0) const {
    if constexpr (UNITS) {
      const int u = min(slot + stride * i, total - 1);
      const int hl = u / rbt;
      head = g0 + hl;
      row0 = (u - hl * rbt) * 16;
    } else {
      head = g0 + min(slot, G - 1);
      row0 = 16 * i;
    }
  }
};

// one unit's text queries: lane (c, g4) holds row row0 + c, d = 32 kk + 8 g4 .. + 7 (rows past T read zeros)
template <int D>
__device__ __forceinline__ void load_q_unit(const ScoreArgs& a, int h, int row0, u32x4 (&q)[D / 32]) {
  const int lane = threadIdx.x & 63, c = lane & 15, g4 = lane >> 4;
  const int bytes = (int)(((int64_t)(a.T - 1) * a.q_st + D) * 2);
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + (int64_t)h * a.q_sh), (short)0, bytes, kBufferFlags);
  const int t = row0 + c;
#pragma unroll
  for (int kk = 0; kk < D / 32; ++kk) {
    const int off = (t < a.T) ? (int)(((int64_t)t * a.q_st + 32 * kk + 8 * g4) * 2) : bytes;
    q[kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
  }
}

// Runs f(integral_constant<C>) with C the wave's unit count: U, U - 1 (unit
// form) or 0, so the key loops are unrolled over exactly the units a wave holds.
template <int U, bool UNITS, class F>
__device__ __forceinline__ void with_count(int n, F&& f) {
  if (n == U) {
    f(std::integral_constant<int, U>{});
  } else if constexpr (UNITS && U > 1) {
    if (n == U - 1) f(std::integral_constant<int, U - 1>{});
    else f(std::integral_constant<int, 0>{});
  } else {
    f(std::integral_constant<int, 0>{});
  }
}

template <int D, int U, int W, int NS, bool UNITS>
__global__ __launch_bounds__(64 * W, 1) void score_pass1(ScoreArgs a0) {
  constexpr int KK = D / 32;
  using Ring = KRing<D, W, NS>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  int layer, g, hg, s;
  if (!decode_block((int)blockIdx.x, a0.S1, a0.Hkv, a0.HG1, a0.layers, layer, g, hg, s)) return;
  const ScoreArgs a = layer_args(a0, layer);
  const WaveUnits<UNITS> wu(a, g, hg, a.HG1, W, wave, U);

  const int k_begin = s * a.kps1;
  const int k_end = min(k_begin + a.kps1, a.q_pos0 + a.T);
  const int n_tiles = (k_end > k_begin) ? (k_end - k_begin + kTileKeys - 1) / kTileKeys : 0;

  __shared__ __align__(16) unsigned char ring[NS * Ring::TB];
  Ring kr;
  kr.init(a.k + (int64_t)g * a.k_sh + (int64_t)k_begin * a.k_sn, max(k_end - k_begin, 0), a.k_sn, ring, wave);
  // tiles below n_full are visible to every row and lie inside the range
  const int vis_all = min(k_end, a.q_pos0 + 1) - k_begin;
  const int n_full = min(n_tiles, vis_all > 0 ? vis_all / kTileKeys : 0);
  // LDS offsets of the lane's K chunks in key block 0 (block 1 is 16 rows on)
  unsigned ko[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) ko[kk] = Ring::koff(c, kk, g4);
  const unsigned ring0 = lds_addr(ring);

  // every wave stages its share of every K tile and meets every barrier; a
  // wave with no units skips the arithmetic
  with_count<U, UNITS>(wu.n, [&](auto cnt) __attribute__((always_inline)) {
    constexpr int C = decltype(cnt)::value;
    constexpr int CQ = C > 0 ? C : 1;
    int uh[CQ], ur[CQ];
#pragma unroll
    for (int i = 0; i < CQ; ++i) wu.at(i, uh[i], ur[i]);
    u32x4 qreg[CQ][KK];
    if constexpr (C > 0) {
#pragma unroll
      for (int i = 0; i < C; ++i) load_q_unit<D>(a, uh[i], ur[i], qreg[i]);
    }
#pragma unroll
    for (int u = 0; u < NS - 1; ++u) kr.stage(u, u);
    wait_vmcnt<(NS - 1) * Ring::PW>();  // the query loads, issued first, have landed

    // per unit and lane group: reference maximum in log2 units of the scaled score, sum
    float mc[CQ], l[CQ];
#pragma unroll
    for (int i = 0; i < CQ; ++i) {
      mc[i] = kNegInf;
      l[i] = 0.f;
    }

    auto tile = [&](int t, bool masked) __attribute__((always_inline)) {
      wait_vmcnt<(NS - 2) * Ring::PW>();  // this wave's share of tile t has landed
      wg_barrier();                       // every share of tile t has landed; tile t-1 is retired
      kr.stage((t + NS - 1) % NS, t + NS - 1);
      if constexpr (C > 0) {
        const unsigned base = ring0 + (unsigned)((t % NS) * Ring::TB);
        u32x4 kq2[2][KK];  // K operands of two blocks per LDS wait
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {  // one 16-key block of products at a time keeps the live registers low
          if (kb % 2 == 0) read_k_pair<KK, 16 * Ring::ROWB>(base + (unsigned)(kb * 16 * Ring::ROWB), ko, kq2);
          const u32x4 (&kq)[KK] = kq2[kb % 2];
          const int key0 = k_begin + t * kTileKeys + 16 * kb;
#pragma unroll
          for (int i = 0; i < C; ++i) {
            f32x4 s0 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) s0 = mfma16(as_bf16x8(kq[kk]), as_bf16x8(qreg[i][kk]), s0);
            float x[4];
            if (masked) {
              const int tq = ur[i] + c;
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
            for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(x[e], a.c, -mc[i]));
            float s4 = (p[0] + p[1]) + (p[2] + p[3]);
            if (!(s4 <= kRescaleSum)) {
              const float lmax = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])) * a.c;
              const float m_new = fmaxf(mc[i], lmax);
              l[i] *= (mc[i] == kNegInf) ? 0.f : fast_exp2(mc[i] - m_new);
              mc[i] = m_new;
              const float mneg = (m_new == kNegInf) ? 0.f : -m_new;
#pragma unroll
              for (int e = 0; e < 4; ++e) p[e] = fast_exp2(fmaf(x[e], a.c, mneg));
              s4 = (p[0] + p[1]) + (p[2] + p[3]);
            }
            l[i] += s4;
          }
        }
      }
    };
    int t = 0;
    for (; t < n_full; ++t) tile(t, false);
    for (; t < n_tiles; ++t) tile(t, true);
    wait_vmcnt<0>();

    // merge the four lane groups (fixed order) and write this split's row
    // state (maximum back in raw-score units)
#pragma unroll
    for (int i = 0; i < C; ++i) {
      float m = (mc[i] == kNegInf) ? kNegInf : mc[i] / a.c, ll = l[i];
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
      const int tq = ur[i] + c;
      if (g4 == 0 && tq < a.T) *(float2*)(a.ml + (((int64_t)uh[i] * a.S1 + s) * a.T + tq) * 2) = make_float2(m, ll);
    }
  });
}

// Pass 2.  Units (group sums): a wave adds the column weights of all its
// units, whatever their heads; per-head output rows take the head form.
template <int D, int U, int W, int NS, bool UNITS>
__global__ __launch_bounds__(64 * W, 1) void score_pass2(ScoreArgs a0) {
  constexpr int KK = D / 32;
  using Ring = KRing<D, W, NS>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c = lane & 15, g4 = lane >> 4;
  int layer, g, hg, s;
  if (!decode_block((int)blockIdx.x, a0.S2, a0.Hkv, a0.HG2, a0.layers, layer, g, hg, s)) return;
  const ScoreArgs a = layer_args(a0, layer);
  const WaveUnits<UNITS> wu(a, g, hg, a.HG2, W, wave, U);

  const int v_begin = a.vis_start + s * a.kps2;
  const int v_end = min(v_begin + a.kps2, a.vis_start + a.n_vis);
  const int n_tiles = (v_end > v_begin) ? (v_end - v_begin + kTileKeys - 1) / kTileKeys : 0;

  static_assert(NS == 3, "three named staging slots");
  __shared__ __align__(16) unsigned char ring[Ring::TB];
  __shared__ __align__(16) unsigned char ring_b[Ring::TB];
  __shared__ __align__(16) unsigned char ring_c[Ring::TB];
  __shared__ float sm_lse[W][U * 16];
  __shared__ float xch[2][W][kTileKeys];
  __shared__ __align__(16) float red[W][kTileKeys][20];
  Ring kr;
  kr.init(a.k + (int64_t)g * a.k_sh + (int64_t)v_begin * a.k_sn, max(v_end - v_begin, 0), a.k_sn, ring, wave);

  // Row log-sum-exp (log2 units of the scaled score) of the wave's unit rows
  // from the pass-1 partials, in split order; padded rows and units past the
  // wave's count get +inf and so contribute exp2(-inf) = 0.  Lane = one row
  // of one unit (the 16 rows of a unit are consecutive rows of one head, so
  // each load reads consecutive rows of one split: the partials are
  // split-major).  The first kLseBatch partials of the lane's rows are loaded
  // before anything else, so their round trip waits behind no other load
  // (memory operations complete in issue order); the K tiles are staged
  // behind them, and the queries are loaded once the partials are merged,
  // when their registers are free.
  constexpr int RPL = (U * 16 + 63) / 64;  // rows per lane
  float M[RPL], L[RPL];
  int row_ok[RPL];
  int64_t row_off[RPL];  // float offset of the lane's row in split 0 of the partials
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int rho = lane + 64 * r;
    const int i = min(rho >> 4, U - 1);
    int h, r0;
    wu.at(i, h, r0);
    const int tq = r0 + (rho & 15);
    row_ok[r] = (rho < U * 16) && (i < wu.n) && (tq < a.T);
    row_off[r] = ((int64_t)h * a.S1 * a.T + min(tq, a.T - 1)) * 2;
  }
  auto load_parts = [&](int s0, float2 (&part)[RPL][kLseBatch]) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      const float2* p = (const float2*)(a.ml + row_off[r]);
#pragma unroll
      for (int j = 0; j < kLseBatch; ++j)
        part[r][j] = (row_ok[r] && s0 + j < a.S1) ? p[(int64_t)(s0 + j) * a.T] : make_float2(kNegInf, 0.f);
    }
  };
  // a batch of partials joins the running (M, L) in two steps: the largest
  // reference first, then every sum weighed against it (one exp2 per
  // partial, no branches; a split that saw no key has (-inf, 0) and adds 0)
  auto merge_parts = [&](const float2 (&part)[RPL][kLseBatch]) {
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float bm = kNegInf;
#pragma unroll
      for (int j = 0; j < kLseBatch; ++j) bm = fmaxf(bm, part[r][j].x);
      const float m_new = fmaxf(M[r], bm);
      const float mref = (m_new == kNegInf) ? 0.f : m_new;
      float acc = (M[r] == kNegInf) ? 0.f : L[r] * fast_exp2((M[r] - mref) * a.c);
#pragma unroll
      for (int j = 0; j < kLseBatch; ++j) acc = fmaf(part[r][j].y, fast_exp2((part[r][j].x - mref) * a.c), acc);
      M[r] = m_new;
      L[r] = acc;
    }
  };
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    M[r] = kNegInf;
    L[r] = 0.f;
  }
  {
    float2 part[RPL][kLseBatch];
    load_parts(0, part);
    kr.stage_to(ring, 0);
    kr.stage_to(ring_b, 1);
    merge_parts(part);
  }
  for (int s0 = kLseBatch; s0 < a.S1; s0 += kLseBatch) {
    float2 part[RPL][kLseBatch];
    load_parts(s0, part);
    merge_parts(part);
  }
#pragma unroll
  for (int r = 0; r < RPL; ++r) {
    const int rho = lane + 64 * r;
    if (rho < U * 16) sm_lse[wave][rho] = (row_ok[r] && L[r] > 0.f) ? M[r] * a.c + log2f(L[r]) : INFINITY;
  }

  const float invT = 1.f / (float)a.T;
  const bool direct = !a.layer_mean && ((a.agg == SVLM_AGG_QHEAD) || (a.agg == SVLM_AGG_KVHEAD && a.HG2 == 1));
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
  // wave 0 adds the waves' column sums of tile tt (published in xch[tt % 2])
  auto flush = [&](int tt) {
    if (wave != 0) return;
    const int key = v_begin + tt * kTileKeys + lane;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) v += xch[tt & 1][w][lane];
    if (key < v_end) emit(direct ? g : g * a.HG2 + hg, key, v * grp_scale);
  };
  const bool qhead = !UNITS && a.agg == SVLM_AGG_QHEAD;

  with_count<U, UNITS>(wu.n, [&](auto cnt) __attribute__((always_inline)) {
    constexpr int C = decltype(cnt)::value;
    constexpr int CQ = C > 0 ? C : 1;
    u32x4 qreg[CQ][KK];
    float lse_t[CQ];  // the lane's text row of each unit
    int h_out = 0;
    if constexpr (C > 0) {
#pragma unroll
      for (int i = 0; i < C; ++i) {
        int h, r0;
        wu.at(i, h, r0);
        load_q_unit<D>(a, h, r0, qreg[i]);
        h_out = h;
      }
    }
    wait_lgkmcnt0();
#pragma unroll
    for (int i = 0; i < CQ; ++i) lse_t[i] = sm_lse[wave][i * 16 + c];

    unsigned ko[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) ko[kk] = Ring::koff(c, kk, g4);

    auto body = [&](int t, const unsigned char* rd, unsigned char* dma) __attribute__((always_inline)) {
      wait_vmcnt<(NS - 2) * Ring::PW>();
      wait_lgkmcnt0();  // this wave's column sums of tile t-1 are in LDS
      wg_barrier();
      kr.stage_to(dma, t + NS - 1);
      if (!qhead && t > 0) flush(t - 1);
      const int key = v_begin + t * kTileKeys + lane;
      if constexpr (C == 0) {  // a wave with no units adds nothing
        if (!qhead) xch[t & 1][wave][lane] = 0.f;
        return;
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          u32x4 kq[KK];
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) kq[kk] = *(const u32x4*)(rd + kb * 16 * Ring::ROWB + ko[kk]);
          f32x4 S[C];
#pragma unroll
          for (int i = 0; i < C; ++i) {
            S[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < KK; ++kk) S[i] = mfma16(as_bf16x8(kq[kk]), as_bf16x8(qreg[i][kk]), S[i]);
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            float e[C];
#pragma unroll
            for (int i = 0; i < C; ++i) e[i] = fast_exp2(fmaf(S[i][q], a.c, -lse_t[i]));
#pragma unroll
            for (int w2 = 1; w2 < C; w2 *= 2)
#pragma unroll
              for (int i = 0; i + w2 < C; i += 2 * w2) e[i] += e[i + w2];
            red[wave][16 * kb + 4 * g4 + q][c] = e[0];
          }
        }
        float4 rr[4];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) rr[q4] = *(const float4*)&red[wave][lane][4 * q4];
        float v = 0.f;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) v = (((v + rr[q4].x) + rr[q4].y) + rr[q4].z) + rr[q4].w;
        v *= invT;
        if (qhead) {
          if (key < v_end) emit(h_out, key, v);
        } else {
          xch[t & 1][wave][lane] = v;
        }
      }
    };
    int t = 0;
    for (; t + 3 <= n_tiles; t += 3) {
      body(t, ring, ring_c);
      body(t + 1, ring_b, ring);
      body(t + 2, ring_c, ring_b);
    }
    if (t < n_tiles) body(t, ring, ring_c);
    if (t + 1 < n_tiles) body(t + 1, ring_b, ring);
  });
  wait_vmcnt<0>();
  if (!qhead && n_tiles > 0) {
    wait_lgkmcnt0();
    wg_barrier();
    flush(n_tiles - 1);
  }
}

constexpr int kAggBatch = 16;

// final mean over the group sums (KV-head rows split over several workgroups,
// or the single all-head row), out = alpha * mean + beta * out
// the group-sum rows behind output row r of a layer, and the head count they cover
__device__ __forceinline__ void group_rows(const ScoreArgs& a, int r, int& r0, int& nr, float& div) {
  if (a.agg == SVLM_AGG_KVHEAD) {
    r0 = r * a.HG2;
    nr = a.HG2;
    div = (float)a.G;
  } else {
    r0 = 0;
    nr = a.Hkv * a.HG2;
    div = (float)a.Hq;
  }
}

// the sum of group rows r0 .. r0 + nr - 1 at one element (g points at row 0 of
// the element's column): kAggBatch loads in flight at a time, every load of a
// batch issued before the first add (rows past the last are clamped to it and
// not added); the adds keep row order
__device__ __forceinline__ float sum_group_rows(const float* g, int64_t row_stride, int r0, int nr) {
  float acc = 0.f;
  for (int k0 = 0; k0 < nr; k0 += kAggBatch) {
    float x[kAggBatch];
#pragma unroll
    for (int j = 0; j < kAggBatch; ++j) x[j] = g[(int64_t)(r0 + min(k0 + j, nr - 1)) * row_stride];
#pragma unroll
    for (int j = 0; j < kAggBatch; ++j)
      if (k0 + j < nr) acc += x[j];
  }
  return acc;
}

// one row set per layer: blockIdx.y = layer * rows + r
__global__ __launch_bounds__(256) void score_agg(ScoreArgs a) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  const int layer = (int)blockIdx.y / a.rows;
  const int r = (int)blockIdx.y - layer * a.rows;
  if (i >= a.n_vis) return;
  int r0, nr;
  float div;
  group_rows(a, r, r0, nr, div);
  float* o = a.out + (int64_t)blockIdx.y * a.n_vis + i;
  const float prev = (a.beta == 0.f) ? 0.f : *o;
  const float v = sum_group_rows(a.grp + layer * a.ws_sl + i, a.n_vis, r0, nr) / div;
  *o = (a.beta == 0.f) ? a.alpha * v : a.alpha * v + a.beta * prev;
}

// the layers averaged into one row set: 64 elements per workgroup, each
// summed by kAggLanes threads over every kAggLanes-th layer, the lanes then
// added in a fixed order
constexpr int kAggLanes = 16;
__global__ __launch_bounds__(64 * kAggLanes) void score_agg_layers(ScoreArgs a) {
  const int e = threadIdx.x & 63, j = threadIdx.x >> 6;
  const int i = blockIdx.x * 64 + e;
  const int r = blockIdx.y;
  int r0, nr;
  float div;
  group_rows(a, r, r0, nr, div);
  __shared__ float part[kAggLanes][64];
  float acc = 0.f;
  if (i < a.n_vis)
    for (int l = j; l < a.layers; l += kAggLanes) acc += sum_group_rows(a.grp + l * a.ws_sl + i, a.n_vis, r0, nr);
  part[j][e] = acc;
  __syncthreads();
  if (j != 0 || i >= a.n_vis) return;
  float tot = 0.f;
#pragma unroll
  for (int jj = 0; jj < kAggLanes; ++jj) tot += part[jj][e];
  const float v = tot / (div * (float)a.layers);
  float* o = a.out + (int64_t)r * a.n_vis + i;
  *o = (a.beta == 0.f) ? a.alpha * v : a.alpha * v + a.beta * (*o);
}

// (layer, g, s) triples in groups of 8 (one per XCD), times the head groups
inline int64_t pass_blocks(int layers, int Hkv, int S, int HG) {
  return (mul_sat(mul_sat(layers, Hkv), S) + 7) / 8 * 8 * HG;
}

template <int D, int U, int W, bool UNITS>
void launch_pass1(const ScoreArgs& a, hipStream_t st) {
  score_pass1<D, U, W, score_ring_depth<D, W, SVLM_SCORE_RING1>(), UNITS><<<(unsigned)pass_blocks(a.layers, a.Hkv, a.S1, a.HG1), 64 * W, 0, st>>>(a);
}
template <int D, int U, int W, bool UNITS>
void launch_pass2(const ScoreArgs& a, hipStream_t st) {
  score_pass2<D, U, W, score_ring_depth<D, W, SVLM_SCORE_RING2>(), UNITS><<<(unsigned)pass_blocks(a.layers, a.Hkv, a.S2, a.HG2), 64 * W, 0, st>>>(a);
}

// one pass (PASS 1 or 2) with w waves; U units or row blocks per wave
template <int D, int PASS, int U, int W, bool UNITS>
void launch_one(const ScoreArgs& a, hipStream_t st) {
  if constexpr (PASS == 1) launch_pass1<D, U, W, UNITS>(a, st);
  else launch_pass2<D, U, W, UNITS>(a, st);
}
template <int D, int PASS, int U, bool UNITS>
void launch_pass(const ScoreArgs& a, int w, hipStream_t st) {
  if constexpr (UNITS) {  // the unit form runs at D = 128 with 4 or 8 waves
    // pass 2 with eight waves never holds more than kUnits2Max8 units
    // (use_units sends those shapes to the head form), so w is 4 here and the
    // eight-wave kernels are not instantiated for them
    if constexpr (PASS == 2 && U > kUnits2Max8) launch_one<D, PASS, U, 4, true>(a, st);
    else if (w == 4) launch_one<D, PASS, U, 4, true>(a, st);
    else launch_one<D, PASS, U, 8, true>(a, st);
  } else {
    switch (w) {
      case 1: launch_one<D, PASS, U, 1, false>(a, st); break;
      case 2: launch_one<D, PASS, U, 2, false>(a, st); break;
      case 4: launch_one<D, PASS, U, 4, false>(a, st); break;
      default: launch_one<D, PASS, U, 8, false>(a, st); break;
    }
  }
}
// unit form: u units per wave, 1 .. 8
template <int PASS>
void launch_units(const ScoreArgs& a, int u, int w, hipStream_t st) {
  switch (u) {
    case 1: launch_pass<128, PASS, 1, true>(a, w, st); break;
    case 2: launch_pass<128, PASS, 2, true>(a, w, st); break;
    case 3: launch_pass<128, PASS, 3, true>(a, w, st); break;
    case 4: launch_pass<128, PASS, 4, true>(a, w, st); break;
    case 5: launch_pass<128, PASS, 5, true>(a, w, st); break;
    case 6: launch_pass<128, PASS, 6, true>(a, w, st); break;
    case 7: launch_pass<128, PASS, 7, true>(a, w, st); break;
    default: launch_pass<128, PASS, 8, true>(a, w, st); break;
  }
}
// head form: rb row blocks per head (1, 2, 4, 6 or 8)
template <int D, int PASS>
void launch_heads(const ScoreArgs& a, int rb, int w, hipStream_t st) {
  switch (rb) {
    case 1: launch_pass<D, PASS, 1, false>(a, w, st); break;
    case 2: launch_pass<D, PASS, 2, false>(a, w, st); break;
    case 4: launch_pass<D, PASS, 4, false>(a, w, st); break;
    case 6: launch_pass<D, PASS, 6, false>(a, w, st); break;
    default: launch_pass<D, PASS, 8, false>(a, w, st); break;
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
// waits).  Pass 2 takes up to 8 on visual ranges of at least kPass2WideKeys
// keys, up to 4 on shorter ones: eight waves hold one head group per
// workgroup (half the workgroups, each over more keys), which pays on long
// rows and loses on short ones, where the per-wave set-up dominates
// (measured: 72B 96-99 against 100-104 us per layer, 32B 56 against 61,
// hour-long 153 against 157; 7B, 8192 keys, 13.8 against 12.0)
constexpr int kPass2WideKeys = 16384;
int pick_waves(int G, int cap) {
  int w = 1;
  while (w < G && w < cap) w *= 2;
  return w;
}

// units per wave of the unit form: G heads x ceil(T / 16) row blocks over HG workgroups of W waves
int units_per_wave(int T, int G, int HG, int W) {
  const int units = G * ((T + 15) / 16);
  return (units + HG * W - 1) / (HG * W);
}
// The unit form where a wave per head would leave waves idle (the head
// count of a group is not a multiple of the waves), at D = 128 with 4 or 8
// waves; the head form elsewhere (and for per-head output rows).  Pass 2 with
// eight waves takes the unit form up to kUnits2Max8 units per wave: beyond
// that its registers (two waves per SIMD share the file) spill inside the
// key loop, where the head form's do not.
bool use_units(int pass, int D, int T, int G, int HG, int W) {
  if (D != 128 || W < 4 || HG * W <= G) return false;
  return pass == 1 || W == 4 || units_per_wave(T, G, HG, W) <= kUnits2Max8;
}

// key splits: one layer takes about one workgroup per compute unit.  Several
// layers in one call take at least SVLM_SCORE_ROUNDS rounds of workgroups
// over the chip (one per CU); among up to four times that many splits, the
// count whose (rounds) x (set-up + tiles per workgroup) is least, which
// prefers long workgroups (set-up paid over more tiles) and whole rounds (no
// idle tail).  Measured against a fixed eight rounds, µs per layer: 72B 94.4
// against 96.1-97.2, 32B 54.8 against 56.2, 7B 11.1 against 12.4-13.3,
// hour-long 142-144 against 153-154.  At least 2 tiles per split; the split
// length is a whole number of tiles.
#ifndef SVLM_SCORE_ROUNDS
#define SVLM_SCORE_ROUNDS 4
#endif
constexpr int64_t kSetupTiles = 4;
int pick_splits(int64_t groups, int64_t keys, int layers, int* kps) {
  const int64_t target = std::max(1, num_cus());
  const int64_t tiles = (keys + kTileKeys - 1) / kTileKeys;
  const int64_t smax = std::max<int64_t>(1, tiles / 2);
  int64_t S;
  if (layers <= 1) {
    S = std::max<int64_t>(1, (target + groups - 1) / groups);
  } else {
    // at least SVLM_SCORE_ROUNDS rounds of workgroups; within four times that
    // many splits, the count that minimises (rounds) x (set-up + tiles per
    // workgroup), the set-up counted as kSetupTiles tiles
    const int64_t units = mul_sat(groups, layers);
    const int64_t need = SVLM_SCORE_ROUNDS * target;
    const int64_t lo = std::min(smax, (units >= need) ? (int64_t)1 : (need + units - 1) / units);
    const int64_t hi = std::min(smax, 4 * lo);
    int64_t best_cost = INT64_MAX;
    S = lo;
    for (int64_t s = lo; s <= hi; ++s) {
      const int64_t n = mul_sat(units, s);
      const int64_t rounds = n / target + (n % target != 0);
      const int64_t cost = mul_sat(rounds, kSetupTiles + (tiles + s - 1) / s);
      if (cost < best_cost) {
        best_cost = cost;
        S = s;
      }
    }
  }
  S = std::max<int64_t>(1, std::min(S, smax));
  const int64_t per_tiles = (tiles + S - 1) / S;
  *kps = (int)(per_tiles * kTileKeys);
  return (int)((keys + *kps - 1) / *kps);
}

struct Geometry {
  int W1, HG1, S1, kps1, W2, HG2, S2, kps2;
};
Geometry geometry(int T, int Hq, int Hkv, int q_pos0, int n_vis, int layers) {
  Geometry gm;
  const int G = Hq / Hkv;
  gm.W1 = pick_waves(G, 8);
  gm.HG1 = (G + gm.W1 - 1) / gm.W1;
  gm.S1 = pick_splits((int64_t)Hkv * gm.HG1, (int64_t)q_pos0 + T, layers, &gm.kps1);
  gm.W2 = pick_waves(G, n_vis >= kPass2WideKeys ? 8 : 4);
  gm.HG2 = (G + gm.W2 - 1) / gm.W2;
  gm.S2 = pick_splits((int64_t)Hkv * gm.HG2, n_vis, layers, &gm.kps2);
  return gm;
}

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// one layer's workspace: the pass-1 row statistics, then the group-sum rows
struct WsParts {
  size_t ml, grp, layer;
};
WsParts ws_parts(const Geometry& gm, int T, int Hq, int Hkv, int n_vis) {
  WsParts w;
  w.ml = align256((size_t)Hq * T * gm.S1 * 2 * sizeof(float));
  w.grp = (size_t)Hkv * gm.HG2 * n_vis * sizeof(float);
  w.layer = w.ml + align256(w.grp);
  return w;
}

bool ws_sizes_ok(int layers, int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  return layers >= 1 && T >= 1 && T <= 128 && Hq >= 1 && Hkv >= 1 && Hq % Hkv == 0 && q_pos0 >= 0 && n_vis >= 1 &&
         n_vis <= (1 << 18);
}

}  // namespace
}  // namespace svlm

using namespace svlm;

static size_t score_ws_bytes(int layers, int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  if (!ws_sizes_ok(layers, T, Hq, Hkv, q_pos0, n_vis)) return 0;
  const Geometry gm = geometry(T, Hq, Hkv, q_pos0, n_vis, layers);
  // sizes past 2^60 bytes are refused rather than wrapped
  if (mul_sat(mul_sat(mul_sat(Hq, T), gm.S1), 8) > ((int64_t)1 << 60) ||
      mul_sat(mul_sat(mul_sat(Hkv, gm.HG2), n_vis), 4) > ((int64_t)1 << 60))
    return 0;
  const WsParts w = ws_parts(gm, T, Hq, Hkv, n_vis);
  // the last layer needs no padding after its rows
  const size_t last = w.ml + w.grp;
  if ((size_t)(layers - 1) > (SIZE_MAX - last) / w.layer) return 0;
  return (size_t)(layers - 1) * w.layer + last;
}

extern "C" size_t svlm_score_workspace(int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  return score_ws_bytes(1, T, Hq, Hkv, q_pos0, n_vis);
}

extern "C" size_t svlm_score_layers_workspace(int layers, int T, int Hq, int Hkv, int q_pos0, int n_vis) {
  return score_ws_bytes(layers, T, Hq, Hkv, q_pos0, n_vis);
}

// shared by svlm_score (one layer) and svlm_score_layers
static int score_impl(const char* name, const void* q_text, int64_t q_st, int64_t q_sh, int64_t q_sl, const void* k,
                      int64_t k_sh, int64_t k_sn, int64_t k_sl, int layers, int dtype, int T, int n_ctx, int q_pos0,
                      int vis_start, int n_vis, int Hq, int Hkv, int D, float scale, int agg, int layer_mean,
                      float alpha, float beta, float* out, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != SVLM_BF16 && dtype != SVLM_F32) return fail(SVLM_E_UNSUPPORTED, "%s: unknown dtype %d", name, dtype);
  const int epc = (dtype == SVLM_F32) ? 4 : 8;  // elements per 16 bytes
  if (D != 64 && D != 128) return fail(SVLM_E_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", name, D);
  if (T < 1 || T > 128) return fail(SVLM_E_UNSUPPORTED, "%s: 1 <= T <= 128 text queries supported (got %d)", name, T);
  if (layers < 1) return fail(SVLM_E_INVALID, "%s: layers must be >= 1", name);
  if (!q_text || !k || !out) return fail(SVLM_E_INVALID, "%s: null pointer", name);
  if (Hq < 1 || Hkv < 1 || Hq % Hkv) return fail(SVLM_E_INVALID, "%s: Hq must be a positive multiple of Hkv", name);
  if (n_ctx < 1 || q_pos0 < 0 || (int64_t)q_pos0 + T > n_ctx)
    return fail(SVLM_E_INVALID, "%s: need 0 <= q_pos0 and q_pos0 + T <= n_ctx", name);
  if (n_vis < 1 || n_vis > (1 << 18) || vis_start < 0 || (int64_t)vis_start + n_vis > (int64_t)q_pos0 + 1)
    return fail(SVLM_E_INVALID, "%s: visual range must lie in [0, q_pos0] (every text query sees it)", name);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVLM_E_INVALID, "%s: scale must be finite and > 0", name);
  if (agg != SVLM_AGG_QHEAD && agg != SVLM_AGG_KVHEAD && agg != SVLM_AGG_ALL)
    return fail(SVLM_E_INVALID, "%s: unknown aggregation %d", name, agg);
  if (layer_mean != 0 && layer_mean != 1) return fail(SVLM_E_INVALID, "%s: layer_mean must be 0 or 1", name);
  if (layers == 1) layer_mean = 0;  // the mean of one layer is that layer
  if (layer_mean && agg == SVLM_AGG_QHEAD)
    return fail(SVLM_E_UNSUPPORTED, "%s: the layer mean takes SVLM_AGG_KVHEAD or SVLM_AGG_ALL", name);
  if (!std::isfinite(alpha) || !std::isfinite(beta)) return fail(SVLM_E_INVALID, "%s: alpha, beta must be finite", name);
  if (!aligned16(q_text) || !aligned16(k)) return fail(SVLM_E_INVALID, "%s: q_text and k must be 16-byte aligned", name);
  if (q_st % epc || q_sh % epc || k_sh % epc || k_sn % epc || q_sl % epc || k_sl % epc || k_sn < D || q_st < 0 ||
      q_sh < 0 || k_sh < 0 || q_sl < 0 || k_sl < 0)
    return fail(SVLM_E_INVALID, "%s: strides must be non-negative multiples of 16 bytes, k_sn >= D", name);
  const int out_rows = (agg == SVLM_AGG_QHEAD) ? Hq : (agg == SVLM_AGG_KVHEAD) ? Hkv : 1;
  // the workspace check, after the launch-limit checks of each path
  auto ws_check = [&]() -> int {
    const size_t need = score_ws_bytes(layers, T, Hq, Hkv, q_pos0, n_vis);
    if (need == 0) return fail(SVLM_E_UNSUPPORTED, "%s: the workspace size overflows", name);
    if (!ws || ws_bytes < need)
      return fail(SVLM_E_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", name, need, ws_bytes);
    if (!aligned16(ws)) return fail(SVLM_E_INVALID, "%s: workspace must be 16-byte aligned", name);
    return SVLM_OK;
  };
  hipStream_t st = (hipStream_t)stream;
  if (dtype == SVLM_F32) {
    // plain fp32 path, one layer at a time: row log-sum-exp into the
    // workspace, then the aggregated column means straight into out (the
    // layer mean accumulates through alpha / beta)
    if (!grid_fits((int64_t)Hq * T, 64) || !grid_fits((n_vis + 255) / 256, 256, out_rows))
      return fail(SVLM_E_UNSUPPORTED, "%s: %d heads exceed the launch limit", name, Hq);
    if (const int e = ws_check()) return e;
    for (int l = 0; l < layers; ++l) {
      ScoreF32Args f;
      f.q = (const float*)q_text + l * q_sl;
      f.q_st = q_st;
      f.q_sh = q_sh;
      f.k = (const float*)k + l * k_sl;
      f.k_sh = k_sh;
      f.k_sn = k_sn;
      f.T = T;
      f.q_pos0 = q_pos0;
      f.vis_start = vis_start;
      f.n_vis = n_vis;
      f.Hq = Hq;
      f.Hkv = Hkv;
      f.D = D;
      f.scale = scale;
      f.lse = (float*)ws;
      f.agg = agg;
      f.alpha = layer_mean ? alpha / (float)layers : alpha;
      f.beta = (layer_mean && l > 0) ? 1.f : beta;
      f.out = out + (layer_mean ? 0 : (int64_t)l * out_rows * n_vis);
      launch_score_f32(f, out_rows, st);
    }
    return check_launch(name);
  }
  // buffer-descriptor ranges and offsets are 32-bit: one head's text queries,
  // and one KV head's keys (plus the tiles staged past a split's end)
  if (((int64_t)(T - 1) * q_st + D) * 2 > INT32_MAX || ((int64_t)n_ctx + 1024) * k_sn * 2 > INT32_MAX)
    return fail(SVLM_E_UNSUPPORTED, "%s: (T-1) * q_st + D and (n_ctx + 1024) * k_sn must stay below 2^30 elements", name);
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
  const Geometry gm = geometry(T, Hq, Hkv, q_pos0, n_vis, layers);
  const int64_t blocks1 = pass_blocks(layers, Hkv, gm.S1, gm.HG1), blocks2 = pass_blocks(layers, Hkv, gm.S2, gm.HG2);
  const bool direct = !layer_mean && ((agg == SVLM_AGG_QHEAD) || (agg == SVLM_AGG_KVHEAD && gm.HG2 == 1));
  if (!grid_fits(blocks1, 64 * gm.W1) || !grid_fits(blocks2, 64 * gm.W2) ||
      !grid_fits((n_vis + 255) / 256, 256, mul_sat(layers, out_rows)) || blocks1 > INT32_MAX || blocks2 > INT32_MAX)
    return fail(SVLM_E_UNSUPPORTED, "%s: %d layers of %d heads exceed the launch limit", name, layers, Hq);
  if (const int e = ws_check()) return e;
  a.HG1 = gm.HG1;
  a.HG2 = gm.HG2;
  a.S1 = gm.S1;
  a.kps1 = gm.kps1;
  a.S2 = gm.S2;
  a.kps2 = gm.kps2;
  const WsParts w = ws_parts(gm, T, Hq, Hkv, n_vis);
  a.ml = (float*)ws;
  a.grp = (float*)((char*)ws + w.ml);
  a.agg = agg;
  a.alpha = alpha;
  a.beta = beta;
  a.out = out;
  a.layers = layers;
  a.q_sl = q_sl;
  a.k_sl = k_sl;
  a.ws_sl = (int64_t)(w.layer / sizeof(float));
  a.layer_mean = layer_mean;
  a.rows = out_rows;
  const int rb = pick_rb(T);
  if (use_units(1, D, T, a.G, gm.HG1, gm.W1)) launch_units<1>(a, units_per_wave(T, a.G, gm.HG1, gm.W1), gm.W1, st);
  else if (D == 128) launch_heads<128, 1>(a, rb, gm.W1, st);
  else launch_heads<64, 1>(a, rb, gm.W1, st);
  if (agg != SVLM_AGG_QHEAD && use_units(2, D, T, a.G, gm.HG2, gm.W2))
    launch_units<2>(a, units_per_wave(T, a.G, gm.HG2, gm.W2), gm.W2, st);
  else if (D == 128) launch_heads<128, 2>(a, rb, gm.W2, st);
  else launch_heads<64, 2>(a, rb, gm.W2, st);
  if (layer_mean) {
    score_agg_layers<<<dim3((unsigned)((n_vis + 63) / 64), (unsigned)out_rows), 64 * kAggLanes, 0, st>>>(a);
  } else if (!direct) {
    score_agg<<<dim3((unsigned)((n_vis + 255) / 256), (unsigned)(layers * out_rows)), 256, 0, st>>>(a);
  }
  return check_launch(name);
}

extern "C" int svlm_score(const void* q_text, int64_t q_st, int64_t q_sh, const void* k, int64_t k_sh, int64_t k_sn,
                          int dtype, int T, int n_ctx, int q_pos0, int vis_start, int n_vis, int Hq, int Hkv, int D,
                          float scale, int agg, float alpha, float beta, float* out, void* ws, size_t ws_bytes,
                          void* stream) {
  return score_impl("svlm_score", q_text, q_st, q_sh, 0, k, k_sh, k_sn, 0, 1, dtype, T, n_ctx, q_pos0, vis_start,
                    n_vis, Hq, Hkv, D, scale, agg, 0, alpha, beta, out, ws, ws_bytes, stream);
}

extern "C" int svlm_score_layers(const void* q_text, int64_t q_st, int64_t q_sh, int64_t q_sl, const void* k,
                                 int64_t k_sh, int64_t k_sn, int64_t k_sl, int layers, int dtype, int T, int n_ctx,
                                 int q_pos0, int vis_start, int n_vis, int Hq, int Hkv, int D, float scale, int agg,
                                 int layer_mean, float alpha, float beta, float* out, void* ws, size_t ws_bytes,
                                 void* stream) {
  return score_impl("svlm_score_layers", q_text, q_st, q_sh, q_sl, k, k_sh, k_sn, k_sl, layers, dtype, T, n_ctx,
                    q_pos0, vis_start, n_vis, Hq, Hkv, D, scale, agg, layer_mean, alpha, beta, out, ws, ws_bytes,
                    stream);
}
