// svlm_decode_attn: split-K grouped-query decode attention for gfx950.
//
// Draft mode (nq = 1 over the compacted kept KV) and dense verify mode
// (nq = gamma + 1 over the whole cache, causal among the new tokens) are the
// same kernel: Sparse-to-Dense explainer, technical summary, "decoding
// process" (drafting over the selected KV; one I/O pass over the full KV to
// verify).  Decoding loads the whole KV cache every step and is bound by
// memory bandwidth (SpecVLM technology-transfer listing, section 4).
//
// Design (one wave = 64 lanes; c = lane % 16, g = lane / 16):
//  * a workgroup owns one (batch, KV head, key split) and up to 80 query rows
//    (at D = 128 and short contexts 48; rows = G * nq, row r = i * G + local
//    head), padded to 16-row MFMA blocks; four waves, one workgroup per
//    compute unit;
//  * wave w takes the 16-key blocks 64 j + 16 w of the split, so the waves stay
//    balanced; it stages its own blocks HBM -> LDS with LDS-DMA transfers
//    (range-checked buffer descriptors, nontemporal) through a private ring
//    of NS slots and reads them with LDS loads the compiler does not track,
//    so its only memory waits are the kernel's own static vmcnt waits;
//  * S^T = K Q^T on v_mfma_f32_16x16x32_bf16 with the queries in registers:
//    lane holds 4 keys x 1 row per 16-key block, so row statistics need two
//    cross-lane steps (v_permlane16/32_swap);
//  * online softmax in the exp2 domain with a lazy rescale (the reference
//    maximum moves only when a block exceeds it by more than 2^8);
//  * O^T += V^T P^T on v_mfma_f32_16x16x32_bf16: the scores already sit in the
//    B-operand layout; P enters as bf16 hi + lo halves in the two halves of
//    the contraction (the V operand repeated), so the weights carry ~2^-16
//    relative error at the cost of one instruction; V^T operands come from
//    16-byte V rows by byte permutes;
//  * the four waves merge through LDS in a fixed order, then the workgroup
//    writes either the final fp32 output (one split) or a partial (max, sum,
//    output) that a second kernel merges in split order.  Deterministic.
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <vector>

#include "svlm_internal.h"

namespace svlm {
namespace {

struct AttnArgs {
  const uint16_t* q;
  int64_t q_sb;
  const uint16_t* k;
  const uint16_t* v;
  int64_t kv_sb, kv_sh, kv_sn;
  const int32_t* kv_len;  // key count of (b, h) at kv_len[b * len_sb + h * len_sh]
  int64_t len_sb, len_sh;
  int max_kv_len;
  int batch, nq, Hq, Hkv, G, rows;
  float c;  // scale * log2(e)
  int causal;
  int splits, keys_per_split;
  float* out;
  float* lse;
  float* ws_o;   // [B*Hkv*rows][splits][D]
  float* ws_ml;  // [B*Hkv*rows][splits][2]
  // indexed variant: key position p of (b, h) is cache row kv_idx[b * idx_sb + h * idx_sh + p]
  // of the kv_rows rows at k + b * kv_sb + h * kv_sh (and likewise for v)
  const int32_t* kv_idx;
  int64_t idx_sb, idx_sh;
  int kv_rows;
};

// keys per split when the keys are addressed through an index list (the
// split's indices are staged in LDS)
constexpr int kMaxIdxSplit = 2048;

constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kBlock = 16;                 // keys per wave per step (one MFMA block)
constexpr int kStep = kWaves * kBlock;     // keys per workgroup step
constexpr int kMaxRB = 5;                  // query row blocks per workgroup (80 rows)
// At D = 128 a chunk of more than three row blocks (48 rows) pays for itself
// only at long contexts: two chunks read every K and V row twice, which costs
// HBM bandwidth once a split's keys outgrow its share of the XCD's L2, while
// four or five row blocks make the key loop arithmetic-bound.  Measured at
// 70 rows: 8266 keys 16.6 us in two chunks against 23.0 us in one; 141194
// keys 90 us against 84 us.  At 50 rows and 20842 keys: 29.2 against 26.9 us.
constexpr int kMaxRBShort = 3;
constexpr int kLongContextKeys = 16384;
constexpr float kNegInf = -INFINITY;
constexpr float kRescaleSum = 256.f;  // a lane's 4-key weight sum above this raises the row references

template <int DV>
struct VRaw;
template <>
struct VRaw<8> { typedef u32x4 T; };
template <>
struct VRaw<4> { typedef u32x2 T; };

// Key blocks each wave keeps in flight: 16 KB of K and V per wave (two blocks
// at D = 128, four at D = 64).  Measured on 103 MB verify calls: deeper rings
// (32 KB per wave) queue more requests without raising the rate and end
// slower (28.9 against 28.1 us per call).
#ifndef SVLM_ATTN_RING_KB
#define SVLM_ATTN_RING_KB 16
#endif
template <int D>
constexpr int ring_depth() {
  constexpr int SLOT = 2 * kBlock * D * 2;  // bytes of one staged K + V block
  constexpr int RING = SVLM_ATTN_RING_KB * 1024;
  return (RING / SLOT) < 2 ? 2 : RING / SLOT;
}

// One workgroup = one (batch, KV head, key split, row chunk) with kWaves waves.
// Wave w takes the 16-key blocks k_begin + 64 j + 16 w of the split against
// every query row of the chunk (RB blocks of 16 rows), staging its own blocks
// through a private ring of NS slots in LDS.  The waves' partial states are
// merged through LDS in wave order at the end.
// IDX: the keys are the rows named by an index list (a draft that reads the
// selected rows of the full cache in place, no compact copy); the row
// positions p below are then positions in the list.
template <int D, int RB, int NS, bool IDX>
__global__ __launch_bounds__(64 * kWaves, 1) void attn_splitk(AttnArgs a) {
  constexpr int KK = D / 32;             // 32-wide d chunks of the QK product
  constexpr int DV = D / 16;             // d values per lane in the PV product
  constexpr int RP = RB * 16;
  constexpr int ROWB = D * 2;            // bytes of one K or V row
  constexpr int CH = ROWB / 16;          // 16-byte chunks per row
  constexpr int QB = kBlock * ROWB;      // bytes of one staged K (or V) block
  constexpr int NQ = QB / 1024;          // 1 KB transfers per K (or V) block
  constexpr int TW = 2 * NQ;             // transfers per K+V block
  constexpr int SLOT = 2 * QB;           // one ring slot: K block then V block
  constexpr int OSTRIDE = D + 4;         // fp32 elements per merge-slice row
  static_assert((NS - 1) * TW <= 63 && NS * TW <= 63, "ring depth");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform, kept scalar
  const int c = lane & 15;
  const int g4 = lane >> 4;

  // block id -> (batch, KV head) pair fastest, then split: workgroups go to
  // the eight XCDs round-robin by id, so with 8 (or 4, 2) pairs every split of
  // one pair runs on one XCD, which shares its queries through that XCD's L2
  // and leaves the partials there for the merge launch (mapped the same way)
  const int pairs = a.batch * a.Hkv;
  const int ph = blockIdx.x % pairs;
  const int s = blockIdx.x / pairs;
  const int h = ph % a.Hkv;
  const int b = ph / a.Hkv;
  const int row_base = blockIdx.y * RP;

  const int n_raw = a.kv_len[(int64_t)b * a.len_sb + (int64_t)h * a.len_sh];
  if (threadIdx.x == 0) debug_check(n_raw >= a.nq && n_raw <= a.max_kv_len, SVLM_DBG_KV_LEN);
  const int n_kv = min(max(n_raw, 0), a.max_kv_len);
  const int k_begin = s * a.keys_per_split;
  const int k_end = min(k_begin + a.keys_per_split, n_kv);
  // this wave's blocks: keys k_begin + 64 j + 16 wave, j < n_my
  const int n_my = (k_end > k_begin + kBlock * wave) ? (k_end - k_begin - kBlock * wave + kStep - 1) / kStep : 0;

  // LDS: the waves' staging rings, each reused after its wave's key loop for
  // that wave's merge slice; per-wave row maxima and sums for the merge.
  // slots allocated per wave: the NS that cycle, or more where the wave's
  // merge slice (RP rows of OSTRIDE floats) needs the room after the loop
  // (capped at 128 KB in all; larger row chunks merge in groups of MG row blocks)
  constexpr int NSA_WANT = (RP * OSTRIDE * 4 + SLOT - 1) / SLOT;
  constexpr int NSA_CAP = 128 * 1024 / (kWaves * SLOT);
  constexpr int NSA = NSA_WANT > NS ? (NSA_WANT < NSA_CAP ? NSA_WANT : NSA_CAP) : NS;
  constexpr int MG = (NSA * SLOT / (OSTRIDE * 4)) / 16 < RB ? (NSA * SLOT / (OSTRIDE * 4)) / 16 : RB;
  static_assert(MG >= 1 && (size_t)kWaves * NSA * SLOT <= 144 * 1024, "LDS");
  __shared__ __align__(16) unsigned char lds[(size_t)kWaves * NSA * SLOT];
  __shared__ float sm_m[kWaves][RP];
  __shared__ float sm_l[kWaves][RP];
  unsigned char* my_ring = lds + (size_t)wave * NSA * SLOT;

  // Range-checked buffer descriptors over exactly this split's keys: transfers
  // past k_end deliver zeros without touching memory, so every transfer is
  // issued unconditionally and the wait counts are static.  Indexed keys: the
  // descriptors cover the whole cache of (b, h) and a position past the list
  // (or an index outside the cache) gets an offset past the end, which reads
  // zeros the same way.
  const int64_t row_bytes = a.kv_sn * 2;
  const int n_rows = max(k_end - k_begin, 0);
  const int64_t off0 = (int64_t)b * a.kv_sb + (int64_t)h * a.kv_sh + (IDX ? 0 : (int64_t)k_begin * a.kv_sn);
  const int range = IDX ? (int)(a.kv_rows * row_bytes) : (int)(n_rows * row_bytes);
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + off0), (short)0, range, kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + off0), (short)0, range, kBufferFlags);
  __shared__ int sm_idx[IDX ? kMaxIdxSplit : 1];
  if constexpr (IDX) {
    const int32_t* idx = a.kv_idx + (int64_t)b * a.idx_sb + (int64_t)h * a.idx_sh;
    for (int p = threadIdx.x; p < a.keys_per_split; p += 64 * kWaves) {
      int r = -1;
      if (k_begin + p < k_end) {
        r = idx[k_begin + p];
        debug_check(r >= 0 && r < a.kv_rows, SVLM_DBG_KV_INDEX);
        if (r < 0 || r >= a.kv_rows) r = -1;
      }
      sm_idx[p] = r;
    }
    __syncthreads();
  }

  // Stage block j of this wave (16 K rows, then the same 16 V rows) into ring
  // slot `slot`: transfer i moves 1 KB = 1024 / ROWB rows, 16-byte chunks
  // XOR-swizzled by row (chunk p of row r holds source chunk p ^ (r % CH));
  // lane l lands at slot + 1 KB * i + 16 l.  The per-lane part of each source
  // offset is fixed; the block's first row enters as the scalar offset (or,
  // indexed, each lane's row comes from the staged list).
  // Nontemporal: each byte is read once.
  static_assert(NQ <= 4, "transfers per block");
  int src_lane[4] = {0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int r = i * (1024 / ROWB) + lane / CH;
    const int p = lane % CH;
    src_lane[i] = (IDX ? 0 : r * (int)row_bytes) + ((p ^ (r % CH)) * 16);
  }
  auto stage = [&](int slot, int j) {
    unsigned char* base = my_ring + slot * SLOT;
    int soff = (j * kStep + kBlock * wave) * (int)row_bytes;  // first row of the block, in bytes
    int voff[4] = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NQ; ++i) voff[i] = src_lane[i];
    if constexpr (IDX) {
      soff = 0;
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        const int pos = j * kStep + kBlock * wave + i * (1024 / ROWB) + lane / CH;  // in the split
        const int r = (pos < a.keys_per_split) ? sm_idx[pos] : -1;
        voff[i] = (r >= 0) ? r * (int)row_bytes + src_lane[i] : range;
      }
    }
#pragma unroll
    for (int kv = 0; kv < 2; ++kv)
#pragma unroll
      for (int i = 0; i < NQ; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(kv ? vrs : krs,
                                                 (__attribute__((address_space(3))) void*)(base + kv * QB + i * 1024),
                                                 16, voff[i], soff, 0, kNT);
  };

  // ---- query rows in registers (B operand of S^T = K Q^T): lane (c, g4) holds
  // row c of block rb, d = 32 kk + 8 g4 .. + 7; rows past the chunk read zeros
  const int64_t qbytes = (int64_t)a.nq * a.Hq * D * 2;
  const __amdgpu_buffer_rsrc_t qrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.q + (int64_t)b * a.q_sb), (short)0, (int)qbytes, kBufferFlags);
  u32x4 qreg[RB][KK];
  int lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row_base + rb * 16 + c;
    const bool valid = r < a.rows;
    const int qi = r / a.G;
    const int hl = r - qi * a.G;
    lim[rb] = valid ? min(k_end, a.causal ? n_kv - a.nq + qi + 1 : n_kv) : k_end;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int off = valid ? ((qi * a.Hq + h * a.G + hl) * D + 32 * kk + 8 * g4) * 2 : (int)qbytes;
      qreg[rb][kk] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(qrs, off, 0, 0));
    }
  }
  // keys every row of this workgroup may see: blocks below this need no mask
  const int lim_all = min(k_end, a.causal ? n_kv - a.nq + row_base / a.G + 1 : n_kv);

  // prologue: this wave's blocks 0 .. NS-1 (past the split: zeros)
#pragma unroll
  for (int u = 0; u < NS; ++u) stage(u, u);
  wait_vmcnt<NS * TW>();  // the query loads, issued first, have landed

  // LDS byte offsets of this lane's operand chunks within a slot:
  //   K (A of S^T): row c, chunk 4 kk + g4;  V (for A of O^T): rows 4 g4 + i, d 8 c (or 4 c)
  unsigned koff[KK], voff[4];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) koff[kk] = c * ROWB + (((kk * 4 + g4) ^ (c % CH)) * 16);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 4 * g4 + i;
    if constexpr (D == 128) voff[i] = QB + r * ROWB + ((c ^ (r % CH)) * 16);
    else voff[i] = QB + r * ROWB + (((c >> 1) ^ (r % CH)) * 16) + (c & 1) * 8;
  }
  const unsigned ring0 = lds_addr(my_ring);

  // Running state per row (lane row c + 16 rb, uniform over the four lane
  // groups): m_use is the reference maximum in log2 units, raised only when
  // some lane's 4-key weight sum passes kRescaleSum, so single weights stay
  // <= 2^8 and the fp32 accumulators are rescaled only rarely.
  float m_use[RB], l_run[RB];
  f32x4 o[DV][RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_use[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < DV; ++mb) o[mb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One 16-key block of this wave.  `masked` blocks reach some row's causal
  // or split limit and mask per key; the others (all but the last one or two
  // of a split) skip the per-key tests.
  auto block = [&](int j, bool masked) {
    const int slot = j % NS;
    // block j has landed once the NS - 1 younger blocks are all that is outstanding
    wait_vmcnt<(NS - 1) * TW>();
    const unsigned base = ring0 + (unsigned)(slot * SLOT);
    u32x4 kq[KK];
    typename VRaw<DV>::T vt[4];
    if constexpr (D == 128) {
      unsigned ad[8];
      u32x4 rd[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) ad[e] = base + koff[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) ad[4 + e] = base + voff[e];
      lds_read_b128x8(rd, ad);
#pragma unroll
      for (int e = 0; e < 4; ++e) kq[e] = rd[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[e] = __builtin_bit_cast(typename VRaw<DV>::T, rd[4 + e]);
    } else {
      unsigned ad[6];
      u32x4 kd[2];
      u32x2 vd[4];
#pragma unroll
      for (int e = 0; e < 2; ++e) ad[e] = base + koff[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) ad[2 + e] = base + voff[e];
      lds_read_b128x2_b64x4(kd, vd, ad);
#pragma unroll
      for (int e = 0; e < 2; ++e) kq[e] = kd[e];
#pragma unroll
      for (int e = 0; e < 4; ++e) vt[e] = __builtin_bit_cast(typename VRaw<DV>::T, vd[e]);
    }
    stage(slot, j + NS);  // refill the slot just read (past the split: zeros)

    // S^T block: lane holds keys key0 + 4 g4 + i of row c + 16 rb
    const int key0 = k_begin + j * kStep + kBlock * wave;
    f32x4 sacc[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) sacc[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[rb] = mfma16(as_bf16x8(kq[kk]), as_bf16x8(qreg[rb][kk]), sacc[rb]);

    // weights against each row's reference.  A lane's 4-key sum exceeds
    // kRescaleSum (or is inf / NaN: no reference yet) only when one of its
    // scores passes the reference by about 6 (log2 units); then, for the whole
    // wave, every row's reference is raised to its block maximum, the
    // accumulators are rescaled and the weights recomputed.  Row maxima are
    // taken only on that rare path.
    float x[RB][4], p[RB][4], s4[RB];
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        x[rb][i] = (!masked || key0 + 4 * g4 + i < lim[rb]) ? sacc[rb][i] : kNegInf;
        p[rb][i] = fast_exp2(fmaf(x[rb][i], a.c, -m_use[rb]));
      }
      s4[rb] = (p[rb][0] + p[rb][1]) + (p[rb][2] + p[rb][3]);
      grow |= !(s4[rb] <= kRescaleSum);
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m = fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3]));
        const float mx = max_xor32(max_xor16(m)) * a.c;  // raw scores -> log2 units (c > 0 keeps the order)
        const float m_new = fmaxf(m_use[rb], mx);
        const float alpha = (m_use[rb] == kNegInf) ? 0.f : fast_exp2(m_use[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < DV; ++mb) o[mb][rb] *= alpha;
        m_use[rb] = m_new;
        const float mneg = (m_new == kNegInf) ? 0.f : -m_new;
#pragma unroll
        for (int i = 0; i < 4; ++i) p[rb][i] = fast_exp2(fmaf(x[rb][i], a.c, mneg));
        s4[rb] = (p[rb][0] + p[rb][1]) + (p[rb][2] + p[rb][3]);
      }
    }
    // P^T as the B operand of the V product: lane (c, g4) holds
    // P[row c][keys 4 g4 .. 4 g4 + 3] exactly where the scores are, as bf16
    // hi + lo halves: the lane's eight contraction slots of one
    // v_mfma_f32_16x16x32_bf16 take the four hi halves, then the four lo
    // halves, and the A operand repeats the same four V values in both, so one
    // instruction (issuing at the rate of the 16x16x16 form) adds V (hi + lo)
    bf16x8 pp[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l_run[rb] += s4[rb];
      u32x4 hl;
#pragma unroll
      for (int qd = 0; qd < 2; ++qd) {
        const unsigned b0 = f_bits(p[rb][2 * qd]), b1 = f_bits(p[rb][2 * qd + 1]);
        hl[qd] = perm(b1, b0, kPermHi);
        const float r0 = p[rb][2 * qd] - bits_f(b0 & 0xFFFF0000u);
        const float r1 = p[rb][2 * qd + 1] - bits_f(b1 & 0xFFFF0000u);
        hl[2 + qd] = perm(f_bits(r1), f_bits(r0), kPermHi);
      }
      pp[rb] = as_bf16x8(hl);
    }
    // O^T += V^T P^T: the A operand of d-block mb holds V[keys 4 g4 .. + 3][d = DV c + mb], twice
#pragma unroll
    for (int mb = 0; mb < DV; ++mb) {
      const int w = mb >> 1;
      const unsigned sel = (mb & 1) ? kPermHi : kPermLo;
      u32x4 vv;
      vv[0] = perm(vt[1][w], vt[0][w], sel);
      vv[1] = perm(vt[3][w], vt[2][w], sel);
      vv[2] = vv[0];
      vv[3] = vv[1];
      const bf16x8 vop = as_bf16x8(vv);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) o[mb][rb] = mfma16(vop, pp[rb], o[mb][rb]);
    }
  };
  // blocks below n_full see every key of every row
  const int full_span = lim_all - k_begin - kBlock * wave - kBlock;  // block j is full iff kStep * j <= full_span
  const int n_full = min(n_my, full_span >= 0 ? full_span / kStep + 1 : 0);
  int jb = 0;
  for (; jb < n_full; ++jb) block(jb, false);
  for (; jb < n_my; ++jb) block(jb, true);
  wait_vmcnt<0>();  // the zero-filled transfers past the end land before the ring is reused

  // ---- merge the waves: each parks its row maxima, row sums and unscaled
  // output sums in a slice inside its own staging ring (which only it has
  // used), so no wave waits for another before writing; after one barrier
  // every thread weights and adds the slices of its (row, 4 columns) items in
  // wave order and writes them with coalesced stores.  All LDS loads of a
  // thread are issued together.  Up to 48 rows (three row blocks at D = 128)
  // merge in one pass; larger chunks in groups of MG row blocks, with a
  // barrier between groups.  (The one-pass form is kept as written for the
  // chunks it covers: the grouped form, compiled for them, measured 1.4 us
  // slower per dense-verify call at the 72B shape.)
  if constexpr (MG >= RB) {
    {
      float* my_slice = (float*)my_ring;
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        l_run[rb] = sum_xor32(sum_xor16(l_run[rb]));
        const int row = rb * 16 + c;
        if (g4 == 0) {
          sm_m[wave][row] = m_use[rb];
          sm_l[wave][row] = l_run[rb];
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int mb = 0; mb < DV; mb += 4)
            *(float4*)(my_slice + row * OSTRIDE + DV * (4 * g4 + i) + mb) =
                make_float4(o[mb][rb][i], o[mb + 1][rb][i], o[mb + 2][rb][i], o[mb + 3][rb][i]);
      }
    }
    __syncthreads();  // every wave's slice and row state are in LDS
    constexpr int C4 = D / 4;
    constexpr int ITEMS = (RP * C4 + 64 * kWaves - 1) / (64 * kWaves);
    float4 part[ITEMS][kWaves];
    float pm[ITEMS][kWaves], pl[ITEMS][kWaves];
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int e = min((int)threadIdx.x + k * 64 * kWaves, RP * C4 - 1);
      const int row = e / C4, d4 = e - row * C4;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        part[k][w] = *(const float4*)((const float*)(lds + (size_t)w * NSA * SLOT) + row * OSTRIDE + 4 * d4);
        pm[k][w] = sm_m[w][row];
        pl[k][w] = sm_l[w][row];
      }
    }
#pragma unroll
    for (int k = 0; k < ITEMS; ++k) {
      const int e = threadIdx.x + k * 64 * kWaves;
      if (e >= RP * C4) break;
      const int row = e / C4, d4 = e - row * C4;
      const int r = row_base + row;
      if (r >= a.rows) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) M = fmaxf(M, pm[k][w]);
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float f = (pm[k][w] == kNegInf) ? 0.f : fast_exp2(pm[k][w] - M);
        L += f * pl[k][w];
        acc.x += f * part[k][w].x;
        acc.y += f * part[k][w].y;
        acc.z += f * part[k][w].z;
        acc.w += f * part[k][w].w;
      }
      const int qi = r / a.G;
      const int hl = r - qi * a.G;
      if (a.splits == 1) {
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        const int64_t orow = ((int64_t)b * a.nq + qi) * a.Hq + (int64_t)h * a.G + hl;
        *(float4*)(a.out + orow * D + 4 * d4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
        if (a.lse && d4 == 0) a.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
      } else {
        const int64_t R = ((int64_t)b * a.Hkv + h) * a.rows + r;
        *(float4*)(a.ws_o + (R * a.splits + s) * D + 4 * d4) = acc;
        if (d4 == 0) *(float2*)(a.ws_ml + (R * a.splits + s) * 2) = make_float2(M, L);
      }
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      l_run[rb] = sum_xor32(sum_xor16(l_run[rb]));
      if (g4 == 0) {
        sm_m[wave][rb * 16 + c] = m_use[rb];
        sm_l[wave][rb * 16 + c] = l_run[rb];
      }
    }
    constexpr int C4 = D / 4;
    constexpr int GROWS = MG * 16;  // rows per merge group
    constexpr int ITEMS = (GROWS * C4 + 64 * kWaves - 1) / (64 * kWaves);
#pragma unroll
    for (int gb = 0; gb < RB; gb += MG) {
      if (gb > 0) __syncthreads();  // the previous group's slices have been read
      {
        float* my_slice = (float*)my_ring;
#pragma unroll
        for (int rb = gb; rb < gb + MG && rb < RB; ++rb) {
          const int row = (rb - gb) * 16 + c;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int mb = 0; mb < DV; mb += 4)
              *(float4*)(my_slice + row * OSTRIDE + DV * (4 * g4 + i) + mb) =
                  make_float4(o[mb][rb][i], o[mb + 1][rb][i], o[mb + 2][rb][i], o[mb + 3][rb][i]);
        }
      }
      __syncthreads();  // every wave's slice and row state are in LDS
      const int grows = min(GROWS, RP - gb * 16);  // rows of this group
      float4 part[ITEMS][kWaves];
      float pm[ITEMS][kWaves], pl[ITEMS][kWaves];
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) {
        const int e = min((int)threadIdx.x + k * 64 * kWaves, grows * C4 - 1);
        const int row = e / C4, d4 = e - row * C4;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          part[k][w] = *(const float4*)((const float*)(lds + (size_t)w * NSA * SLOT) + row * OSTRIDE + 4 * d4);
          pm[k][w] = sm_m[w][gb * 16 + row];
          pl[k][w] = sm_l[w][gb * 16 + row];
        }
      }
#pragma unroll
      for (int k = 0; k < ITEMS; ++k) {
        const int e = threadIdx.x + k * 64 * kWaves;
        if (e >= grows * C4) break;
        const int row = e / C4, d4 = e - row * C4;
        const int r = row_base + gb * 16 + row;
        if (r >= a.rows) continue;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, pm[k][w]);
        float L = 0.f;
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          const float f = (pm[k][w] == kNegInf) ? 0.f : fast_exp2(pm[k][w] - M);
          L += f * pl[k][w];
          acc.x += f * part[k][w].x;
          acc.y += f * part[k][w].y;
          acc.z += f * part[k][w].z;
          acc.w += f * part[k][w].w;
        }
        const int qi = r / a.G;
        const int hl = r - qi * a.G;
        if (a.splits == 1) {
          const float inv = (L > 0.f) ? 1.f / L : 0.f;
          const int64_t orow = ((int64_t)b * a.nq + qi) * a.Hq + (int64_t)h * a.G + hl;
          *(float4*)(a.out + orow * D + 4 * d4) = make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
          if (a.lse && d4 == 0) a.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
        } else {
          const int64_t R = ((int64_t)b * a.Hkv + h) * a.rows + r;
          *(float4*)(a.ws_o + (R * a.splits + s) * D + 4 * d4) = acc;
          if (d4 == 0) *(float2*)(a.ws_ml + (R * a.splits + s) * 2) = make_float2(M, L);
        }
      }
    }
  }
}

// Merge launch: kCombineRows rows per workgroup, 128 threads per row = D/4
// column groups x (512/D) split parts.  With at most SPAN splits per part, a
// thread loads all of its (max, sum, output) partials at once — one memory
// round trip — and merges them in split order; SPAN = 0 takes any number, in
// batches of kCombineSpan, one round trip each.
// The parts are then combined in a fixed order through LDS.  Deterministic.
constexpr int kCombineRows = 2;
constexpr int kCombineSpan = 8;
template <int D, int SPAN>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  constexpr int C4 = D / 4;
  constexpr int PARTS = 128 / C4;
  __shared__ float4 s_acc[256];
  __shared__ float2 s_ml[256];
  const int t = threadIdx.x;
  // block id -> (batch, KV head) pair fastest, as in the split kernel, then
  // kCombineRows rows of that pair
  const int pairs = a.batch * a.Hkv;
  const int r_in = (int)(blockIdx.x / pairs) * kCombineRows + t / 128;
  const bool valid = r_in < a.rows;
  const int64_t R = (int64_t)(blockIdx.x % pairs) * a.rows + r_in;  // (b * Hkv + h) * rows + r
  const int d4 = (t & 127) % C4, part = (t & 127) / C4;
  const int S = a.splits;
  const int span = (S + PARTS - 1) / PARTS;
  const int s_lo = min(S, part * span), s_hi = min(S, s_lo + span);
  float M = kNegInf, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (valid) {
    const float2* ml = (const float2*)a.ws_ml + R * S;
    const float4* po = (const float4*)(a.ws_o + R * S * D) + d4;
    if constexpr (SPAN > 0) {
      float2 st[SPAN];
      float4 v[SPAN];
#pragma unroll
      for (int i = 0; i < SPAN; ++i) {
        const int sp = s_lo + i;
        st[i] = (sp < s_hi) ? ml[sp] : make_float2(kNegInf, 0.f);
        v[i] = (sp < s_hi) ? po[(int64_t)sp * C4] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int i = 0; i < SPAN; ++i) M = fmaxf(M, st[i].x);
      if (M != kNegInf) {
#pragma unroll
        for (int i = 0; i < SPAN; ++i) {
          const float w = (st[i].x == kNegInf) ? 0.f : exp2f(st[i].x - M);
          L += w * st[i].y;
          acc.x += w * v[i].x;
          acc.y += w * v[i].y;
          acc.z += w * v[i].z;
          acc.w += w * v[i].w;
        }
      }
    } else {
      // batches of kCombineSpan partials, each loaded at once and joined to
      // the running (M, L, acc): the batch's largest maximum first, then
      // every partial weighed against the new reference
      for (int s0 = s_lo; s0 < s_hi; s0 += kCombineSpan) {
        float2 st[kCombineSpan];
        float4 v[kCombineSpan];
#pragma unroll
        for (int i = 0; i < kCombineSpan; ++i) {
          const int sp = s0 + i;
          st[i] = (sp < s_hi) ? ml[sp] : make_float2(kNegInf, 0.f);
          v[i] = (sp < s_hi) ? po[(int64_t)sp * C4] : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        float bm = kNegInf;
#pragma unroll
        for (int i = 0; i < kCombineSpan; ++i) bm = fmaxf(bm, st[i].x);
        const float m_new = fmaxf(M, bm);
        if (m_new == kNegInf) continue;
        const float f = (M == kNegInf) ? 0.f : exp2f(M - m_new);
        L *= f;
        acc.x *= f;
        acc.y *= f;
        acc.z *= f;
        acc.w *= f;
#pragma unroll
        for (int i = 0; i < kCombineSpan; ++i) {
          const float w = (st[i].x == kNegInf) ? 0.f : exp2f(st[i].x - m_new);
          L += w * st[i].y;
          acc.x += w * v[i].x;
          acc.y += w * v[i].y;
          acc.z += w * v[i].z;
          acc.w += w * v[i].w;
        }
        M = m_new;
      }
    }
  }
  s_acc[t] = acc;
  s_ml[t] = make_float2(M, L);
  __syncthreads();
  if (!valid || part != 0) return;
  float Mt = kNegInf;
  for (int p = 0; p < PARTS; ++p) Mt = fmaxf(Mt, s_ml[t + p * C4].x);
  float Lt = 0.f;
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  if (Mt != kNegInf) {
    for (int p = 0; p < PARTS; ++p) {
      const float2 st = s_ml[t + p * C4];
      const float w = (st.x == kNegInf) ? 0.f : exp2f(st.x - Mt);
      const float4 v = s_acc[t + p * C4];
      Lt += w * st.y;
      o.x += w * v.x;
      o.y += w * v.y;
      o.z += w * v.z;
      o.w += w * v.w;
    }
  }
  const int r = (int)(R % a.rows);
  const int64_t bh = R / a.rows;
  const int h = (int)(bh % a.Hkv), b = (int)(bh / a.Hkv);
  const int qi = r / a.G, hl = r - qi * a.G;
  const int64_t orow = ((int64_t)b * a.nq + qi) * a.Hq + (int64_t)h * a.G + hl;
  const float inv = (Lt > 0.f) ? 1.f / Lt : 0.f;
  *(float4*)(a.out + orow * D + 4 * d4) = make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  if (a.lse && d4 == 0) a.lse[orow] = (Lt > 0.f) ? (Mt + log2f(Lt)) * kLn2 : kNegInf;
}

template <int D>
void launch_combine(const AttnArgs& a, int batch, hipStream_t st) {
  constexpr int PARTS = 128 / (D / 4);
  const unsigned blocks = (unsigned)((int64_t)batch * a.Hkv * ((a.rows + kCombineRows - 1) / kCombineRows));
  if ((a.splits + PARTS - 1) / PARTS <= kCombineSpan) attn_combine<D, kCombineSpan><<<blocks, 256, 0, st>>>(a);
  else attn_combine<D, 0><<<blocks, 256, 0, st>>>(a);
}

template <int D, int RB>
void launch_rb(const AttnArgs& a, int batch, int row_chunks, hipStream_t st) {
  dim3 grid((unsigned)((int64_t)batch * a.Hkv * a.splits), (unsigned)row_chunks);
  if (a.kv_idx) attn_splitk<D, RB, ring_depth<D>(), true><<<grid, 64 * kWaves, 0, st>>>(a);
  else attn_splitk<D, RB, ring_depth<D>(), false><<<grid, 64 * kWaves, 0, st>>>(a);
}

template <int D>
void launch_d(const AttnArgs& a, int rb, int batch, int row_chunks, hipStream_t st) {
  switch (rb) {
    case 1: launch_rb<D, 1>(a, batch, row_chunks, st); break;
    case 2: launch_rb<D, 2>(a, batch, row_chunks, st); break;
    case 3: launch_rb<D, 3>(a, batch, row_chunks, st); break;
    case 4: launch_rb<D, 4>(a, batch, row_chunks, st); break;
    default: launch_rb<D, 5>(a, batch, row_chunks, st); break;
  }
}

struct Plan {
  int64_t rb, row_chunks, splits, keys_per_split;
};

// SVLM_NUM_SPLITS in the environment (a positive integer) replaces the
// planner's split count for calls that leave it to the library
// (num_splits = 0); read once per process.  0 when unset or invalid.
int env_num_splits() {
  static const int v = [] {
    const char* e = std::getenv("SVLM_NUM_SPLITS");
    if (!e || !*e) return 0;
    char* end = nullptr;
    const long n = std::strtol(e, &end, 10);
    return (*end == 0 && n > 0 && n <= (1L << 20)) ? (int)n : 0;
  }();
  return v;
}

// max_steps_per_split > 0 caps the split length (indexed keys: the split's
// list is staged in LDS).  64-bit throughout: the workspace queries take any
// int sizes, and plan_fits() decides what can be launched.
Plan make_plan(int batch, int nq, int Hq, int Hkv, int D, int max_kv_len, int num_splits,
               int max_steps_per_split = 0) {
  Plan p;
  const int64_t rows = (int64_t)(Hq / Hkv) * nq;
  const int64_t max_rb = (D == 128 && max_kv_len < kLongContextKeys) ? kMaxRBShort : kMaxRB;
  // row blocks per chunk: as few chunks as possible, then as few padded rows
  const int64_t chunks = (rows + max_rb * 16 - 1) / (max_rb * 16);
  p.rb = ((rows + chunks - 1) / chunks + 15) / 16;
  p.row_chunks = (rows + p.rb * 16 - 1) / (p.rb * 16);
  const int64_t steps = ((int64_t)max_kv_len + kStep - 1) / kStep;
  int64_t splits = num_splits > 0 ? num_splits : env_num_splits();
  if (splits <= 0) {
    // Workgroups for about seven eighths of the compute units: the key loop
    // is bound by HBM bandwidth before every unit is busy, each extra split
    // adds partial state for the merge, and one workgroup past the chip
    // (one per CU) starts a second round.  Short key ranges split down to one
    // step per workgroup: against a two-step minimum, the hour-long in-place
    // draft (1089 keys per head) took 8.9 against 9.1 us and the 7B draft
    // (885 keys) 7.5 against 7.6 us; longer ranges do not reach it.
    const int64_t units = std::max<int64_t>(1, mul_sat(mul_sat(batch, Hkv), p.row_chunks));
    splits = std::max<int64_t>(1, (7 * num_cus() / 8 + units - 1) / units);
  }
  splits = std::max<int64_t>(1, std::min(splits, steps));
  if (max_steps_per_split > 0) splits = std::max(splits, (steps + max_steps_per_split - 1) / max_steps_per_split);
  const int64_t steps_per_split = (steps + splits - 1) / splits;
  p.keys_per_split = steps_per_split * kStep;
  p.splits = ((int64_t)max_kv_len + p.keys_per_split - 1) / p.keys_per_split;
  return p;
}

// the split-K pass and the merge both fit the dispatch limits
bool plan_fits(const Plan& p, int batch, int Hq, int Hkv, int nq) {
  const int64_t rows = (int64_t)(Hq / Hkv) * nq;
  const int64_t units = mul_sat(batch, Hkv);
  return grid_fits(mul_sat(units, p.splits), 64 * kWaves, p.row_chunks) &&
         (p.splits <= 1 || grid_fits(mul_sat(units, (rows + kCombineRows - 1) / kCombineRows), 256));
}

// Workspace layout: the partial outputs, then the partial (max, sum) pairs.
struct WsLayout {
  size_t o_off, ml_off, total;
};
WsLayout ws_layout(const Plan& p, int batch, int Hq, int nq, int D) {
  WsLayout w{};
  if (p.splits <= 1) return w;
  const size_t rows_total = (size_t)batch * Hq * nq;
  w.o_off = 0;
  w.ml_off = w.o_off + rows_total * p.splits * D * sizeof(float);
  w.total = w.ml_off + rows_total * p.splits * 2 * sizeof(float);
  return w;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

namespace {
constexpr int kIdxMaxSteps = kMaxIdxSplit / kStep;

// shared by the contiguous and the indexed entry points; kv_idx == nullptr
// means keys are rows 0 .. kv_len - 1 of the cache
int decode_attn_impl(const char* name, const void* q, int64_t q_sb, const void* k, const void* v, int64_t kv_sb,
                     int64_t kv_sh, int64_t kv_sn, const int32_t* kv_idx, int64_t idx_sb, int64_t idx_sh,
                     int kv_rows, const int32_t* kv_len, int64_t len_sb, int64_t len_sh, int max_kv_len, int dtype,
                     int batch, int nq, int Hq, int Hkv, int D, float scale, int causal_tail, float* out, float* lse,
                     int num_splits, void* ws, size_t ws_bytes, void* stream) {
  if (dtype != SVLM_BF16 && dtype != SVLM_F32) return fail(SVLM_E_UNSUPPORTED, "%s: unknown dtype %d", name, dtype);
  if (D != 64 && D != 128) return fail(SVLM_E_UNSUPPORTED, "%s: D must be 64 or 128 (got %d)", name, D);
  const int epc = (dtype == SVLM_F32) ? 4 : 8;  // elements per 16 bytes
  if (!q || !k || !v || !kv_len || !out) return fail(SVLM_E_INVALID, "%s: null pointer", name);
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || max_kv_len < 1)
    return fail(SVLM_E_INVALID, "%s: batch, nq, Hq, Hkv and the key count bound must be >= 1", name);
  if (Hq % Hkv) return fail(SVLM_E_INVALID, "%s: Hq (%d) must be a multiple of Hkv (%d)", name, Hq, Hkv);
  // one batch entry's queries span a 32-bit buffer range
  if ((int64_t)nq * Hq > INT32_MAX / (2 * D))
    return fail(SVLM_E_UNSUPPORTED, "%s: nq * Hq * D * 2 must be below 2^31", name);
  if (causal_tail != 0 && causal_tail != 1) return fail(SVLM_E_INVALID, "%s: causal_tail must be 0 or 1", name);
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(SVLM_E_INVALID, "%s: scale must be finite and > 0", name);
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(SVLM_E_INVALID, "%s: q, k, v, out must be 16-byte aligned", name);
  if (kv_sn < D || kv_sn % epc || kv_sh % epc || kv_sb % epc || kv_sh < 0 || kv_sb < 0)
    return fail(SVLM_E_INVALID, "%s: KV strides must be multiples of 16 bytes with kv_sn >= D", name);
  if (q_sb % epc || (batch > 1 && q_sb < (int64_t)nq * Hq * D))
    return fail(SVLM_E_INVALID, "%s: q batch stride must be a multiple of 16 bytes and >= nq*Hq*D", name);
  if (num_splits < 0) return fail(SVLM_E_INVALID, "%s: num_splits must be >= 0", name);
  if (len_sb < 0 || len_sh < 0) return fail(SVLM_E_INVALID, "%s: length strides must be >= 0", name);
  if (kv_idx) {
    if (kv_rows < 1 || (dtype == SVLM_BF16 && (int64_t)kv_rows * kv_sn * 2 > INT32_MAX))
      return fail(SVLM_E_INVALID, "%s: kv_rows must be >= 1 with kv_rows * kv_sn * 2 < 2^31", name);
    if (idx_sb < 0 || idx_sh < 0) return fail(SVLM_E_INVALID, "%s: index strides must be >= 0", name);
  }
  if (dtype == SVLM_F32) {
    // plain fp32 rows, one wave each; no split state, so no workspace
    if (!grid_fits((int64_t)batch * nq * Hq, 64))
      return fail(SVLM_E_UNSUPPORTED, "%s: batch * nq * Hq output rows exceed the launch limit", name);
    AttnF32Args f;
    f.q = (const float*)q;
    f.q_sb = q_sb;
    f.k = (const float*)k;
    f.v = (const float*)v;
    f.kv_sb = kv_sb;
    f.kv_sh = kv_sh;
    f.kv_sn = kv_sn;
    f.kv_len = kv_len;
    f.len_sb = len_sb;
    f.len_sh = len_sh;
    f.max_kv_len = max_kv_len;
    f.kv_idx = kv_idx;
    f.idx_sb = idx_sb;
    f.idx_sh = idx_sh;
    f.kv_rows = kv_rows;
    f.batch = batch;
    f.nq = nq;
    f.Hq = Hq;
    f.Hkv = Hkv;
    f.D = D;
    f.scale = scale;
    f.causal = causal_tail;
    f.out = out;
    f.lse = lse;
    launch_attn_f32(f, (hipStream_t)stream);
    return check_launch(name);
  }
  // buffer-descriptor ranges and offsets are 32-bit: one split's keys (plus
  // the blocks staged past its end)
  const Plan p = make_plan(batch, nq, Hq, Hkv, D, max_kv_len, num_splits, kv_idx ? kIdxMaxSteps : 0);
  if (!plan_fits(p, batch, Hq, Hkv, nq))
    return fail(SVLM_E_UNSUPPORTED, "%s: %lld splits for %d sequences x %d KV heads exceed the launch limit", name,
                (long long)p.splits, batch, Hkv);
  if (!kv_idx && (p.keys_per_split + 8 * kStep) * kv_sn * 2 > INT32_MAX)
    return fail(SVLM_E_UNSUPPORTED, "%s: one key split spans %lld rows of %lld bytes; must stay below 2^31 bytes",
                name, (long long)p.keys_per_split, (long long)(kv_sn * 2));
  const size_t need = ws_layout(p, batch, Hq, nq, D).total;
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(SVLM_E_WORKSPACE, "%s: workspace of %zu bytes needed (got %zu)", name, need, ws_bytes);
  if (need > 0 && !aligned16(ws)) return fail(SVLM_E_INVALID, "%s: workspace must be 16-byte aligned", name);

  AttnArgs a;
  a.q = (const uint16_t*)q;
  a.q_sb = q_sb;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kv_sb = kv_sb;
  a.kv_sh = kv_sh;
  a.kv_sn = kv_sn;
  a.kv_len = kv_len;
  a.len_sb = len_sb;
  a.len_sh = len_sh;
  a.max_kv_len = max_kv_len;
  a.batch = batch;
  a.nq = nq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.rows = a.G * nq;
  a.c = scale * kLog2e;
  a.causal = causal_tail;
  a.splits = (int)p.splits;
  a.keys_per_split = (int)p.keys_per_split;
  a.out = out;
  a.lse = lse;
  a.kv_idx = kv_idx;
  a.idx_sb = idx_sb;
  a.idx_sh = idx_sh;
  a.kv_rows = kv_rows;
  const WsLayout wl = ws_layout(p, batch, Hq, nq, D);
  a.ws_o = ws ? (float*)((char*)ws + wl.o_off) : nullptr;
  a.ws_ml = ws ? (float*)((char*)ws + wl.ml_off) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (D == 128) launch_d<128>(a, (int)p.rb, batch, (int)p.row_chunks, st);
  else launch_d<64>(a, (int)p.rb, batch, (int)p.row_chunks, st);
  if (p.splits > 1) {
    if (D == 128) launch_combine<128>(a, batch, st);
    else launch_combine<64>(a, batch, st);
  }
  return check_launch(name);
}
}  // namespace

extern "C" size_t svlm_decode_attn_workspace(int batch, int nq, int Hq, int Hkv, int D, int max_kv_len,
                                             int num_splits) {
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || max_kv_len < 1) return 0;
  if ((int64_t)nq * Hq > INT32_MAX / (2 * D)) return 0;  // refused by the call
  const Plan p = make_plan(batch, nq, Hq, Hkv, D, max_kv_len, num_splits);
  if (!plan_fits(p, batch, Hq, Hkv, nq)) return 0;
  return ws_layout(p, batch, Hq, nq, D).total;
}

extern "C" int svlm_decode_attn(const void* q, int64_t q_sb, const void* k, const void* v, int64_t kv_sb,
                                int64_t kv_sh, int64_t kv_sn, const int32_t* kv_len, int max_kv_len, int dtype,
                                int batch, int nq, int Hq, int Hkv, int D, float scale, int causal_tail,
                                float* out, float* lse, int num_splits, void* ws, size_t ws_bytes,
                                void* stream) {
  return decode_attn_impl("svlm_decode_attn", q, q_sb, k, v, kv_sb, kv_sh, kv_sn, nullptr, 0, 0, 0, kv_len, 1, 0,
                          max_kv_len, dtype, batch, nq, Hq, Hkv, D, scale, causal_tail, out, lse, num_splits, ws,
                          ws_bytes, stream);
}

extern "C" size_t svlm_decode_attn_indexed_workspace(int batch, int nq, int Hq, int Hkv, int D, int max_n_idx,
                                                     int num_splits) {
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || max_n_idx < 1) return 0;
  if ((int64_t)nq * Hq > INT32_MAX / (2 * D)) return 0;
  const Plan p = make_plan(batch, nq, Hq, Hkv, D, max_n_idx, num_splits, kIdxMaxSteps);
  if (!plan_fits(p, batch, Hq, Hkv, nq)) return 0;
  return ws_layout(p, batch, Hq, nq, D).total;
}

extern "C" int svlm_decode_attn_indexed(const void* q, int64_t q_sb, const void* k, const void* v, int64_t kv_sb,
                                        int64_t kv_sh, int64_t kv_sn, int kv_rows, const int32_t* kv_idx,
                                        int64_t idx_sb, int64_t idx_sh, const int32_t* n_idx, int64_t n_sb,
                                        int64_t n_sh, int max_n_idx, int dtype, int batch, int nq, int Hq, int Hkv, int D, float scale,
                                        int causal_tail, float* out, float* lse, int num_splits, void* ws,
                                        size_t ws_bytes, void* stream) {
  if (!kv_idx) return fail(SVLM_E_INVALID, "svlm_decode_attn_indexed: null index list");
  return decode_attn_impl("svlm_decode_attn_indexed", q, q_sb, k, v, kv_sb, kv_sh, kv_sn, kv_idx, idx_sb, idx_sh,
                          kv_rows, n_idx, n_sb, n_sh, max_n_idx, dtype, batch, nq, Hq, Hkv, D, scale, causal_tail, out, lse,
                          num_splits, ws, ws_bytes, stream);
}

// ---------------------------------------------------------------------------
// svlm_decode_attn_noalloc: svlm_decode_attn with the split-K partial state in
// a static device array instead of a caller workspace, for callers that
// cannot allocate (graph capture, serving loops).  Each device holds its own
// copy of the array; its address is looked up once per device.
// ---------------------------------------------------------------------------
namespace {
constexpr size_t kScratchBytes = (size_t)SVLM_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::vector<void*> g_scratch_ptr;  // per device: the device address of `scratch`

int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SVLM_E_HIP, "svlm_decode_attn_noalloc: hipGetDevice: %s", hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if ((int)g_scratch_ptr.size() <= dev) g_scratch_ptr.resize(dev + 1, nullptr);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(SVLM_E_HIP, "svlm_decode_attn_noalloc: hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return SVLM_OK;
}
}  // namespace

extern "C" int svlm_decode_attn_noalloc(const void* q, int64_t q_sb, const void* k, const void* v, int64_t kv_sb,
                                        int64_t kv_sh, int64_t kv_sn, const int32_t* kv_len, int max_kv_len,
                                        int dtype, int batch, int nq, int Hq, int Hkv, int D, float scale,
                                        int causal_tail, float* out, float* lse, int num_splits, void* stream) {
  size_t need = 0;
  if (dtype == SVLM_BF16) {
    need = svlm_decode_attn_workspace(batch, nq, Hq, Hkv, D, max_kv_len, num_splits);
    if (need > kScratchBytes)
      return fail(SVLM_E_UNSUPPORTED,
                  "svlm_decode_attn_noalloc: this call needs %zu bytes of split-K state; the static scratch "
                  "holds %zu (use svlm_decode_attn with a workspace, or fewer splits)", need, kScratchBytes);
  }
  void* ws = nullptr;
  if (need > 0) {
    const int st = scratch_address(&ws);
    if (st != SVLM_OK) return st;
  }
  return decode_attn_impl("svlm_decode_attn_noalloc", q, q_sb, k, v, kv_sb, kv_sh, kv_sn, nullptr, 0, 0, 0, kv_len,
                          1, 0, max_kv_len, dtype, batch, nq, Hq, Hkv, D, scale, causal_tail, out, lse, num_splits,
                          ws, need > 0 ? kScratchBytes : 0, stream);
}

#ifdef SVLM_DEBUG
bool svlm::debug_take_decode_attn(unsigned* out) { return debug_take_here(out); }
#endif
