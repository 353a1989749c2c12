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
//    (rows = G * nq, row r = i * G + local head), padded to 16-row blocks;
//  * K and V are read straight from HBM into registers in matrix-core operand
//    layout, 32 keys per wave per step, double buffered, each byte once;
//  * S^T = K * Q^T on v_mfma_f32_16x16x32_bf16: lane holds 4 keys x 1 row per
//    16-key block, so every lane owns one query row throughout;
//  * online softmax in the exp2 domain (scale * log2 e folded into one fp32
//    multiply); row maxima cross the four lane groups with two xor-shuffles;
//  * O^T += V^T * P^T with P split into bf16 hi + lo (two products), which
//    keeps the weights at ~2^-16 relative error; V^T operands come from the
//    16-byte V loads by byte permutes (no LDS round trip);
//  * waves of a workgroup merge through LDS in a fixed order, then either
//    write the final fp32 output (one split) or a partial (max, sum, output)
//    that a second kernel merges in split order.
#include <cmath>
#include <cstdio>

#include "svlm_internal.h"

namespace svlm {
namespace {

struct AttnArgs {
  const uint16_t* q;
  int64_t q_sb;
  const uint16_t* k;
  const uint16_t* v;
  int64_t kv_sb, kv_sh, kv_sn;
  const int32_t* kv_len;
  int max_kv_len;
  int batch, nq, Hq, Hkv, G, rows;
  float c;  // scale * log2(e)
  int causal;
  int splits, keys_per_split;
  float* out;
  float* lse;
  float* ws_o;   // [B*Hkv*rows][splits][D]
  float* ws_ml;  // [B*Hkv*rows][splits][2]
};

constexpr int kTile = 32;      // keys per wave step
constexpr int kMaxRB64 = 5;    // up to 80 query rows per workgroup at D = 64
constexpr int kMaxRB128 = 3;   // 48 rows at D = 128 (more would spill registers)
constexpr float kNegInf = -INFINITY;
constexpr float kRescale = 8.f;  // log2 headroom before the running maximum is raised

// buffer descriptor word 3 for gfx9-family raw buffer loads (no swizzle, no stride)
constexpr int kBufferFlags = 0x00020000;
// cache policy of the streaming KV loads: nontemporal
constexpr int kNT = 2;

template <int DV>
struct VRaw;
template <>
struct VRaw<8> { typedef unsigned __attribute__((ext_vector_type(4))) T; };
template <>
struct VRaw<4> { typedef unsigned __attribute__((ext_vector_type(2))) T; };

// Wait until at most N vector-memory operations of this wave are outstanding
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt at max).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  constexpr int enc = (N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8);
  __builtin_amdgcn_s_waitcnt(enc);
  __asm__ volatile("" ::: "memory");
}
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
  __asm__ volatile("" ::: "memory");
}

template <int DV>
__device__ __forceinline__ typename VRaw<DV>::T load_v(__amdgpu_buffer_rsrc_t rs, int off);
template <>
__device__ __forceinline__ VRaw<8>::T load_v<8>(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kNT);
}
template <>
__device__ __forceinline__ VRaw<4>::T load_v<4>(__amdgpu_buffer_rsrc_t rs, int off) {
  return __builtin_amdgcn_raw_buffer_load_b64(rs, off, 0, kNT);
}

// Depth of the per-wave staging ring: as many K/V tiles in flight as the LDS
// (160 KB per CU, one workgroup per CU) holds, with every outstanding transfer
// countable by the 6-bit vector-memory wait counter.
template <int D, int RB, int NW>
constexpr int ring_depth() {
  constexpr int TB = kTile * D * 2;
  constexpr int NI = TB / 1024;
  constexpr int RP = RB * 16;
  constexpr size_t slice_bytes = (size_t)RP * (D + 4) * 4;
  int best = 1;
  for (int ns = 1; ns <= 4; ++ns) {
    const size_t slot = (size_t)NW * ns * TB;
    const size_t ks = slot > ((NW + 1) / 2) * slice_bytes ? slot : ((NW + 1) / 2) * slice_bytes;
    const size_t vs = slot > (NW / 2) * slice_bytes ? slot : (NW / 2) * slice_bytes;
    const size_t lds = ks + vs + (size_t)RP * D * 2 + 2 * (size_t)NW * RP * 4 + 64;
    if (2 * ns * NI <= 63 && lds <= 160 * 1024) best = ns;
  }
  return best;
}

template <int D, int RB, int NW, int NS>
__global__ __launch_bounds__(64 * NW, 1) void attn_splitk(AttnArgs a) {
  constexpr int KK = D / 32;             // 32-wide d chunks of the QK product
  constexpr int DV = D / 16;             // d values per lane in the PV product
  constexpr int RP = RB * 16;
  constexpr int ROWB = D * 2;            // bytes of one K or V row in a staged tile
  constexpr int CH = ROWB / 16;          // 16-byte chunks per row
  constexpr int TB = kTile * ROWB;       // bytes of one staged K (or V) tile
  constexpr int NI = TB / 1024;          // 1 KB transfers per K (or V) tile
  constexpr int OSTRIDE = D + 4;         // fp32 elements per merge-slice row
  typedef typename VRaw<DV>::T vraw_t;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int c = lane & 15;
  const int g4 = lane >> 4;

  int bid = blockIdx.x;
  const int s = bid % a.splits;
  bid /= a.splits;
  const int h = bid % a.Hkv;
  const int b = bid / a.Hkv;
  const int row_base = blockIdx.y * RP;

  const int n_kv = min(max(a.kv_len[b], 0), a.max_kv_len);
  const int k_begin = s * a.keys_per_split;
  const int k_end = min(k_begin + a.keys_per_split, n_kv);

  // LDS: one K + V staging slot per wave; staged query rows; per-wave row state.
  // The slot area is reused for the merge slices after the key loop.
  // K and V slots are distinct objects so the compiler can tell their transfers apart.
  // NS staging slots per wave form a ring, so NS tiles are in flight per wave.
  // After the key loop the slots hold the merge slices: the first half of the
  // slices in kslots, the rest in vslots.
  constexpr size_t SLOT_BYTES = (size_t)NW * NS * TB;
  constexpr int NSLICE = NW;
  constexpr size_t SLICE_BYTES = (size_t)RP * OSTRIDE * 4;
  constexpr size_t KS_BYTES = SLOT_BYTES > ((NSLICE + 1) / 2) * SLICE_BYTES ? SLOT_BYTES : ((NSLICE + 1) / 2) * SLICE_BYTES;
  constexpr size_t VS_BYTES = SLOT_BYTES > (NSLICE / 2) * SLICE_BYTES ? SLOT_BYTES : (NSLICE / 2) * SLICE_BYTES;
  __shared__ __align__(16) unsigned char kslots[KS_BYTES];
  __shared__ __align__(16) unsigned char vslots[VS_BYTES];
  __shared__ __align__(16) unsigned char sq[RP * ROWB];  // query rows, chunks swizzled like the KV tiles
  __shared__ float sm_m[NW][RP];
  __shared__ float sm_l[NW][RP];

  // Range-checked buffer descriptors over exactly this split's keys: transfers
  // past k_end deliver zeros without touching memory, so every transfer is
  // issued unconditionally and the wait counts below are static.
  const int64_t row_bytes = a.kv_sn * 2;
  const int n_rows = max(k_end - k_begin, 0);
  const int64_t off0 = (int64_t)b * a.kv_sb + (int64_t)h * a.kv_sh + (int64_t)k_begin * a.kv_sn;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + off0), (short)0, (int)(n_rows * row_bytes), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + off0), (short)0, (int)(n_rows * row_bytes), kBufferFlags);

  unsigned char* kring = kslots + (size_t)wave * NS * TB;
  unsigned char* vring = vslots + (size_t)wave * NS * TB;

  // Global -> LDS transfer of 32 rows, row-major with 16-byte chunks XOR-swizzled
  // by row (chunk p of row r holds source chunk p ^ (r % CH)); every lane moves
  // 16 bytes and lands at slot + 1 KB * i + 16 * lane.  Nontemporal: read once.
  auto stage = [&](__amdgpu_buffer_rsrc_t rs, unsigned char* slot, int t0) {
    const int r0 = t0 - k_begin;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int r = i * (1024 / ROWB) + lane / CH;
      const int p = lane % CH;
      const int src = (r0 + r) * (int)row_bytes + ((p ^ (r % CH)) * 16);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(slot + i * 1024), 16,
                                               src, 0, 0, kNT);
    }
  };
  // chunk `ch` of staged row r
  auto chunk_at = [&](const unsigned char* slot, int r, int ch) { return slot + r * ROWB + ((ch ^ (r % CH)) * 16); };

  // ---- stage the query rows of this workgroup (B operand of S^T = K Q^T) by
  // LDS DMA, first; rows past the last query read as zeros
  {
    const int64_t qbytes = (int64_t)a.nq * a.Hq * D * 2;
    const __amdgpu_buffer_rsrc_t qrs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(a.q + (int64_t)b * a.q_sb), (short)0, (int)qbytes, kBufferFlags);
    constexpr int QI = RP * ROWB / 1024;  // 1 KB transfers for the staged rows
    for (int i = wave; i < QI; i += NW) {
      const int rr = i * (1024 / ROWB) + lane / CH;
      const int p = lane % CH;
      const int r = row_base + rr;
      int src = (int)qbytes;  // out of range: zeros
      if (r < a.rows) {
        const int qi = r / a.G;
        const int hl = r - qi * a.G;
        src = ((qi * a.Hq + h * a.G + hl) * D) * 2 + ((p ^ (rr % CH)) * 16);
      }
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qrs, (__attribute__((address_space(3))) void*)(sq + i * 1024), 16, src,
                                               0, 0, 0);
    }
  }

  // this wave's tiles: t = t_first + j * step, j < n_my
  const int step = kTile * NW;
  const int t_first = k_begin + kTile * wave;
  const int n_my = (t_first < k_end) ? (k_end - t_first + step - 1) / step : 0;
#pragma unroll
  for (int q = 0; q < NS; ++q) {  // unconditional: past k_end these deliver zeros
    stage(krs, kring + q * TB, t_first + q * step);
    stage(vrs, vring + q * TB, t_first + q * step);
  }
  wait_vmcnt<2 * NS * NI>();  // this wave's query transfers have landed
  int lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row_base + rb * 16 + c;
    const int i = r / a.G;
    lim[rb] = (r < a.rows) ? min(k_end, a.causal ? n_kv - a.nq + i + 1 : n_kv) : k_end;
  }
  // keys every row of this workgroup may see: tiles below this need no mask
  const int lim_all = min(k_end, a.causal ? n_kv - a.nq + 1 : n_kv);
  __syncthreads();

  // Running state per row (lane row c + 16 rb, uniform over the four lane
  // groups): m_use is the reference maximum in log2 units, raised only when a
  // tile's maximum exceeds it by more than kRescale, so the weights stay
  // <= 2^kRescale and the fp32 accumulators are rescaled only rarely.
  float m_use[RB], l_run[RB];
  f32x4 o[DV][RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_use[rb] = kNegInf;
    l_run[rb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < DV; ++mb) o[mb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  for (int j = 0; j < n_my; ++j) {
    const int t0 = t_first + j * step;
    unsigned char* kslot = kring + (j % NS) * TB;
    unsigned char* vslot = vring + (j % NS) * TB;
    // Issue order is K(t) V(t) K(t+1) V(t+1) ... K(t+NS-1) V(t+NS-1): K(t) has
    // landed once at most 2 NS - 1 groups of NI transfers are outstanding.
    wait_vmcnt<(2 * NS - 1) * NI>();
    u32x4 kt_[2][KK];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) kt_[kt][kk] = *(const u32x4*)chunk_at(kslot, 16 * kt + c, kk * 4 + g4);
    wait_lgkmcnt0();
    stage(krs, kslot, t0 + NS * step);  // K(t+NS): out of range past the last tile, i.e. zeros

    // S^T blocks: lane holds keys t0 + 16kt + 4g4 + ii for its row
    f32x4 sacc[2][RB];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) sacc[kt][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const bf16x8 qv = as_bf16x8(*(const u32x4*)chunk_at(sq, rb * 16 + c, kk * 4 + g4));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt][rb] = mfma16(as_bf16x8(kt_[kt][kk]), qv, sacc[kt][rb]);
      }

    // V(t) has landed once at most 2 NS - 1 groups are outstanding (K(t+NS) included)
    wait_vmcnt<(2 * NS - 1) * NI>();
    vraw_t vt[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int r = (jj < 4) ? (4 * g4 + jj) : (16 + 4 * g4 + jj - 4);
      if constexpr (DV == 8) vt[jj] = *(const vraw_t*)chunk_at(vslot, r, c);
      else vt[jj] = *(const vraw_t*)(chunk_at(vslot, r, c >> 1) + (c & 1) * 8);
    }
    wait_lgkmcnt0();
    stage(vrs, vslot, t0 + NS * step);

    const bool full = (t0 + kTile <= lim_all);  // wave-uniform
    float x[RB][8], mx[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = sacc[e >> 2][rb][e & 3];
        x[rb][e] = (full || t0 + 16 * (e >> 2) + 4 * g4 + (e & 3) < lim[rb]) ? v : kNegInf;
      }
      float m = fmaxf(fmaxf(fmaxf(x[rb][0], x[rb][1]), fmaxf(x[rb][2], x[rb][3])),
                      fmaxf(fmaxf(x[rb][4], x[rb][5]), fmaxf(x[rb][6], x[rb][7])));
      mx[rb] = max_xor32(max_xor16(m)) * a.c;  // raw scores -> log2 units (c > 0 keeps the order)
    }
    bool grow = false;
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) grow |= (mx[rb] > m_use[rb] + kRescale);
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const float m_new = fmaxf(m_use[rb], mx[rb]);
        const float alpha = (m_use[rb] == kNegInf) ? 0.f : fast_exp2(m_use[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < DV; ++mb) o[mb][rb] *= alpha;
        m_use[rb] = m_new;
      }
    }
    bf16x8 phi[RB], plo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const float mneg = (m_use[rb] == kNegInf) ? 0.f : -m_use[rb];
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(x[rb][e], a.c, mneg));
      l_run[rb] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      u32x4 hi, lo;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        const unsigned b0 = f_bits(p[2 * qd]), b1 = f_bits(p[2 * qd + 1]);
        hi[qd] = perm(b1, b0, kPermHi);
        const float r0 = p[2 * qd] - bits_f(b0 & 0xFFFF0000u);
        const float r1 = p[2 * qd + 1] - bits_f(b1 & 0xFFFF0000u);
        lo[qd] = perm(f_bits(r1), f_bits(r0), kPermHi);
      }
      phi[rb] = as_bf16x8(hi);
      plo[rb] = as_bf16x8(lo);
    }
    // O^T += V^T P^T, two column blocks at a time (hi and lo products into one
    // accumulator are 2 * RB instructions apart)
#pragma unroll
    for (int mb = 0; mb < DV; mb += 2) {
      bf16x8 vop[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int w = (mb + u) >> 1;
        const unsigned sel = ((mb + u) & 1) ? kPermHi : kPermLo;
        u32x4 vv;
#pragma unroll
        for (int qd = 0; qd < 4; ++qd) vv[qd] = perm(vt[2 * qd + 1][w], vt[2 * qd][w], sel);
        vop[u] = as_bf16x8(vv);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[mb + u][rb] = mfma16(vop[u], phi[rb], o[mb + u][rb]);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[mb + u][rb] = mfma16(vop[u], plo[rb], o[mb + u][rb]);
    }
  }
  wait_vmcnt<0>();  // the zero-filled transfers past the end must land before the slots are reused

  // row sums: add the four lane groups (the reference maxima are uniform across them)
  float m_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] = sum_xor32(sum_xor16(l_run[rb]));
    m_run[rb] = m_use[rb];
  }

  // ---- merge the waves of the workgroup: each wave scales its sums to the
  // common row maximum and parks them in its own LDS slice; then all threads
  // add the slices in wave order and write the rows with coalesced stores.
  if constexpr (NW > 1) {
    if (g4 == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        sm_m[wave][rb * 16 + c] = m_run[rb];
        sm_l[wave][rb * 16 + c] = l_run[rb];
      }
    }
    __syncthreads();  // every wave is past its key loop: the slot area is reused below
    auto slice = [&](int k) {
      constexpr int KH = (NSLICE + 1) / 2;
      return (k < KH) ? (float*)kslots + (size_t)k * RP * OSTRIDE : (float*)vslots + (size_t)(k - KH) * RP * OSTRIDE;
    };
    {
      float* sl = slice(wave);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        const int row = rb * 16 + c;
        float M = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][row]);
        const float f = (m_run[rb] == kNegInf) ? 0.f : exp2f(m_run[rb] - M);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int mb = 0; mb < DV; mb += 4)
            *(float4*)(sl + row * OSTRIDE + DV * (4 * g4 + i) + mb) =
                make_float4(o[mb][rb][i] * f, o[mb + 1][rb][i] * f, o[mb + 2][rb][i] * f, o[mb + 3][rb][i] * f);
      }
    }
    __syncthreads();
    constexpr int C4 = D / 4;
    for (int e = threadIdx.x; e < RP * C4; e += 64 * NW) {
      const int row = e / C4, d4 = e - row * C4;
      const int r = row_base + row;
      if (r >= a.rows) continue;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][row]);
      float L = 0.f;
      float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w][row];
        L += (mw == kNegInf) ? 0.f : sm_l[w][row] * exp2f(mw - M);
        const float4 v = *(const float4*)(slice(w) + row * OSTRIDE + 4 * d4);
        acc.x += v.x;
        acc.y += v.y;
        acc.z += v.z;
        acc.w += v.w;
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
    // ---- one wave: write the final output (one split) or this split's partial state
  #pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int r = row_base + rb * 16 + c;
      if (r >= a.rows) continue;
      const int i = r / a.G;
      const int hl = r - i * a.G;
      if (a.splits == 1) {
        const float L = l_run[rb];
        const float inv = (L > 0.f) ? 1.f / L : 0.f;
        float* orow = a.out + (((int64_t)b * a.nq + i) * a.Hq + (int64_t)h * a.G + hl) * D;
  #pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
  #pragma unroll
          for (int mb = 0; mb < DV; mb += 4) {
            float4 vv = make_float4(o[mb][rb][i4] * inv, o[mb + 1][rb][i4] * inv, o[mb + 2][rb][i4] * inv,
                                    o[mb + 3][rb][i4] * inv);
            *(float4*)(orow + DV * (4 * g4 + i4) + mb) = vv;
          }
        if (a.lse && g4 == 0)
          a.lse[((int64_t)b * a.nq + i) * a.Hq + (int64_t)h * a.G + hl] =
              (L > 0.f) ? (m_run[rb] + log2f(L)) * kLn2 : kNegInf;
      } else {
        const int64_t R = ((int64_t)b * a.Hkv + h) * a.rows + r;
        float* orow = a.ws_o + (R * a.splits + s) * D;
  #pragma unroll
        for (int i4 = 0; i4 < 4; ++i4)
  #pragma unroll
          for (int mb = 0; mb < DV; mb += 4) {
            float4 vv = make_float4(o[mb][rb][i4], o[mb + 1][rb][i4], o[mb + 2][rb][i4], o[mb + 3][rb][i4]);
            *(float4*)(orow + DV * (4 * g4 + i4) + mb) = vv;
          }
        if (g4 == 0) *(float2*)(a.ws_ml + (R * a.splits + s) * 2) = make_float2(m_run[rb], l_run[rb]);
      }
    }
  }

}

// Separate merge launch for large partial volumes: kCombineRows rows per
// workgroup, 128 threads per row = D/4 column groups x (512/D) split parts.
// Every thread issues all loads of its splits at once (one memory round trip),
// merges them against its own running maximum, and the parts are combined in
// a fixed order through LDS.  Deterministic.
constexpr int kCombineRows = 2;
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a) {
  constexpr int C4 = D / 4;
  constexpr int PARTS = 128 / C4;
  __shared__ float4 s_acc[256];
  __shared__ float2 s_ml[256];
  const int t = threadIdx.x;
  const int64_t R = (int64_t)blockIdx.x * kCombineRows + t / 128;  // (b * Hkv + h) * rows + r
  const int64_t rows_total = (int64_t)a.batch * a.Hkv * a.rows;
  const int d4 = (t & 127) % C4, part = (t & 127) / C4;
  const int S = a.splits;
  const int span = (S + PARTS - 1) / PARTS;
  const int s_lo = min(S, part * span), s_hi = min(S, s_lo + span);
  float M = kNegInf, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (R < rows_total) {
    const float2* ml = (const float2*)a.ws_ml + R * S;
    const float4* po = (const float4*)(a.ws_o + R * S * D) + d4;
    for (int sp = s_lo; sp < s_hi; ++sp) M = fmaxf(M, ml[sp].x);
    if (M != kNegInf) {
#pragma unroll 8
      for (int sp = s_lo; sp < s_hi; ++sp) {
        const float2 st = ml[sp];
        const float4 v = po[(int64_t)sp * C4];
        const float w = (st.x == kNegInf) ? 0.f : exp2f(st.x - M);
        L += w * st.y;
        acc.x += w * v.x;
        acc.y += w * v.y;
        acc.z += w * v.z;
        acc.w += w * v.w;
      }
    }
  }
  s_acc[t] = acc;
  s_ml[t] = make_float2(M, L);
  __syncthreads();
  if (R >= rows_total || part != 0) return;
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

template <int D, int RB, int NW>
void launch_rb(const AttnArgs& a, int batch, int row_chunks, hipStream_t st) {
  dim3 grid((unsigned)(batch * a.Hkv * a.splits), (unsigned)row_chunks);
  attn_splitk<D, RB, NW, ring_depth<D, RB, NW>()><<<grid, 64 * NW, 0, st>>>(a);
}

template <int D, int NW>
void launch_nw(const AttnArgs& a, int rb, int batch, int row_chunks, hipStream_t st) {
  switch (rb) {
    case 1: launch_rb<D, 1, NW>(a, batch, row_chunks, st); break;
    case 2: launch_rb<D, 2, NW>(a, batch, row_chunks, st); break;
    case 3: launch_rb<D, 3, NW>(a, batch, row_chunks, st); break;
    default:
      if constexpr (D == 64) {
        if (rb == 4) launch_rb<D, 4, NW>(a, batch, row_chunks, st);
        else launch_rb<D, 5, NW>(a, batch, row_chunks, st);
      }
      break;
  }
}

template <int D>
void launch_d(const AttnArgs& a, int nw, int rb, int batch, int row_chunks, hipStream_t st) {
  if (nw == 4) launch_nw<D, 4>(a, rb, batch, row_chunks, st);
  else if (nw == 2) launch_nw<D, 2>(a, rb, batch, row_chunks, st);
  else launch_nw<D, 1>(a, rb, batch, row_chunks, st);
}

struct Plan {
  int rb, row_chunks, nw, splits, keys_per_split;
};



Plan make_plan(int batch, int nq, int Hq, int Hkv, int D, int max_kv_len, int num_splits) {
  Plan p;
  const int rows = (Hq / Hkv) * nq;
  const int max_rb = (D == 128) ? kMaxRB128 : kMaxRB64;
  p.rb = std::min(max_rb, (rows + 15) / 16);
  p.row_chunks = (rows + p.rb * 16 - 1) / (p.rb * 16);
  const int tiles = (max_kv_len + kTile - 1) / kTile;
  int splits = num_splits;
  if (splits <= 0) {
    // about one workgroup per compute unit
    const int units = std::max(1, batch * Hkv * p.row_chunks);
    splits = std::max(1, (num_cus() + units - 1) / units);
  }
  splits = std::max(1, std::min(splits, tiles));
  const int tiles_per_split = (tiles + splits - 1) / splits;
  p.keys_per_split = tiles_per_split * kTile;
  p.splits = (max_kv_len + p.keys_per_split - 1) / p.keys_per_split;
  p.nw = tiles_per_split >= 4 ? 4 : (tiles_per_split >= 2 ? 2 : 1);
  return p;
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

extern "C" size_t svlm_decode_attn_workspace(int batch, int nq, int Hq, int Hkv, int D, int max_kv_len,
                                             int num_splits) {
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || max_kv_len < 1) return 0;
  const Plan p = make_plan(batch, nq, Hq, Hkv, D, max_kv_len, num_splits);
  return ws_layout(p, batch, Hq, nq, D).total;
}

extern "C" int svlm_decode_attn(const void* q, int64_t q_sb, const void* k, const void* v, int64_t kv_sb,
                                int64_t kv_sh, int64_t kv_sn, const int32_t* kv_len, int max_kv_len, int dtype,
                                int batch, int nq, int Hq, int Hkv, int D, float scale, int causal_tail,
                                float* out, float* lse, int num_splits, void* ws, size_t ws_bytes,
                                void* stream) {
  if (dtype != SVLM_BF16) return fail(SVLM_E_UNSUPPORTED, "svlm_decode_attn: only SVLM_BF16 operands are supported");
  if (D != 64 && D != 128) return fail(SVLM_E_UNSUPPORTED, "svlm_decode_attn: D must be 64 or 128 (got %d)", D);
  if (!q || !k || !v || !kv_len || !out) return fail(SVLM_E_INVALID, "svlm_decode_attn: null pointer");
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || max_kv_len < 1)
    return fail(SVLM_E_INVALID, "svlm_decode_attn: batch, nq, Hq, Hkv, max_kv_len must be >= 1");
  if (Hq % Hkv) return fail(SVLM_E_INVALID, "svlm_decode_attn: Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (causal_tail != 0 && causal_tail != 1) return fail(SVLM_E_INVALID, "svlm_decode_attn: causal_tail must be 0 or 1");
  if (!std::isfinite(scale)) return fail(SVLM_E_INVALID, "svlm_decode_attn: scale must be finite");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out))
    return fail(SVLM_E_INVALID, "svlm_decode_attn: q, k, v, out must be 16-byte aligned");
  if (kv_sn < D || kv_sn % 8 || kv_sh % 8 || kv_sb % 8 || kv_sh < 0 || kv_sb < 0)
    return fail(SVLM_E_INVALID, "svlm_decode_attn: KV strides must be multiples of 8 elements with kv_sn >= D");
  if (q_sb % 8 || (batch > 1 && q_sb < (int64_t)nq * Hq * D))
    return fail(SVLM_E_INVALID, "svlm_decode_attn: q batch stride must be a multiple of 8 and >= nq*Hq*D");
  if (num_splits < 0) return fail(SVLM_E_INVALID, "svlm_decode_attn: num_splits must be >= 0");
  const Plan p = make_plan(batch, nq, Hq, Hkv, D, max_kv_len, num_splits);
  const size_t need = svlm_decode_attn_workspace(batch, nq, Hq, Hkv, D, max_kv_len, num_splits);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(SVLM_E_WORKSPACE, "svlm_decode_attn: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (need > 0 && !aligned16(ws)) return fail(SVLM_E_INVALID, "svlm_decode_attn: workspace must be 16-byte aligned");

  AttnArgs a;
  a.q = (const uint16_t*)q;
  a.q_sb = q_sb;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.kv_sb = kv_sb;
  a.kv_sh = kv_sh;
  a.kv_sn = kv_sn;
  a.kv_len = kv_len;
  a.max_kv_len = max_kv_len;
  a.batch = batch;
  a.nq = nq;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.G = Hq / Hkv;
  a.rows = a.G * nq;
  a.c = scale * kLog2e;
  a.causal = causal_tail;
  a.splits = p.splits;
  a.keys_per_split = p.keys_per_split;
  a.out = out;
  a.lse = lse;
  const WsLayout wl = ws_layout(p, batch, Hq, nq, D);
  a.ws_o = ws ? (float*)((char*)ws + wl.o_off) : nullptr;
  a.ws_ml = ws ? (float*)((char*)ws + wl.ml_off) : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (D == 128) launch_d<128>(a, p.nw, p.rb, batch, p.row_chunks, st);
  else launch_d<64>(a, p.nw, p.rb, batch, p.row_chunks, st);
  if (p.splits > 1) {
    const unsigned blocks = (unsigned)(((int64_t)batch * Hkv * a.rows + kCombineRows - 1) / kCombineRows);
    if (D == 128) attn_combine<128><<<blocks, 256, 0, st>>>(a);
    else attn_combine<64><<<blocks, 256, 0, st>>>(a);
  }
  return check_launch("svlm_decode_attn");
}
