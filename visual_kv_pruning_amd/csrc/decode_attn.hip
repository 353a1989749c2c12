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
  int nq, Hq, Hkv, G, rows;
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

template <int D, int RB, int NW, int NB>
__global__ __launch_bounds__(64 * NW, 1) void attn_splitk(AttnArgs a) {
  constexpr int KK = D / 32;  // 32-wide d chunks of the QK product
  constexpr int DV = D / 16;  // d values per lane in the PV product
  constexpr int RP = RB * 16;
  constexpr int QSTRIDE = D + 8;       // bf16 elements per staged query row (16-byte pad)
  constexpr int OSTRIDE = D + 4;       // fp32 elements per merge-slice row
  constexpr int NSLICE = (NW >= 8) ? 4 : (NW >= 4 ? 2 : 1);
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

  // Range-checked buffer descriptors over exactly this split's keys: loads past
  // k_end return zeros without touching memory, so every load in the stream
  // is unconditional and the wait counts stay exact.
  const int64_t row_bytes = a.kv_sn * 2;
  const int n_rows = max(k_end - k_begin, 0);
  const int64_t off0 = (int64_t)b * a.kv_sb + (int64_t)h * a.kv_sh + (int64_t)k_begin * a.kv_sn;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + off0), (short)0, (int)(n_rows * row_bytes), kBufferFlags);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.v + off0), (short)0, (int)(n_rows * row_bytes), kBufferFlags);

  struct Tile {
    u32x4 k[2][KK];
    vraw_t v[8];
  };
  // K operand: lane holds K[t0 + 16 kt + c][32 kk + 8 g4 .. +8]; V: the 8 keys
  // {4g4 .. 4g4+3, 16+4g4 .. 16+4g4+3} of the tile at d = DV*c .. DV*c + DV - 1.
  // Streaming KV is read once: nontemporal loads.
  auto load_tile = [&](Tile& t, int t0) {
    const int r0 = t0 - k_begin;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const int off = (r0 + 16 * kt + c) * (int)row_bytes + g4 * 16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) t.k[kt][kk] = __builtin_amdgcn_raw_buffer_load_b128(krs, off + kk * 64, 0, kNT);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int row = r0 + ((j < 4) ? (4 * g4 + j) : (16 + 4 * g4 + j - 4));
      t.v[j] = load_v<DV>(vrs, row * (int)row_bytes + DV * 2 * c);
    }
  };

  // this wave's tiles: t = t_first + j * step, j < n_my
  const int step = kTile * NW;
  const int t_first = k_begin + kTile * wave;
  const int n_my = (t_first < k_end) ? (k_end - t_first + step - 1) / step : 0;
  Tile buf[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) load_tile(buf[i], t_first + i * step);  // first requests go out before anything else

  // ---- stage the query rows of this workgroup in LDS (B operand of S^T = K Q^T)
  __shared__ __align__(16) unsigned char smem[(size_t)RP * QSTRIDE * 2 > (size_t)NSLICE * RP * OSTRIDE * 4
                                                    ? (size_t)RP * QSTRIDE * 2
                                                    : (size_t)NSLICE * RP * OSTRIDE * 4];
  __shared__ float sm_m[NW][RP];
  __shared__ float sm_l[NW][RP];
  uint16_t* sq = (uint16_t*)smem;
  for (int e = threadIdx.x; e < RP * (D / 8); e += 64 * NW) {
    const int rr = e / (D / 8), ch = e - rr * (D / 8);
    const int r = row_base + rr;
    u32x4 val = {0u, 0u, 0u, 0u};
    if (r < a.rows) {
      const int i = r / a.G;
      const int hl = r - i * a.G;
      val = *(const u32x4*)(a.q + (int64_t)b * a.q_sb + ((int64_t)i * a.Hq + (int64_t)h * a.G + hl) * D + ch * 8);
    }
    *(u32x4*)(sq + rr * QSTRIDE + ch * 8) = val;
  }
  int lim[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = row_base + rb * 16 + c;
    const int i = r / a.G;
    lim[rb] = (r < a.rows) ? min(k_end, a.causal ? n_kv - a.nq + i + 1 : n_kv) : k_end;
  }
  __syncthreads();

  // keys every row of this workgroup may see: tiles below this need no mask
  const int lim_all = min(k_end, a.causal ? n_kv - a.nq + 1 : n_kv);

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

  auto compute_tile = [&](const Tile& t, int t0) {
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
        const bf16x8 qv = as_bf16x8(*(const u32x4*)(sq + (rb * 16 + c) * QSTRIDE + kk * 32 + g4 * 8));
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) sacc[kt][rb] = mfma16(as_bf16x8(t.k[kt][kk]), qv, sacc[kt][rb]);
      }

    const bool full = (t0 + kTile <= lim_all);  // wave-uniform
    bf16x8 phi[RB], plo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = sacc[e >> 2][rb][e & 3];
      if (!full) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (t0 + 16 * (e >> 2) + 4 * g4 + (e & 3) >= lim[rb]) x[e] = kNegInf;
      }
      float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])), fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
      mx = max_xor32(max_xor16(mx)) * a.c;  // raw scores -> log2 units (c > 0 keeps the order)
      if (__builtin_amdgcn_ballot_w64(mx > m_use[rb] + kRescale) != 0) {
        const float m_new = fmaxf(m_use[rb], mx);
        const float alpha = (m_use[rb] == kNegInf) ? 0.f : fast_exp2(m_use[rb] - m_new);
        l_run[rb] *= alpha;
#pragma unroll
        for (int mb = 0; mb < DV; ++mb) o[mb][rb] *= alpha;
        m_use[rb] = m_new;
      }
      const float mneg = (m_use[rb] == kNegInf) ? 0.f : -m_use[rb];
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) p[e] = fast_exp2(fmaf(x[e], a.c, mneg));
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

    // O^T += V^T P^T; lane's A operand for block mb is d = DV*c + mb over its 8 keys
#pragma unroll
    for (int mb = 0; mb < DV; ++mb) {
      const int w = mb >> 1;
      const unsigned sel = (mb & 1) ? kPermHi : kPermLo;
      u32x4 vv;
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) vv[qd] = perm(t.v[2 * qd + 1][w], t.v[2 * qd][w], sel);
      const bf16x8 vop = as_bf16x8(vv);
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        o[mb][rb] = mfma16(vop, phi[rb], o[mb][rb]);
        o[mb][rb] = mfma16(vop, plo[rb], o[mb][rb]);
      }
    }
  };

  // ---- steady state: unconditional loads keep NB tiles in flight; then the tail
  {
    int j = 0;
    for (; j + NB <= n_my; j += NB) {
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        const int t = t_first + (j + i) * step;
        compute_tile(buf[i], t);
        load_tile(buf[i], t + NB * step);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
      if (j + i < n_my) compute_tile(buf[i], t_first + (j + i) * step);
  }

  // row sums: add the four lane groups (the reference maxima are uniform across them)
  float m_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] = sum_xor32(sum_xor16(l_run[rb]));
    m_run[rb] = m_use[rb];
  }

  // ---- merge the waves of the workgroup in a fixed tree order
  if constexpr (NW > 1) {
    if (g4 == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        sm_m[wave][rb * 16 + c] = m_run[rb];
        sm_l[wave][rb * 16 + c] = l_run[rb];
      }
    }
    __syncthreads();  // also ends every use of the staged queries: smem is reused below
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int row = rb * 16 + c;
      float M = kNegInf;
#pragma unroll
      for (int w = 0; w < NW; ++w) M = fmaxf(M, sm_m[w][row]);
      float L = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm_m[w][row];
        L += (mw == kNegInf) ? 0.f : sm_l[w][row] * exp2f(mw - M);
      }
      const float f = (m_run[rb] == kNegInf) ? 0.f : exp2f(m_run[rb] - M);
#pragma unroll
      for (int mb = 0; mb < DV; ++mb) o[mb][rb] *= f;
      m_run[rb] = M;
      l_run[rb] = L;
    }
    float* slices = (float*)smem;
    auto slice = [&](int k) { return slices + (size_t)k * RP * OSTRIDE; };
    auto store_slice = [&](float* sl) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int mb = 0; mb < DV; mb += 4)
            *(float4*)(sl + (rb * 16 + c) * OSTRIDE + DV * (4 * g4 + i) + mb) =
                make_float4(o[mb][rb][i], o[mb + 1][rb][i], o[mb + 2][rb][i], o[mb + 3][rb][i]);
    };
    auto add_slice = [&](const float* sl) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int mb = 0; mb < DV; mb += 4) {
            const float4 v = *(const float4*)(sl + (rb * 16 + c) * OSTRIDE + DV * (4 * g4 + i) + mb);
            o[mb][rb][i] += v.x;
            o[mb + 1][rb][i] += v.y;
            o[mb + 2][rb][i] += v.z;
            o[mb + 3][rb][i] += v.w;
          }
    };
    // rounds: waves [half, width) hand their sums to waves [0, half)
#pragma unroll
    for (int width = NW; width > 1; width >>= 1) {
      const int half = width >> 1;
      if (wave >= half && wave < width) store_slice(slice(wave - half));
      __syncthreads();
      if (wave < half) add_slice(slice(wave));
      __syncthreads();
    }
    if (wave != 0) return;
  }

  // ---- write: final output (one split) or the partial state of this split
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

// Merge the split partials of one query row per wave, in split order.  Every
// partial load of a row is independent, so they are all in flight at once.
template <int D>
__global__ __launch_bounds__(256) void attn_combine(AttnArgs a, int64_t rows_total) {
  constexpr int PL = D / 64;  // output columns per lane
  const int lane = threadIdx.x & 63;
  const int64_t R = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (R >= rows_total) return;
  const float* ml = a.ws_ml + R * a.splits * 2;
  const float* po = a.ws_o + R * a.splits * D + lane * PL;
  float M = kNegInf;
  for (int s0 = lane; s0 < a.splits; s0 += 64) M = fmaxf(M, ml[2 * s0]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  float L = 0.f;
  float acc[PL];
#pragma unroll
  for (int e = 0; e < PL; ++e) acc[e] = 0.f;
  if (M != kNegInf) {
#pragma unroll 16
    for (int s = 0; s < a.splits; ++s) {
      const float2 st = *(const float2*)(ml + 2 * s);
      const float w = (st.x == kNegInf) ? 0.f : exp2f(st.x - M);
      L += st.y * w;
      if constexpr (PL == 2) {
        const float2 v = *(const float2*)(po + (int64_t)s * D);
        acc[0] += w * v.x;
        acc[1] += w * v.y;
      } else {
        acc[0] += w * po[(int64_t)s * D];
      }
    }
  }
  const int r = (int)(R % a.rows);
  const int64_t bh = R / a.rows;
  const int h = (int)(bh % a.Hkv);
  const int b = (int)(bh / a.Hkv);
  const int i = r / a.G;
  const int hl = r - i * a.G;
  const int64_t orow = ((int64_t)b * a.nq + i) * a.Hq + (int64_t)h * a.G + hl;
  const float inv = (L > 0.f) ? 1.f / L : 0.f;
#pragma unroll
  for (int e = 0; e < PL; ++e) a.out[orow * D + lane * PL + e] = acc[e] * inv;
  if (a.lse && lane == 0) a.lse[orow] = (L > 0.f) ? (M + log2f(L)) * kLn2 : kNegInf;
}

// tiles in flight per wave: eight-wave workgroups run two waves per SIMD, which
// hide each other's memory latency, so one tile per wave fits their register
// budget; narrower workgroups keep two.
template <int D, int RB, int NW>
constexpr int pipeline_depth() {
  return (NW >= 8) ? 1 : 2;
}

template <int D, int RB, int NW>
void launch_rb(const AttnArgs& a, int batch, int row_chunks, hipStream_t st) {
  dim3 grid((unsigned)(batch * a.Hkv * a.splits), (unsigned)row_chunks);
  attn_splitk<D, RB, NW, pipeline_depth<D, RB, NW>()><<<grid, 64 * NW, 0, st>>>(a);
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
  if (nw == 8) launch_nw<D, 8>(a, rb, batch, row_chunks, st);
  else if (nw == 4) launch_nw<D, 4>(a, rb, batch, row_chunks, st);
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
  p.nw = tiles_per_split >= 8 ? 8 : (tiles_per_split >= 4 ? 4 : (tiles_per_split >= 2 ? 2 : 1));
  return p;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" size_t svlm_decode_attn_workspace(int batch, int nq, int Hq, int Hkv, int D, int max_kv_len,
                                             int num_splits) {
  if (batch < 1 || nq < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || D < 1 || max_kv_len < 1) return 0;
  const Plan p = make_plan(batch, nq, Hq, Hkv, D, max_kv_len, num_splits);
  if (p.splits <= 1) return 0;
  const size_t rows_total = (size_t)batch * Hq * nq;
  return rows_total * p.splits * ((size_t)D + 2) * sizeof(float);
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
  a.ws_o = (float*)ws;
  const size_t rows_total = (size_t)batch * Hq * nq;
  a.ws_ml = ws ? (float*)ws + rows_total * p.splits * D : nullptr;
  hipStream_t st = (hipStream_t)stream;
  if (D == 128) launch_d<128>(a, p.nw, p.rb, batch, p.row_chunks, st);
  else launch_d<64>(a, p.nw, p.rb, batch, p.row_chunks, st);
  if (p.splits > 1) {
    const unsigned blocks = (unsigned)((rows_total + 3) / 4);
    if (D == 128) attn_combine<128><<<blocks, 256, 0, st>>>(a, (int64_t)rows_total);
    else attn_combine<64><<<blocks, 256, 0, st>>>(a, (int64_t)rows_total);
  }
  return check_launch("svlm_decode_attn");
}
