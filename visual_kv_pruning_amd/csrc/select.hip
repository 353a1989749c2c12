// svlm_select: two-stage visual token selection, one workgroup per row.
//
// SpecVLM technology-transfer listing, section 5 ("solution"): tokens split by
// score into high-information and low-attention ones; (i) the former are kept
// by Top-P on the share of attention score, (ii) among the latter a spatially
// uniform subset is kept.  SpecVLM abstract: stage I verifier-guided, stage
// II spatially uniform.  Sparse-to-Dense explainer, "KV cache selection":
// plain top-K per layer and head (top_p >= 1).
//
// Exactness: masses are floor(s * 2^40) integers (exact for fp32 s in [0,1]),
// sums are uint64, the target is ceil(double(Q) * P) in round-to-nearest
// doubles; stage I is found by a 32-step bitwise descent over the fp32 key
// bits with block-wide (count, mass) reductions - no atomics, so no
// contention on nearly flat rows and no order dependence; stage II is a
// per-token integer test on its rank in the remainder.  Ranks and output
// positions come from ordered block scans, so `kept` is written ascending.
#pragma clang fp contract(off)

#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kPer = 4;                     // elements per thread per scan chunk
constexpr int kChunk = kThreads * kPer;

struct SelArgs {
  const float* scores;
  int64_t row_stride;
  int N, budget, gh_gw;
  double top_p;
  int32_t* kept;
  int32_t* n_stage1;
  uint8_t* tag;
};

__device__ __forceinline__ unsigned key_of(float s) {
  unsigned k = f_bits(s);
  return (k == 0x80000000u) ? 0u : k;       // -0 orders as +0
}

__device__ __forceinline__ uint64_t mass_of_key(unsigned key) {
  return (uint64_t)(bits_f(key) * 0x1p40f);  // exact: power-of-two scale, then floor
}

struct Red {
  unsigned cnt;
  uint64_t mass;
};

// block-wide sums; every thread gets the totals
__device__ Red block_sum(Red r, Red* sm) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    r.cnt += __shfl_xor(r.cnt, off);
    r.mass += __shfl_xor(r.mass, off);
  }
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  __syncthreads();
  if (lane == 0) sm[wv] = r;
  __syncthreads();
  Red t = {0u, 0ull};
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    t.cnt += sm[w].cnt;
    t.mass += sm[w].mass;
  }
  return t;
}

// block-wide exclusive scan of per-thread counts in thread order
__device__ unsigned block_excl_scan(unsigned x, unsigned* total, unsigned* sm) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  unsigned incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const unsigned y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) sm[wv] = incl;
  __syncthreads();
  unsigned before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const unsigned v = sm[w];
    if (w < wv) before += v;
    tot += v;
  }
  *total = tot;
  return before + incl - x;
}

__global__ __launch_bounds__(kThreads) void select_rows(SelArgs a) {
  __shared__ Red sm_red[kWaves];
  __shared__ unsigned sm_scan[kWaves];
  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const float* s = a.scores + (int64_t)row * a.row_stride;
  const int N = a.N, B = a.budget;

  // ---- total fixed-point mass of the row
  Red mine = {0u, 0ull};
  for (int n = tid; n < N; n += kThreads) mine.mass += mass_of_key(key_of(s[n]));
  const uint64_t Q = block_sum(mine, sm_red).mass;

  // ---- stage I: k1 = a_cnt + c taken, keys > vstar all taken, c ties at vstar by index
  unsigned vstar = 0xFFFFFFFFu;  // nothing taken when k1 == 0
  int k1 = 0, c_ties = 0;
  bool any_stage1 = (B > 0) && (a.top_p > 0.0);
  uint64_t Tm = ~0ull;
  if (any_stage1 && a.top_p < 1.0) {
    Tm = (uint64_t)ceil((double)Q * a.top_p);
    if (Tm == 0) any_stage1 = false;
  }
  if (any_stage1) {
    unsigned prefix = 0;
    unsigned cnt_above = 0;
    uint64_t mass_above = 0;
    for (int j = 31; j >= 0; --j) {
      const unsigned cand = prefix | (1u << j);
      Red r = {0u, 0ull};
      for (int n = tid; n < N; n += kThreads) {
        const unsigned key = key_of(s[n]);
        if ((key >> j) == (cand >> j)) {
          r.cnt += 1;
          r.mass += mass_of_key(key);
        }
      }
      r = block_sum(r, sm_red);
      if (cnt_above + r.cnt >= (unsigned)B || mass_above + r.mass >= Tm) {
        prefix = cand;
      } else {
        cnt_above += r.cnt;
        mass_above += r.mass;
      }
    }
    vstar = prefix;
    int c = B - (int)cnt_above;
    if (a.top_p < 1.0) {
      const uint64_t ms = mass_of_key(vstar);
      if (ms > 0) {
        const uint64_t need = (Tm - mass_above + ms - 1) / ms;
        if (need < (uint64_t)c) c = (int)need;
      }
    }
    c_ties = c;
    k1 = (int)cnt_above + c;
  }

  // ---- stage II parameters
  const int64_t n_rem = N - k1;
  const int64_t m_fill = B - k1;

  // ---- ordered pass: ties -> stage-I flags -> remainder ranks -> stage-II flags -> positions
  unsigned tie_carry = 0, s1_carry = 0, kept_carry = 0;
  for (int base = 0; base < N; base += kChunk) {
    const int n0 = base + tid * kPer;
    unsigned key[kPer];
    unsigned tie_cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      key[e] = (n0 + e < N) ? key_of(s[n0 + e]) : 0u;
      tie_cnt += (n0 + e < N && k1 > 0 && key[e] == vstar) ? 1u : 0u;
    }
    unsigned tot;
    unsigned tie_before = tie_carry + block_excl_scan(tie_cnt, &tot, sm_scan);
    tie_carry += tot;

    bool s1[kPer];
    unsigned s1_cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      bool f = false;
      if (n0 + e < N && k1 > 0) {
        if (key[e] > vstar) f = true;
        else if (key[e] == vstar) {
          f = tie_before < (unsigned)c_ties;
          ++tie_before;
        }
      }
      s1[e] = f;
      s1_cnt += f ? 1u : 0u;
    }
    unsigned s1_before = s1_carry + block_excl_scan(s1_cnt, &tot, sm_scan);
    s1_carry += tot;

    bool kp[kPer];
    uint8_t tg[kPer];
    unsigned kept_cnt = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int n = n0 + e;
      bool k = false;
      uint8_t t = 0;
      if (n < N) {
        if (s1[e]) {
          k = true;
          t = 1;
          ++s1_before;
        } else if (m_fill > 0) {
          const int64_t rho = (int64_t)n - s1_before;   // rank among the remainder
          const int64_t num = 2 * m_fill * rho - n_rem;
          const int64_t den = 2 * n_rem;
          int64_t j = (num <= 0) ? 0 : (num + den - 1) / den;
          if (j < m_fill && ((2 * j + 1) * n_rem) / (2 * m_fill) == rho) {
            k = true;
            t = 2;
          }
        }
      }
      kp[e] = k;
      tg[e] = t;
      kept_cnt += k ? 1u : 0u;
    }
    unsigned pos = kept_carry + block_excl_scan(kept_cnt, &tot, sm_scan);
    kept_carry += tot;
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      const int n = n0 + e;
      if (n >= N) continue;
      if (kp[e]) {
        if (pos < (unsigned)B) a.kept[(int64_t)row * B + pos] = n;
        ++pos;
      }
      if (a.tag) a.tag[(int64_t)row * N + n] = tg[e];
    }
  }
  if (tid == 0) a.n_stage1[row] = k1;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" size_t svlm_select_workspace(int R, int n_vis) {
  (void)R;
  (void)n_vis;
  return 0;  // everything lives in registers and LDS
}

extern "C" int svlm_select(const float* scores, int64_t row_stride, int R, int F, int H, int W, double top_p,
                           int budget, int32_t* kept, int32_t* n_stage1, uint8_t* tag, void* ws, size_t ws_bytes,
                           void* stream) {
  (void)ws;
  (void)ws_bytes;
  if (R < 0 || F < 1 || H < 1 || W < 1) return fail(SVLM_E_INVALID, "svlm_select: R >= 0 and F, H, W >= 1 required");
  const int64_t N = (int64_t)F * H * W;
  if (N > (1 << 18)) return fail(SVLM_E_UNSUPPORTED, "svlm_select: n_vis = F*H*W must be <= 2^18 (got %lld)", (long long)N);
  if (budget < 0 || budget > N) return fail(SVLM_E_INVALID, "svlm_select: budget %d outside [0, %lld]", budget, (long long)N);
  if (std::isnan(top_p)) return fail(SVLM_E_INVALID, "svlm_select: top_p is NaN");
  if (R == 0) return SVLM_OK;
  if (!scores || !n_stage1 || (budget > 0 && !kept)) return fail(SVLM_E_INVALID, "svlm_select: null pointer");
  if (row_stride < N) return fail(SVLM_E_INVALID, "svlm_select: row_stride must be >= F*H*W");
  SelArgs a;
  a.scores = scores;
  a.row_stride = row_stride;
  a.N = (int)N;
  a.budget = budget;
  a.gh_gw = H * W;
  a.top_p = top_p;
  a.kept = kept;
  a.n_stage1 = n_stage1;
  a.tag = tag;
  select_rows<<<R, kThreads, 0, (hipStream_t)stream>>>(a);
  return check_launch("svlm_select");
}
