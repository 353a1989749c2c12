// svlm_verify: acceptance of gamma drafted tokens.
//
// Greedy: Sparse-to-Dense explainer, technical summary, "decoding process"
// (longest prefix of the drafts that matches the dense model's predictions,
// plus one bonus token).  Rejection sampling: ParallelVLM notes, background
// and "parallel decoding" (rejection sampling keeps the target's output
// distribution; a rejected token is resampled from the target), taken as the
// standard speculative-sampling rule: accept d_i iff u_i * q_i(d_i) <=
// p_i(d_i); at the first rejection draw from max(0, p_i - q_i), else draw the
// bonus from p_gamma.  The draw is a fixed-point (2^-40) inverse CDF, so the
// result is exact integer arithmetic and independent of reduction order.
//
// One launch per call: a chunk pass spread over the vocabulary (argmax per
// row for greedy; masses and argmax of the row to draw from for rejection,
// with every candidate row's chunk loaded up front on windows of up to 9);
// the last workgroup of a sequence to finish its chunk (an arrival counter
// per sequence in the workspace) then reduces the chunk results in chunk
// order and, for rejection, walks the one chunk where the inverse CDF lands.
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kThreads * kPerThread;  // 4096 vocabulary entries per rejection chunk
// greedy chunks are 4x longer: (gamma + 1) x chunks workgroups each count in
// on the sequence's arrival counter, and fewer, longer chunks keep that count
// (and its device-scope release per workgroup) low while a thread's 64 loads
// still go out in one round trip
constexpr int kGreedyPerThread = 64;
// rejection windows of at most kPfMaxGamma drafts load every candidate row's
// chunk at once: 1024-entry chunks keep those (2 gamma + 1) x 4 values per
// thread in registers
constexpr int kPfMaxGamma = 9;
constexpr int kPfPerThread = 4;
constexpr int kGreedyChunk = kThreads * kGreedyPerThread;  // 16384

struct ArgMax {
  float v;
  int i;
};

// larger value wins; equal values -> lower index (associative and commutative)
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  if (b.v > a.v || (b.v == a.v && b.i < a.i)) return b;
  return a;
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    ArgMax o;
    o.v = __shfl_xor(a.v, off);
    o.i = __shfl_xor(a.i, off);
    a = better(a, o);
  }
  return a;
}

__device__ __forceinline__ uint64_t mass40(float w) {
  // floor(w * 2^40) for w in [0, 1]: the product is exact in fp32, truncation is floor
  return (uint64_t)(w * 0x1p40f);
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

struct VerifyArgs {
  int batch, gamma, V, chunks;
  const int32_t* draft;
  const float* target;  // [B][gamma+1][V]
  const float* q;       // [B][gamma][V]
  const float* u;       // [B][gamma+1]
  int32_t* n_accept;
  int32_t* next_tok;
  ArgMax* g_part;       // greedy: [B][gamma+1][chunks]
  uint64_t* r_mass;     // reject: [B][chunks][2]  (residual-or-bonus row, fallback row)
  ArgMax* r_arg;        // reject: [B][chunks]
  uint32_t* arrived;    // [B] arrival counters: zero between calls
};

// Called by every thread once the workgroup's results are stored (by thread
// 0).  Counts the workgroup in for sequence b and returns true in all threads
// of the one workgroup that arrives last, which resets the counter.  The
// count is an acquire-release atomic at device scope: the results stored
// before it by every workgroup are visible to the last one after it.
__device__ __forceinline__ bool arrive_last(const VerifyArgs& a, int b, uint32_t expected) {
  __shared__ int s_last;
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(&a.arrived[b], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == expected - 1;
    if (last) __hip_atomic_store(&a.arrived[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

__device__ __forceinline__ int clamp_tok(int t, int V) {
  debug_check(t >= 0 && t < V, SVLM_DBG_DRAFT_TOKEN);
  return min(max(t, 0), V - 1);
}

// first rejected position (gamma if all accepted); identical in every
// workgroup.  Called by one whole wave: lane i tests position i0 + i, all
// tests of a round issue their loads together, and the lowest rejecting
// position is the first set bit of the ballot.  Every lane returns it.
__device__ int first_reject_wave(const VerifyArgs& a, int b) {
  const int G = a.gamma;
  const int lane = threadIdx.x & 63;
  for (int i0 = 0; i0 < G; i0 += 64) {
    const int i = i0 + lane;
    bool rej = false;
    if (i < G) {
      const int d = clamp_tok(a.draft[(int64_t)b * G + i], a.V);
      const double pd = a.target[((int64_t)b * (G + 1) + i) * a.V + d];
      const double qd = a.q[((int64_t)b * G + i) * a.V + d];
      const double ui = a.u[(int64_t)b * (G + 1) + i];
      debug_check(pd >= 0.0 && pd <= 1.0 && qd >= 0.0 && qd <= 1.0, SVLM_DBG_PROB_RANGE);
      rej = !(ui * qd <= pd);
    }
    const unsigned long long m = __builtin_amdgcn_ballot_w64(rej);
    if (m != 0ull) return i0 + (int)__builtin_ctzll(m);
  }
  return G;
}

// the last workgroup of sequence b, 64 rows of the window at a time: wave w
// reduces the chunk results of rows w, w + 4, ... (every load of a round
// issued before any reduction), then wave 0 compares the rows' argmaxes with
// the drafts (one lane per row, loaded alongside) and the first mismatch, or
// the bonus row, is the lowest set bit of a ballot
__device__ void greedy_final(const VerifyArgs& a, int b) {
  constexpr int kRowsPerWave = 64 / (kThreads / 64);
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int G = a.gamma;
  __shared__ int s_am[64];
  __shared__ int s_done;
  for (int i0 = 0; i0 <= G; i0 += 64) {
    const int rows = min(64, G + 1 - i0);
    const int dtok = (tid < rows && i0 + tid < G) ? a.draft[(int64_t)b * G + i0 + tid] : 0;
    ArgMax best[kRowsPerWave];
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) best[k] = ArgMax{-INFINITY, 0x7fffffff};
    for (int c0 = 0; c0 < a.chunks; c0 += 64) {
      const int c = c0 + lane;
      ArgMax v[kRowsPerWave];
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) {
        const int r = wv + (kThreads / 64) * k;
        v[k] = (r < rows && c < a.chunks) ? a.g_part[((int64_t)b * (G + 1) + i0 + r) * a.chunks + c]
                                          : ArgMax{-INFINITY, 0x7fffffff};
      }
#pragma unroll
      for (int k = 0; k < kRowsPerWave; ++k) best[k] = better(best[k], v[k]);
    }
#pragma unroll
    for (int k = 0; k < kRowsPerWave; ++k) {
      const int r = wv + (kThreads / 64) * k;
      if (r < rows) {  // wave-uniform
        const ArgMax m = wave_argmax(best[k]);
        if (lane == 0) s_am[r] = (m.i == 0x7fffffff) ? 0 : m.i;  // all entries NaN: token 0
      }
    }
    __syncthreads();
    if (wv == 0) {
      const int i = i0 + lane;
      if (lane < rows && i < G) debug_check(dtok >= 0 && dtok < a.V, SVLM_DBG_DRAFT_TOKEN);
      const int am = (lane < rows) ? s_am[lane] : 0;
      const bool stop = lane < rows && (i == G || dtok != am);
      const unsigned long long m = __builtin_amdgcn_ballot_w64(stop);
      if (m != 0ull && lane == (int)__builtin_ctzll(m)) {
        a.n_accept[b] = i;
        a.next_tok[b] = am;
      }
      if (lane == 0) s_done = (m != 0ull);
    }
    __syncthreads();
    if (s_done) return;
  }
}

__global__ __launch_bounds__(kThreads) void greedy_chunks(VerifyArgs a) {
  const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const float* row = a.target + ((int64_t)b * (a.gamma + 1) + i) * a.V;
  const int base = c * kGreedyChunk;
  // all loads first (indices clamped into the row, so none is conditional), then the reduction
  float x[kGreedyPerThread];
#pragma unroll
  for (int k = 0; k < kGreedyPerThread; ++k) x[k] = row[min(base + k * kThreads + (int)threadIdx.x, a.V - 1)];
  ArgMax best = {-INFINITY, 0x7fffffff};
#pragma unroll
  for (int k = 0; k < kGreedyPerThread; ++k) {
    const int v = base + k * kThreads + threadIdx.x;
    if (v < a.V) best = better(best, ArgMax{x[k], v});
  }
  best = wave_argmax(best);
  __shared__ ArgMax sm[kThreads / 64];
  if ((threadIdx.x & 63) == 0) sm[threadIdx.x >> 6] = best;
  __syncthreads();
  if (threadIdx.x == 0) {
    ArgMax r = sm[0];
    for (int w = 1; w < kThreads / 64; ++w) r = better(r, sm[w]);
    a.g_part[((int64_t)b * (a.gamma + 1) + i) * a.chunks + c] = r;
  }
  if (arrive_last(a, b, (uint32_t)a.chunks * (uint32_t)(a.gamma + 1))) greedy_final(a, b);
}

// the last workgroup of sequence b (first rejection at n, or n == gamma):
// row totals over the chunk results, the chunk where the inverse CDF with
// uniform uu lands, then that chunk walked in index order
template <int PT>
__device__ void reject_final(const VerifyArgs& a, int b, int n, double uu) {
  constexpr int kCh = kThreads * PT;  // vocabulary entries per chunk
  const int G = a.gamma;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  __shared__ int sm_mode, sm_chunk, sm_tok;
  __shared__ uint64_t sm_t;
  __shared__ uint64_t s_excl[kThreads / 64];
  __shared__ uint64_t s_w[kThreads / 64], s_p[kThreads / 64];
  __shared__ ArgMax s_a[kThreads / 64];
  // row totals over the chunks (chunk-parallel; integer sums are exact in any
  // order); a thread keeps the masses of its first chunk for the ordered scan
  uint64_t mw = 0, mp = 0, first_w = 0, first_p = 0;
  ArgMax best = {-INFINITY, 0x7fffffff};
  for (int c = tid; c < a.chunks; c += kThreads) {
    const uint64_t xw = a.r_mass[((int64_t)b * a.chunks + c) * 2 + 0];
    const uint64_t xp = a.r_mass[((int64_t)b * a.chunks + c) * 2 + 1];
    if (c == tid) {
      first_w = xw;
      first_p = xp;
    }
    mw += xw;
    mp += xp;
    best = better(best, a.r_arg[(int64_t)b * a.chunks + c]);
  }
  mw = wave_sum_u64(mw);
  mp = wave_sum_u64(mp);
  best = wave_argmax(best);
  if (lane == 0) {
    s_w[wv] = mw;
    s_p[wv] = mp;
    s_a[wv] = best;
  }
  __syncthreads();
  uint64_t Ww = 0, Wp = 0;
  ArgMax bb = s_a[0];
#pragma unroll
  for (int w = 0; w < kThreads / 64; ++w) {
    Ww += s_w[w];
    Wp += s_p[w];
    if (w) bb = better(bb, s_a[w]);
  }
  // 0: residual / bonus row, 1: fallback to p_n, 2: argmax of p_n
  const int mode0 = (Ww > 0) ? 0 : (Wp > 0) ? 1 : 2;
  const uint64_t W = (mode0 == 0) ? Ww : Wp;
  uint64_t t = 0;
  if (mode0 < 2) {
    t = (uint64_t)floor(uu * (double)W);
    if (t > W - 1) t = W - 1;
  }
  if (tid == 0) {
    sm_mode = mode0;
    sm_tok = (bb.i == 0x7fffffff) ? 0 : bb.i;
    sm_chunk = a.chunks - 1;
    sm_t = 0;
  }
  if (mode0 < 2) {
    // the chunk whose cumulative mass passes t: an ordered scan of the chunk
    // masses, kThreads chunks per round
    uint64_t carry = 0;
    for (int c0 = 0; c0 < a.chunks; c0 += kThreads) {
      const int c = c0 + tid;
      // the first round's masses are already in registers
      const uint64_t m = (c >= a.chunks) ? 0ull
                         : (c0 == 0)     ? ((mode0 == 0) ? first_w : first_p)
                                         : a.r_mass[((int64_t)b * a.chunks + c) * 2 + mode0];
      uint64_t incl = m;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint64_t y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      __syncthreads();  // s_excl of the previous round is read
      if (lane == 63) s_excl[wv] = incl;
      __syncthreads();
      uint64_t before = carry;
      uint64_t total = carry;
#pragma unroll
      for (int w = 0; w < kThreads / 64; ++w) {
        if (w < wv) before += s_excl[w];
        total += s_excl[w];
      }
      const uint64_t excl = before + incl - m;
      if (m > 0 && excl <= t && t < excl + m) {
        sm_chunk = c;
        sm_t = t - excl;
      }
      if (total > t) break;  // uniform: every thread has the same total
      carry = total;
    }
  }
  __syncthreads();
  const int mode = sm_mode;
  if (mode == 2) {
    if (tid == 0) {
      a.n_accept[b] = n;
      a.next_tok[b] = sm_tok;
    }
    return;
  }
  // walk the chosen chunk in index order: thread t owns [base + PT t, base + PT t + PT)
  const float* prow = a.target + ((int64_t)b * (G + 1) + n) * a.V;
  const float* qrow = (n < G && mode == 0) ? a.q + ((int64_t)b * G + n) * a.V : nullptr;
  const int base = sm_chunk * kCh + tid * PT;
  float w[PT], qv[PT];
#pragma unroll
  for (int k = 0; k < PT; ++k) {  // loads first, indices clamped into the row
    const int v = min(base + k, a.V - 1);
    w[k] = prow[v];
    qv[k] = qrow ? qrow[v] : 0.f;
  }
  uint64_t mine = 0;
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const float p = w[k];
    const float x = (base + k < a.V) ? (qrow ? fmaxf(p - qv[k], 0.f) : p) : 0.f;
    w[k] = x;
    mine += mass40(x);
  }
  // exclusive scan of per-thread masses
  uint64_t incl = mine;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) s_excl[wv] = incl;
  __syncthreads();
  uint64_t before = 0;
  for (int w2 = 0; w2 < wv; ++w2) before += s_excl[w2];
  const uint64_t excl = before + incl - mine;
  const uint64_t tc = sm_t;  // target offset inside the chosen chunk
  if (mine > 0 && excl <= tc && tc < excl + mine) {
    uint64_t cum = excl;
    int tok = base + PT - 1;
    for (int k = 0; k < PT; ++k) {
      cum += mass40(w[k]);
      if (cum > tc) { tok = base + k; break; }
    }
    a.n_accept[b] = n;
    a.next_tok[b] = tok;
  }
}


// The chunk's masses (residual row or bonus row, the fallback row p) and
// argmax of p, stored by thread 0 for the last workgroup.
template <int PT>
__device__ __forceinline__ void reject_chunk_masses(const VerifyArgs& a, int b, int c, bool has_q,
                                                    const float (&pv)[PT], const float (&qv)[PT]) {
  const int base = c * kThreads * PT;
  uint64_t mw = 0, mp = 0;
  ArgMax best = {-INFINITY, 0x7fffffff};
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    const int v = base + k * kThreads + threadIdx.x;
    if (v < a.V) {
      const float p = pv[k];
      const float w = has_q ? fmaxf(p - qv[k], 0.f) : p;
      mw += mass40(w);
      mp += mass40(p);
      best = better(best, ArgMax{p, v});
    }
  }
  mw = wave_sum_u64(mw);
  mp = wave_sum_u64(mp);
  best = wave_argmax(best);
  __shared__ uint64_t sw[kThreads / 64], sp[kThreads / 64];
  __shared__ ArgMax sa[kThreads / 64];
  const int wv = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sw[wv] = mw;
    sp[wv] = mp;
    sa[wv] = best;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint64_t tw = 0, tp = 0;
    ArgMax r = sa[0];
    for (int w = 0; w < kThreads / 64; ++w) {
      tw += sw[w];
      tp += sp[w];
      if (w) r = better(r, sa[w]);
    }
    a.r_mass[((int64_t)b * a.chunks + c) * 2 + 0] = tw;
    a.r_mass[((int64_t)b * a.chunks + c) * 2 + 1] = tp;
    a.r_arg[(int64_t)b * a.chunks + c] = r;
  }
}

// Any window: the first rejection n first, then the chunk of row n (p_n and
// q_n, or the bonus row p_gamma).
__global__ __launch_bounds__(kThreads) void reject_chunks(VerifyArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  __shared__ int sm_n;
  if (threadIdx.x < 64) {
    const int n0 = first_reject_wave(a, b);
    if (threadIdx.x == 0) sm_n = n0;
  }
  __syncthreads();
  const int n = sm_n;
  const int G = a.gamma;
  const double uu = a.u[(int64_t)b * (G + 1) + G];  // the draw's uniform, used by the last workgroup
  const float* prow = a.target + ((int64_t)b * (G + 1) + n) * a.V;
  const float* qrow = (n < G) ? a.q + ((int64_t)b * G + n) * a.V : nullptr;
  const int base = c * kChunk;
  // all loads first (indices clamped into the row, so none is conditional), then the sums
  float pv[kPerThread], qv[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int v = min(base + k * kThreads + (int)threadIdx.x, a.V - 1);
    pv[k] = prow[v];
    qv[k] = qrow ? qrow[v] : 0.f;
  }
  reject_chunk_masses<kPerThread>(a, b, c, qrow != nullptr, pv, qv);
  if (arrive_last(a, b, (uint32_t)a.chunks)) reject_final<kPerThread>(a, b, n, uu);
}

// Windows of at most GMAX drafts: the chunk of every row the draw could take
// (p_0 .. p_gamma and q_0 .. q_gamma-1) is loaded while the first rejection
// is found, so the row's values are in registers when n is known.  One memory
// round trip less than the generic form, for 2 gamma + 1 rows read instead of
// two.  Wave 0's draft tokens and uniforms are loaded before the rows, so its
// wait for them does not wait for the rows (loads complete in issue order).
template <int GMAX>
__global__ __launch_bounds__(kThreads) void reject_chunks_pf(VerifyArgs a) {
  constexpr int PT = kPfPerThread;
  const int c = blockIdx.x, b = blockIdx.y;
  const int G = a.gamma;  // <= GMAX
  const int lane = threadIdx.x & 63;
  __shared__ int sm_n;
  int dtok = 0;
  double ui = 0.0;
  if (threadIdx.x < 64 && lane < G) {
    dtok = a.draft[(int64_t)b * G + lane];
    ui = a.u[(int64_t)b * (G + 1) + lane];
  }
  const double uu = a.u[(int64_t)b * (G + 1) + G];
  const int base = c * kThreads * PT;
  float pv[GMAX + 1][PT], qv[GMAX][PT];
#pragma unroll
  for (int r = 0; r <= GMAX; ++r) {
    if (r <= G) {
      const float* row = a.target + ((int64_t)b * (G + 1) + r) * a.V;
#pragma unroll
      for (int k = 0; k < PT; ++k) pv[r][k] = row[min(base + k * kThreads + (int)threadIdx.x, a.V - 1)];
    }
  }
#pragma unroll
  for (int r = 0; r < GMAX; ++r) {
    if (r < G) {
      const float* row = a.q + ((int64_t)b * G + r) * a.V;
#pragma unroll
      for (int k = 0; k < PT; ++k) qv[r][k] = row[min(base + k * kThreads + (int)threadIdx.x, a.V - 1)];
    }
  }
  if (threadIdx.x < 64) {
    bool rej = false;
    if (lane < G) {
      const int d = clamp_tok(dtok, a.V);
      const double pd = a.target[((int64_t)b * (G + 1) + lane) * a.V + d];
      const double qd = a.q[((int64_t)b * G + lane) * a.V + d];
      debug_check(pd >= 0.0 && pd <= 1.0 && qd >= 0.0 && qd <= 1.0, SVLM_DBG_PROB_RANGE);
      rej = !(ui * qd <= pd);
    }
    const unsigned long long m = __builtin_amdgcn_ballot_w64(rej);
    if (threadIdx.x == 0) sm_n = (m != 0ull) ? (int)__builtin_ctzll(m) : G;
  }
  __syncthreads();
  const int n = sm_n;
  float ps[PT], qs[PT];
#pragma unroll
  for (int k = 0; k < PT; ++k) {
    ps[k] = 0.f;
    qs[k] = 0.f;
  }
#pragma unroll
  for (int r = 0; r <= GMAX; ++r)
    if (r == n) {  // uniform
#pragma unroll
      for (int k = 0; k < PT; ++k) ps[k] = pv[r][k];
    }
#pragma unroll
  for (int r = 0; r < GMAX; ++r)
    if (r == n) {
#pragma unroll
      for (int k = 0; k < PT; ++k) qs[k] = qv[r][k];
    }
  reject_chunk_masses<PT>(a, b, c, n < G, ps, qs);
  if (arrive_last(a, b, (uint32_t)a.chunks)) reject_final<PT>(a, b, n, uu);
}

}  // namespace
}  // namespace svlm

using namespace svlm;

static int verify_chunks(int V) { return (int)(((int64_t)V + kChunk - 1) / kChunk); }
static int greedy_chunks_of(int V) { return (int)(((int64_t)V + kGreedyChunk - 1) / kGreedyChunk); }
static int pf_chunks(int V) { return (int)(((int64_t)V + kThreads * kPfPerThread - 1) / (kThreads * kPfPerThread)); }

// the greedy pass is a (chunks, gamma + 1, batch) grid, the rejection pass
// (chunks, batch); the prefetching rejection form has the most chunks
static bool verify_fits(int batch, int gamma, int V) {
  return grid_fits(pf_chunks(V), kThreads, (int64_t)gamma + 1, batch);
}

// The workspace opens with one arrival counter per possible sequence (the
// batch stays below 65536), so the counters sit at the same place whatever
// the call's shape and the chunk results of one call never land on another
// call's counters; the chunk results follow them.
constexpr size_t kCounterBytes = (size_t)65536 * sizeof(uint32_t);

static size_t verify_results_bytes(int batch, int gamma, int V) {
  const size_t greedy = (size_t)batch * ((size_t)gamma + 1) * (size_t)greedy_chunks_of(V) * sizeof(ArgMax);
  // rejection: the prefetching form's shorter chunks (the larger count)
  const size_t reject = (size_t)batch * (size_t)pf_chunks(V) * (2 * sizeof(uint64_t) + sizeof(ArgMax));
  return greedy > reject ? greedy : reject;
}

extern "C" size_t svlm_verify_workspace(int batch, int gamma, int V) {
  if (batch < 1 || gamma < 1 || V < 1 || !verify_fits(batch, gamma, V)) return 0;
  return kCounterBytes + verify_results_bytes(batch, gamma, V);
}

extern "C" int svlm_verify(int mode, int batch, int gamma, int V, const int32_t* draft_tok, const float* target,
                           const float* draft_prob, const float* u, int32_t* n_accept, int32_t* next_tok, void* ws,
                           size_t ws_bytes, void* stream) {
  if (mode != SVLM_VERIFY_GREEDY && mode != SVLM_VERIFY_REJECT)
    return fail(SVLM_E_INVALID, "svlm_verify: mode must be SVLM_VERIFY_GREEDY or SVLM_VERIFY_REJECT");
  if (batch < 1 || gamma < 1 || V < 1) return fail(SVLM_E_INVALID, "svlm_verify: batch, gamma, V must be >= 1");
  if (!draft_tok || !target || !n_accept || !next_tok) return fail(SVLM_E_INVALID, "svlm_verify: null pointer");
  if (!verify_fits(batch, gamma, V))
    return fail(SVLM_E_UNSUPPORTED, "svlm_verify: batch %d and gamma %d must stay below 65536", batch, gamma);
  if (mode == SVLM_VERIFY_REJECT && (!draft_prob || !u))
    return fail(SVLM_E_INVALID, "svlm_verify: rejection mode needs draft_prob and u");
  const size_t need = svlm_verify_workspace(batch, gamma, V);
  if (!ws || ws_bytes < need)
    return fail(SVLM_E_WORKSPACE, "svlm_verify: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
  if (!aligned16(ws)) return fail(SVLM_E_INVALID, "svlm_verify: workspace must be 16-byte aligned");
  VerifyArgs a;
  a.batch = batch;
  a.gamma = gamma;
  a.V = V;
  // chunk count of the form that runs
  a.chunks = (mode == SVLM_VERIFY_GREEDY) ? greedy_chunks_of(V) : (gamma <= kPfMaxGamma) ? pf_chunks(V) : verify_chunks(V);
  a.draft = draft_tok;
  a.target = target;
  a.q = draft_prob;
  a.u = u;
  a.n_accept = n_accept;
  a.next_tok = next_tok;
  a.arrived = (uint32_t*)ws;
  char* results = (char*)ws + kCounterBytes;
  a.g_part = (ArgMax*)results;
  a.r_mass = (uint64_t*)results;
  a.r_arg = (ArgMax*)((uint64_t*)results + (size_t)batch * a.chunks * 2);
  hipStream_t st = (hipStream_t)stream;
  if (mode == SVLM_VERIFY_GREEDY)
    greedy_chunks<<<dim3(a.chunks, gamma + 1, batch), kThreads, 0, st>>>(a);
  else if (gamma <= kPfMaxGamma)
    reject_chunks_pf<kPfMaxGamma><<<dim3(a.chunks, batch), kThreads, 0, st>>>(a);
  else
    reject_chunks<<<dim3(a.chunks, batch), kThreads, 0, st>>>(a);
  return check_launch("svlm_verify");
}

#ifdef SVLM_DEBUG
bool svlm::debug_take_verify(unsigned* out) { return debug_take_here(out); }
#endif
