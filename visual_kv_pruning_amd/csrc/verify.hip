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
// Two launches per call: a chunk pass spread over the vocabulary (argmax per
// row for greedy; masses and argmax of the row to draw from for rejection),
// then one workgroup per sequence that reduces the chunk results in chunk
// order and, for rejection, walks the one chunk where the inverse CDF lands.
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr int kThreads = 256;
constexpr int kPerThread = 16;
constexpr int kChunk = kThreads * kPerThread;  // 4096 vocabulary entries per chunk

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
  int32_t* r_first;     // reject: [B] first rejected position (written by chunk 0)
};

__device__ __forceinline__ int clamp_tok(int t, int V) { return min(max(t, 0), V - 1); }

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
      rej = !(ui * qd <= pd);
    }
    const unsigned long long m = __builtin_amdgcn_ballot_w64(rej);
    if (m != 0ull) return i0 + (int)__builtin_ctzll(m);
  }
  return G;
}

__global__ __launch_bounds__(kThreads) void greedy_chunks(VerifyArgs a) {
  const int c = blockIdx.x, i = blockIdx.y, b = blockIdx.z;
  const float* row = a.target + ((int64_t)b * (a.gamma + 1) + i) * a.V;
  const int base = c * kChunk;
  // all loads first (indices clamped into the row, so none is conditional), then the reduction
  float x[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) x[k] = row[min(base + k * kThreads + (int)threadIdx.x, a.V - 1)];
  ArgMax best = {-INFINITY, 0x7fffffff};
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
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
}

// one workgroup per sequence: the waves reduce the chunk results of up to 64
// rows at a time (a row per wave in turn), then thread 0 walks them in row
// order to the first draft that differs from the dense argmax
__global__ __launch_bounds__(kThreads) void greedy_final(VerifyArgs a) {
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ int s_am[64];
  __shared__ int s_done;
  for (int i0 = 0; i0 <= a.gamma; i0 += 64) {
    const int rows = min(64, a.gamma + 1 - i0);
    for (int r = wv; r < rows; r += kThreads / 64) {
      const int i = i0 + r;
      ArgMax best = {-INFINITY, 0x7fffffff};
      for (int c = lane; c < a.chunks; c += 64)
        best = better(best, a.g_part[((int64_t)b * (a.gamma + 1) + i) * a.chunks + c]);
      best = wave_argmax(best);
      if (lane == 0) s_am[r] = (best.i == 0x7fffffff) ? 0 : best.i;  // all entries NaN: token 0
    }
    __syncthreads();
    if (tid == 0) {
      int done = 0;
      for (int r = 0; r < rows; ++r) {
        const int i = i0 + r;
        const int am = s_am[r];
        if (i == a.gamma || a.draft[(int64_t)b * a.gamma + i] != am) {
          a.n_accept[b] = i;
          a.next_tok[b] = am;
          done = 1;
          break;
        }
      }
      s_done = done;
    }
    __syncthreads();
    if (s_done) return;
  }
}

__global__ __launch_bounds__(kThreads) void reject_chunks(VerifyArgs a) {
  const int c = blockIdx.x, b = blockIdx.y;
  __shared__ int sm_n;
  if (threadIdx.x < 64) {
    const int n0 = first_reject_wave(a, b);
    if (threadIdx.x == 0) {
      sm_n = n0;
      if (c == 0) a.r_first[b] = n0;
    }
  }
  __syncthreads();
  const int n = sm_n;
  const int G = a.gamma;
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
  uint64_t mw = 0, mp = 0;
  ArgMax best = {-INFINITY, 0x7fffffff};
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    const int v = base + k * kThreads + threadIdx.x;
    if (v < a.V) {
      const float p = pv[k];
      const float w = qrow ? fmaxf(p - qv[k], 0.f) : p;
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

__global__ __launch_bounds__(kThreads) void reject_final(VerifyArgs a) {
  const int b = blockIdx.x;
  const int G = a.gamma;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wv = tid >> 6;
  __shared__ int sm_n, sm_mode, sm_chunk, sm_tok;
  __shared__ uint64_t sm_t;
  __shared__ uint64_t s_excl[kThreads / 64];
  __shared__ uint64_t s_w[kThreads / 64], s_p[kThreads / 64];
  __shared__ ArgMax s_a[kThreads / 64];
  if (tid == 0) sm_n = a.r_first[b];
  // row totals over the chunks (chunk-parallel; integer sums are exact in any order)
  uint64_t mw = 0, mp = 0;
  ArgMax best = {-INFINITY, 0x7fffffff};
  for (int c = tid; c < a.chunks; c += kThreads) {
    mw += a.r_mass[((int64_t)b * a.chunks + c) * 2 + 0];
    mp += a.r_mass[((int64_t)b * a.chunks + c) * 2 + 1];
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
    const double uu = a.u[(int64_t)b * (G + 1) + G];
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
      const uint64_t m = (c < a.chunks) ? a.r_mass[((int64_t)b * a.chunks + c) * 2 + mode0] : 0ull;
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
  const int n = sm_n;
  const int mode = sm_mode;
  if (mode == 2) {
    if (tid == 0) {
      a.n_accept[b] = n;
      a.next_tok[b] = sm_tok;
    }
    return;
  }
  // walk the chosen chunk in index order: thread t owns [base + 16t, base + 16t + 16)
  const float* prow = a.target + ((int64_t)b * (G + 1) + n) * a.V;
  const float* qrow = (n < G && mode == 0) ? a.q + ((int64_t)b * G + n) * a.V : nullptr;
  const int base = sm_chunk * kChunk + tid * kPerThread;
  float w[kPerThread], qv[kPerThread];
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {  // loads first, indices clamped into the row
    const int v = min(base + k, a.V - 1);
    w[k] = prow[v];
    qv[k] = qrow ? qrow[v] : 0.f;
  }
  uint64_t mine = 0;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
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
    int tok = base + kPerThread - 1;
    for (int k = 0; k < kPerThread; ++k) {
      cum += mass40(w[k]);
      if (cum > tc) { tok = base + k; break; }
    }
    a.n_accept[b] = n;
    a.next_tok[b] = tok;
  }
}

}  // namespace
}  // namespace svlm

using namespace svlm;

static int verify_chunks(int V) { return (V + kChunk - 1) / kChunk; }

extern "C" size_t svlm_verify_workspace(int batch, int gamma, int V) {
  if (batch < 1 || gamma < 1 || V < 1) return 0;
  const size_t ch = (size_t)verify_chunks(V);
  const size_t greedy = (size_t)batch * (gamma + 1) * ch * sizeof(ArgMax);
  const size_t reject = (size_t)batch * ch * (2 * sizeof(uint64_t) + sizeof(ArgMax)) + (size_t)batch * sizeof(int32_t);
  return (greedy > reject ? greedy : reject) + 256;
}

extern "C" int svlm_verify(int mode, int batch, int gamma, int V, const int32_t* draft_tok, const float* target,
                           const float* draft_prob, const float* u, int32_t* n_accept, int32_t* next_tok, void* ws,
                           size_t ws_bytes, void* stream) {
  if (mode != SVLM_VERIFY_GREEDY && mode != SVLM_VERIFY_REJECT)
    return fail(SVLM_E_INVALID, "svlm_verify: mode must be SVLM_VERIFY_GREEDY or SVLM_VERIFY_REJECT");
  if (batch < 1 || gamma < 1 || V < 1) return fail(SVLM_E_INVALID, "svlm_verify: batch, gamma, V must be >= 1");
  if (!draft_tok || !target || !n_accept || !next_tok) return fail(SVLM_E_INVALID, "svlm_verify: null pointer");
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
  a.chunks = verify_chunks(V);
  a.draft = draft_tok;
  a.target = target;
  a.q = draft_prob;
  a.u = u;
  a.n_accept = n_accept;
  a.next_tok = next_tok;
  a.g_part = (ArgMax*)ws;
  a.r_mass = (uint64_t*)ws;
  a.r_arg = (ArgMax*)((uint64_t*)ws + (size_t)batch * a.chunks * 2);
  a.r_first = (int32_t*)(a.r_arg + (size_t)batch * a.chunks);
  hipStream_t st = (hipStream_t)stream;
  if (mode == SVLM_VERIFY_GREEDY) {
    greedy_chunks<<<dim3(a.chunks, gamma + 1, batch), kThreads, 0, st>>>(a);
    greedy_final<<<batch, kThreads, 0, st>>>(a);
  } else {
    reject_chunks<<<dim3(a.chunks, batch), kThreads, 0, st>>>(a);
    reject_final<<<batch, kThreads, 0, st>>>(a);
  }
  return check_launch("svlm_verify");
}
