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
// doubles.  The stage-I threshold key is found by a four-level radix descent
// (8 bits of the fp32 key per level) over per-wave LDS histograms of integer
// (count, mass), so the result does not depend on the order of the additions.
// A thread owns a contiguous run of tokens; one ordered block scan of its
// (above-threshold, tie) counts gives every token its stage-I rank, and the
// stage-II picks before any remainder rank have a closed form, so `kept` is
// written ascending without further scans.
//
// Pure top-K on long rows (the hour-long case: 112 rows of 141120 scores) is
// split: one workgroup per row segment finds the segment's top K, and a
// second pass takes the top K of the candidates, so the chip is not left with
// one workgroup per row.
#pragma clang fp contract(off)

#include <algorithm>
#include <cmath>

#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kRegKeys = 32;  // keys per thread held in registers (rows up to 32768 tokens)
constexpr int kSegRegKeys = 36;   // keys per thread in the segment pass of the split top-K
constexpr int kChunkRunKeys = 16;  // keys per thread per chunk for longer rows (fits 128 VGPRs)
constexpr int kCopies = 32;
constexpr int kCntStride = 257;   // words
constexpr int kMassStride = 257;  // 8-byte words

struct SelArgs {
  const float* scores;
  int64_t row_stride;
  int N, budget;
  double top_p;
  int32_t* kept;
  int64_t kept_stride;
  int32_t* n_stage1;  // may be NULL (segment pass)
  uint8_t* tag;
  // split top-K.  Segment pass: workgroup w takes segment p = w % segs of row
  // r = w / segs (seg_len tokens, the last one shorter) with budget
  // min(budget, its length) and writes its kept tokens and their scores to
  // candidate slots r * C + p * budget + j.  Candidate pass: row r is the C
  // candidate scores, and a kept position n is written as cand_tok[r * C + n].
  int segs, seg_len, C;
  float* cand_score;
  int32_t* cand_tok;
};

enum : int { kPlain = 0, kSegmentPass = 1, kCandidatePass = 2 };

__device__ __forceinline__ unsigned key_of(float s) {
  debug_check(s >= 0.f && s <= 1.f, SVLM_DBG_SCORE_RANGE);
  unsigned k = f_bits(s);
  return (k == 0x80000000u) ? 0u : k;       // -0 orders as +0
}

__device__ __forceinline__ uint64_t mass_of_key(unsigned key) {
  return (uint64_t)(bits_f(key) * 0x1p40f);  // exact: power-of-two scale, then floor
}

// wave-wide sum of a 64-bit value (every lane gets it)
__device__ __forceinline__ uint64_t wave_sum64(uint64_t v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

// block-wide exclusive scan (thread order) of two counters packed in 64 bits
// (each part < 2^32; tokens per row < 2^18); *total gets the block's sum
__device__ uint64_t block_excl_scan64(uint64_t x, uint64_t* sm, uint64_t* total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  uint64_t incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint64_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sm[wv] = incl;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    if (w < wv) before += sm[w];
    all += sm[w];
  }
  *total = all;
  return before + incl - x;
}

// Rows of up to kThreads * kRegKeys tokens: each thread's run of tokens lives
// in registers for the whole kernel.  Longer rows (CHUNKED): the row is taken
// in chunks of kThreads * kChunkRunKeys tokens, thread t owning the run of
// kChunkRunKeys tokens at chunk offset t * kChunkRunKeys; every pass loads a chunk's run into
// registers (all loads of a run issued together) and the ordered scans carry
// their totals from chunk to chunk, so raster order and exactness are those
// of the one-chunk case.
// MASS: the row has a Top-P stage I (0 < top_p < 1), so per-token masses are
// summed; pure top-K and fill-only selections count tokens alone.
// KR: keys per thread of a register-resident row when not the default (a
// candidate row of at most kThreads * KR tokens)
template <bool CHUNKED, bool MASS, int SPLIT = kPlain, int KR = kRegKeys>
__global__ __launch_bounds__(kThreads) void select_rows(SelArgs a) {
  constexpr int KREG = CHUNKED ? kChunkRunKeys : (SPLIT == kSegmentPass ? kSegRegKeys : KR);
  // kCopies histogram copies, lane l adding to copy l % kCopies, so that at
  // most 64 / kCopies lanes of a wave meet on one counter (scores cluster in
  // a few exponents, and a shared counter serialises every lane on it); the
  // padded strides put one bin's copies in different banks
  // Rows held in registers share one LDS area between phases: the scores are
  // staged through it with coalesced loads (thread t loads tokens t, t + 1024,
  // ...; word i sits at i + i / 32, so the runs read back without bank
  // conflicts), then it holds the level histograms, then the kept positions
  // on their way to coalesced stores.  Chunked rows keep separate arrays.
  constexpr int kCntWords = kCopies * kCntStride;
  constexpr int kHistBytes = kCntWords * 4 + (MASS ? kCopies * kMassStride * 8 : 0);
  constexpr int kStageWords = kThreads * KREG + (kThreads * KREG) / 32;
  constexpr int kAreaBytes = CHUNKED ? kHistBytes : (kStageWords * 4 > kHistBytes ? kStageWords * 4 : kHistBytes);
  __shared__ __align__(16) unsigned char area[kAreaBytes];
  unsigned* const h_cnt = (unsigned*)area;
  unsigned long long* const h_mass = (unsigned long long*)(area + kCntWords * 4);
  unsigned* const stage = (unsigned*)area;
  // level totals, double-buffered by level parity: every wave derives the
  // level's digit from them, and the next level's totals go to the other
  // buffer, so no barrier is needed after the digit search
  __shared__ unsigned t_cnt[2][256];
  __shared__ unsigned long long t_mass[2][256];
  __shared__ unsigned sm_digit;  // Top-P rows: wave 0's digit and totals, broadcast
  __shared__ unsigned sm_cnt_above;
  __shared__ unsigned long long sm_mass_above;
  __shared__ unsigned long long sm_q[kWaves];
  __shared__ uint64_t sm_scan[kWaves];

  const int row = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const float* srow = a.scores + (int64_t)row * a.row_stride;
  int N = a.N, B = a.budget;
  int64_t cand0 = 0;  // segment pass: this segment's first candidate slot
  int tok0 = 0;       // and its first token
  if constexpr (SPLIT == kSegmentPass) {
    const int r = row / a.segs, p = row - r * a.segs;
    tok0 = p * a.seg_len;
    srow = a.scores + (int64_t)r * a.row_stride + tok0;
    N = min(a.seg_len, a.N - tok0);
    B = min(B, N);
    cand0 = (int64_t)r * a.C + (int64_t)p * a.budget;
  }
  constexpr int kChunk = kThreads * KREG;
  const int n_chunks = CHUNKED ? (N + kChunk - 1) / kChunk : 1;
  // this thread's run of tokens (in the current chunk): [n_begin, n_begin + n_mine)
  const int per = CHUNKED ? KREG : (N + kThreads - 1) / kThreads;
  int n_begin = min(N, tid * per);
  int n_mine = min(per, N - n_begin);

  unsigned keys[KREG];
  auto load_run = [&](int ch) {
    if constexpr (CHUNKED) {
      n_begin = min(N, ch * kChunk + tid * KREG);
      n_mine = max(0, min(KREG, N - n_begin));
    }
    if constexpr (CHUNKED) {
#pragma unroll
      for (int e = 0; e < KREG; ++e) keys[e] = key_of(srow[min(n_begin + e, N - 1)]);  // loads first, unconditional
    } else {
#pragma unroll
      for (int e = 0; e < KREG; ++e) keys[e] = key_of(srow[min(e * kThreads + tid, N - 1)]);
#pragma unroll
      for (int e = 0; e < KREG; ++e) {
        const int i = e * kThreads + tid;
        if (i < N) stage[i + (i >> 5)] = keys[e];
      }
      __syncthreads();
#pragma unroll
      for (int e = 0; e < KREG; ++e) {
        const int i = min(n_begin + e, N - 1);
        keys[e] = stage[i + (i >> 5)];
      }
      __syncthreads();  // the area becomes the histograms
    }
#pragma unroll
    for (int e = 0; e < KREG; ++e) keys[e] = (e < n_mine) ? keys[e] : 0u;
  };
  if constexpr (!CHUNKED) load_run(0);

  // ---- total fixed-point mass of the row
  uint64_t q = 0;
  if constexpr (MASS) {
    for (int ch = 0; ch < n_chunks; ++ch) {
      if constexpr (CHUNKED) load_run(ch);
#pragma unroll
      for (int e = 0; e < KREG; ++e)
        if (e < n_mine) q += mass_of_key(keys[e]);
    }
  }
  q = wave_sum64(q);
  if (lane == 0) sm_q[wv] = q;
  __syncthreads();
  uint64_t Q = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) Q += sm_q[w];

  // ---- stage I: threshold key vstar; cnt_above / mass_above over keys > vstar
  unsigned vstar = 0xFFFFFFFFu;  // nothing taken when k1 == 0
  unsigned cnt_above = 0;
  uint64_t mass_above = 0;
  int k1 = 0, c_ties = 0;
  bool any_stage1 = (B > 0) && (a.top_p > 0.0);
  uint64_t Tm = ~0ull;
  if (any_stage1 && a.top_p < 1.0) {
    Tm = (uint64_t)ceil((double)Q * a.top_p);
    if (Tm == 0) any_stage1 = false;
  }
  if (any_stage1) {
    unsigned prefix = 0;
    for (int i = tid; i < kCopies * kCntStride; i += kThreads) {
      h_cnt[i] = 0u;
      if constexpr (MASS) h_mass[i] = 0ull;
    }
    __syncthreads();
    unsigned* const my_cnt = h_cnt + (lane % kCopies) * kCntStride;
    unsigned long long* const my_mass = h_mass + (lane % kCopies) * kMassStride;
    for (int level = 0; level < 4; ++level) {
      const int shift = 24 - 8 * level;
      // keys under the current prefix, binned by their next 8 bits
      auto bin_key = [&](unsigned key) {
        asm volatile("" : "+v"(key));  // keeps the per-key masses from being hoisted out of the level loop
        if (level == 0 || (key >> (shift + 8)) == (prefix >> (shift + 8))) {
          const unsigned bin = (key >> shift) & 255u;
          atomicAdd(&my_cnt[bin], 1u);
          if constexpr (MASS) atomicAdd(&my_mass[bin], (unsigned long long)mass_of_key(key));
        }
      };
      for (int ch = 0; ch < n_chunks; ++ch) {
        if constexpr (CHUNKED) load_run(ch);
#pragma unroll
        for (int e = 0; e < KREG; ++e)
          if (e < n_mine) bin_key(keys[e]);
      }
      __syncthreads();
      // four threads per bin add up a quarter of its copies each (clearing
      // them for the next level), then combine across the four lanes
      {
        static_assert(kThreads == 4 * 256 && kCopies % 4 == 0, "four threads per bin");
        const int bin = tid >> 2, c0 = (tid & 3) * (kCopies / 4);
        unsigned cc = 0;
        uint64_t mm = 0;
#pragma unroll
        for (int c = c0; c < c0 + kCopies / 4; ++c) {
          cc += h_cnt[c * kCntStride + bin];
          h_cnt[c * kCntStride + bin] = 0u;
          if constexpr (MASS) {
            mm += h_mass[c * kMassStride + bin];
            h_mass[c * kMassStride + bin] = 0ull;
          }
        }
        cc += __shfl_xor(cc, 1);
        cc += __shfl_xor(cc, 2);
        if constexpr (MASS) {
          mm += __shfl_xor(mm, 1);
          mm += __shfl_xor(mm, 2);
        }
        if ((tid & 3) == 0) {
          t_cnt[level & 1][bin] = cc;
          t_mass[level & 1][bin] = mm;
        }
      }
      __syncthreads();
      if constexpr (MASS) {
        // Top-P rows: wave 0 finds the highest digit d whose bins d..255
        // (added to the keys above the prefix) reach the budget or the mass
        // target, and broadcasts it (one wave's 64-bit scans cost less than
        // every wave's)
        if (wv == 0) {
          unsigned c4[4];
          uint64_t m4[4];
          unsigned ct = 0;
          uint64_t mt = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {  // lane holds bins 255 - 4 lane - i (top-down)
            const int bin = 255 - 4 * lane - i;
            c4[i] = t_cnt[level & 1][bin];
            m4[i] = t_mass[level & 1][bin];
            ct += c4[i];
            mt += m4[i];
          }
          uint64_t ci = ct, mi = mt;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const uint64_t yc = __shfl_up(ci, off);
            const uint64_t ym = __shfl_up(mi, off);
            if (lane >= off) {
              ci += yc;
              mi += ym;
            }
          }
          uint64_t cb = ci - ct, mb = mi - mt;
          int found = -1;
          uint64_t c_above_d = 0, m_above_d = 0;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const uint64_t c_incl = cb + c4[i], m_incl = mb + m4[i];
            if (found < 0 && (cnt_above + c_incl >= (uint64_t)B || mass_above + m_incl >= Tm)) {
              found = i;
              c_above_d = cb;
              m_above_d = mb;
            }
            cb = c_incl;
            mb = m_incl;
          }
          // some bin always qualifies: all N >= B keys lie under the prefix at
          // level 0, and the chosen bin qualifies again one level down
          const unsigned long long hit = __builtin_amdgcn_ballot_w64(found >= 0);
          const int first = (hit != 0ull) ? (int)__builtin_ctzll(hit) : 63;
          if (lane == first) {
            sm_digit = (unsigned)(255 - 4 * lane - (found >= 0 ? found : 3));
            sm_cnt_above = cnt_above + (unsigned)c_above_d;
            sm_mass_above = mass_above + m_above_d;
          }
        }
        __syncthreads();
        // read before the next level's wave-0 step rewrites them, which is two
        // barriers away
        prefix |= sm_digit << shift;
        cnt_above = sm_cnt_above;
        mass_above = sm_mass_above;
      } else {
        // count-only rows: every wave finds the digit from the totals itself
        // (the next level's totals go to the other buffer, so no barrier
        // follows)
        const unsigned* const tc = t_cnt[level & 1];
        unsigned c4[4];
        unsigned ct = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {  // lane holds bins 255 - 4 lane - i (top-down)
          c4[i] = tc[255 - 4 * lane - i];
          ct += c4[i];
        }
        // inclusive prefix over lanes, then the part above this lane's bins
        // (counts stay below 2^19)
        unsigned ci = ct;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const unsigned yc = __shfl_up(ci, off);
          if (lane >= off) ci += yc;
        }
        unsigned cb = ci - ct;
        int found = -1;
        unsigned c_above_d = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const unsigned c_incl = cb + c4[i];
          if (found < 0 && cnt_above + c_incl >= (unsigned)B) {
            found = i;
            c_above_d = cb;
          }
          cb = c_incl;
        }
        // some bin always qualifies (as above)
        const unsigned long long hit = __builtin_amdgcn_ballot_w64(found >= 0);
        const int first = (hit != 0ull) ? (int)__builtin_ctzll(hit) : 63;
        const unsigned dig = (unsigned)(255 - 4 * lane - (found >= 0 ? found : 3));
        prefix |= (unsigned)__builtin_amdgcn_readlane((int)dig, first) << shift;
        cnt_above += (unsigned)__builtin_amdgcn_readlane((int)c_above_d, first);
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

  // ---- stage-I ranks: one ordered scan per chunk of (keys above vstar,
  // ties at vstar), carried across the chunks
  const int n_rem = N - k1;
  const int m_fill = B - k1;
  const unsigned two_m = 2u * (unsigned)max(m_fill, 1);
  const unsigned step_q = (unsigned)(2 * n_rem) / two_m, step_r = (unsigned)(2 * n_rem) % two_m;
  int32_t* const kept_row = (SPLIT == kSegmentPass) ? nullptr : a.kept + (int64_t)row * a.kept_stride;
  // register rows park each kept token's position (and, in the segment pass,
  // its key) in LDS for the coalesced stores at the end
  int* const kpos = (int*)area;
  unsigned* const kkey = (unsigned*)area + B;
  uint8_t* const tag_row = a.tag ? a.tag + (int64_t)row * N : nullptr;
  unsigned carry_above = 0, carry_ties = 0;
  for (int ch = 0; ch < n_chunks; ++ch) {
    if constexpr (CHUNKED) {
      if (ch > 0) __syncthreads();  // the previous chunk's scan totals have been read
      load_run(ch);
    }
    unsigned my_above = 0, my_ties = 0;
    if (k1 > 0) {
#pragma unroll
      for (int e = 0; e < KREG; ++e)
        if (e < n_mine) {
          my_above += keys[e] > vstar ? 1u : 0u;
          my_ties += keys[e] == vstar ? 1u : 0u;
        }
    }
    uint64_t chunk_total;
    const uint64_t before = block_excl_scan64(((uint64_t)my_ties << 32) | my_above, sm_scan, &chunk_total);
    const unsigned above_before = carry_above + (unsigned)before;
    unsigned ties_before = carry_ties + (unsigned)(before >> 32);
    carry_above += (unsigned)chunk_total;
    carry_ties += (unsigned)(chunk_total >> 32);

    // ---- flags and output positions, token by token in raster order.
    // Stage-I tokens before n: above_before + min(c_ties, ties_before).  A
    // remainder token's rank is rho = n - that; stage II keeps the ranks
    // floor((2j+1) n_rem / (2m)), j < m, and the picks at ranks below rho
    // number min(m, ceil((2 m rho - n_rem) / (2 n_rem))).  The thread finds
    // its first pending pick with one division and steps to the next ones by
    // adding n_rem / m with a carried remainder.
    unsigned s1_before = above_before + min(ties_before, (unsigned)c_ties);
    int rho = n_begin - (int)s1_before;
    int pb = 0;              // stage-II picks at ranks below rho
    unsigned next_q = ~0u;   // rank of pick pb (none when pb == m)
    unsigned next_r = 0;     // (2 pb + 1) n_rem mod 2m
    if (m_fill > 0) {
      const int64_t num = 2 * (int64_t)m_fill * rho - n_rem;
      int64_t j = (num <= 0) ? 0 : (num + 2 * (int64_t)n_rem - 1) / (2 * (int64_t)n_rem);
      pb = (int)(j < m_fill ? j : m_fill);
      if (pb < m_fill) {
        const uint64_t t = (uint64_t)(2 * pb + 1) * (uint64_t)n_rem;
        next_q = (unsigned)(t / two_m);
        next_r = (unsigned)(t % two_m);
      }
    }
    auto put = [&](unsigned pos, int n, unsigned key) {
      if constexpr (CHUNKED) {
        kept_row[pos] = n;
      } else {
        kpos[pos] = n;
        if constexpr (SPLIT == kSegmentPass) kkey[pos] = key;
      }
    };
    auto emit = [&](int e, unsigned key) {
      const int n = n_begin + e;
      const bool is_above = (k1 > 0) && key > vstar;
      const bool is_tie = (k1 > 0) && key == vstar;
      const bool s1 = is_above || (is_tie && ties_before < (unsigned)c_ties);
      uint8_t tg = 0;
      if (s1) {
        tg = 1;
        put(s1_before + pb, n, key);
      } else {
        if ((unsigned)rho == next_q) {
          tg = 2;
          put(s1_before + pb, n, key);
          ++pb;
          if (pb < m_fill) {
            next_q += step_q;
            next_r += step_r;
            if (next_r >= two_m) {
              next_r -= two_m;
              ++next_q;
            }
          } else {
            next_q = ~0u;
          }
        }
      }
      // counters advance arithmetically (a branch on which one to bump makes the
      // compiler address them through memory)
      s1_before += s1 ? 1u : 0u;
      rho += s1 ? 0 : 1;
      if (tag_row) tag_row[n] = tg;
      ties_before += is_tie ? 1u : 0u;
    };
#pragma unroll
    for (int e = 0; e < KREG; ++e)
      if (e < n_mine) emit(e, keys[e]);
  }
  if constexpr (!CHUNKED) {
    __syncthreads();
    for (int j = tid; j < B; j += kThreads) {
      if constexpr (SPLIT == kSegmentPass) {
        a.cand_tok[cand0 + j] = tok0 + kpos[j];
        a.cand_score[cand0 + j] = bits_f(kkey[j]);
      } else if constexpr (SPLIT == kCandidatePass) {
        kept_row[j] = a.cand_tok[(int64_t)row * a.C + kpos[j]];
      } else {
        kept_row[j] = kpos[j];
      }
    }
  }
  if (tid == 0 && a.n_stage1) a.n_stage1[row] = k1;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

namespace {

// Split top-K for long rows (pure top-K, no tags): every row is cut into
// `segs` segments of seg_len tokens, each segment's top-K is found by its own
// workgroup, and a second pass takes the top-K of the segments' candidates.
// Exact: a token among the row's top K (score descending, index ascending)
// has fewer than K tokens ahead of it in its segment, so it is among its
// segment's top K; the candidate row keeps ascending token order, so the
// second pass breaks ties exactly as a one-pass selection would.
constexpr int kSegTargetKeys = 24576;  // preferred tokens per segment workgroup (24 per thread)

inline size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

struct SegPlan {
  int segs = 1, seg_len = 0, C = 0;  // C: candidates per row
};

SegPlan seg_plan(int R, int64_t N, int budget, double top_p) {
  SegPlan sp;
  constexpr int64_t cap = (int64_t)kThreads * kRegKeys;         // tokens of a register-resident row
  constexpr int64_t seg_cap = (int64_t)kThreads * kSegRegKeys;  // tokens of one segment
  if (!(top_p >= 1.0) || budget < 1 || N <= cap || R < 1) return sp;
  // segments of about kSegTargetKeys tokens, but no more than the fewest
  // possible take in the same number of rounds of one workgroup per CU
  const int64_t fewest = (N + seg_cap - 1) / seg_cap, cus = num_cus();
  auto rounds = [&](int64_t n) { return ((int64_t)R * n + cus - 1) / cus; };
  int64_t segs = std::max(fewest, (N + kSegTargetKeys - 1) / kSegTargetKeys);
  while (segs > fewest && rounds(segs) > rounds(fewest)) --segs;
  int64_t seg = (N + segs - 1) / segs;
  segs = (N + seg - 1) / seg;  // no empty last segment
  if (segs < 2 || seg < budget || segs * budget > cap) return sp;
  sp.segs = (int)segs;
  sp.seg_len = (int)seg;
  sp.C = (int)((segs - 1) * budget + std::min<int64_t>(budget, N - (segs - 1) * seg));
  return sp;
}

size_t seg_ws_bytes(int R, const SegPlan& sp, int budget) {
  if (sp.segs <= 1) return 0;
  return 2 * align256((size_t)R * sp.C * 4);  // candidate scores and tokens
}

}  // namespace

extern "C" size_t svlm_select_workspace(int R, int n_vis, int budget, double top_p) {
  if (R <= 0 || n_vis <= 0 || n_vis > (1 << 18) || budget <= 0 || budget > n_vis) return 0;
  const SegPlan sp = seg_plan(R, n_vis, budget, top_p);
  if (!grid_fits((int64_t)R * sp.segs, kThreads)) return 0;
  return seg_ws_bytes(R, sp, budget);
}

extern "C" int svlm_select(const float* scores, int64_t row_stride, int R, int F, int H, int W, double top_p,
                           int budget, int32_t* kept, int32_t* n_stage1, uint8_t* tag, void* ws, size_t ws_bytes,
                           void* stream) {
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
  a.top_p = top_p;
  a.kept = kept;
  a.kept_stride = budget;
  a.n_stage1 = n_stage1;
  a.tag = tag;
  a.segs = 1;
  a.seg_len = 0;
  a.C = 0;
  a.cand_score = nullptr;
  a.cand_tok = nullptr;
  hipStream_t st = (hipStream_t)stream;
  const SegPlan sp = seg_plan(R, N, budget, top_p);
  if (!grid_fits((int64_t)R * sp.segs, kThreads))
    return fail(SVLM_E_UNSUPPORTED, "svlm_select: %d rows exceed the launch limit", R);
  if (sp.segs > 1 && !tag) {
    const size_t need = seg_ws_bytes(R, sp, budget);
    if (!ws || ws_bytes < need)
      return fail(SVLM_E_WORKSPACE, "svlm_select: workspace of %zu bytes needed (got %zu)", need, ws_bytes);
    if (!aligned16(ws)) return fail(SVLM_E_INVALID, "svlm_select: workspace must be 16-byte aligned");
    a.cand_score = (float*)ws;
    a.cand_tok = (int32_t*)((char*)ws + align256((size_t)R * sp.C * 4));
    a.segs = sp.segs;
    a.seg_len = sp.seg_len;
    a.C = sp.C;
    SelArgs s1 = a;
    s1.n_stage1 = nullptr;
    select_rows<false, false, kSegmentPass><<<(unsigned)((int64_t)R * sp.segs), kThreads, 0, st>>>(s1);
    SelArgs s2 = a;
    s2.scores = a.cand_score;
    s2.row_stride = sp.C;
    s2.N = sp.C;
    if (sp.C <= kThreads * 8) select_rows<false, false, kCandidatePass, 8><<<R, kThreads, 0, st>>>(s2);
    else select_rows<false, false, kCandidatePass><<<R, kThreads, 0, st>>>(s2);
    return check_launch("svlm_select");
  }
  const bool mass = top_p > 0.0 && top_p < 1.0;
  const bool chunked = N > (int64_t)kThreads * kRegKeys;
  if (chunked) {
    if (mass) select_rows<true, true><<<R, kThreads, 0, st>>>(a);
    else select_rows<true, false><<<R, kThreads, 0, st>>>(a);
  } else {
    if (mass) select_rows<false, true><<<R, kThreads, 0, st>>>(a);
    else select_rows<false, false><<<R, kThreads, 0, st>>>(a);
  }
  return check_launch("svlm_select");
}

#ifdef SVLM_DEBUG
bool svlm::debug_take_select(unsigned* out) { return debug_take_here(out); }
#endif
