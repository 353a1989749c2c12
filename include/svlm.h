/*
 * svlm.h - C ABI of libsvlm: the data-parallel hot path of verifier-guided
 * visual-token / KV selection and draft/verify decode attention for lossless
 * speculative decoding of video LLMs, written for AMD Instinct MI355X (gfx950).
 *
 * Sources (cited by page title and section):
 *   [SpecVLM-5]  SpecVLM, Zhejiang University technology-transfer listing,
 *                section 5 "solution": text-to-visual mean attention from the
 *                target; two-stage pruning (Top-P by attention share, then a
 *                spatially uniform pick of the low-attention rest).
 *   [SpecVLM-A]  SpecVLM abstract (arXiv 2508.16201): verifier-guided stage I,
 *                spatially uniform stage II, up to 90% of video tokens pruned.
 *   [StD-dec]    Sparse-to-Dense explainer (arXiv 2505.19155), technical
 *                summary, "decoding process": gamma drafted tokens, verified by
 *                the dense model in one I/O pass over the full KV cache; longest
 *                matching prefix plus one bonus token.
 *   [StD-sel]    Same page, "KV cache selection": top-K visual KV picked at
 *                prefill from mean text-to-visual attention, per layer and head;
 *                "dual-module architecture": the sparse draft reads only the
 *                selected KV.
 *   [PVLM-PD]    ParallelVLM notes (CVPR 2026), background and "parallel
 *                decoding": candidates accepted by rejection sampling, which
 *                keeps the target's output distribution; a rejected token is
 *                resampled from the target.
 *   [PVLM-UV]    Same page, method section 1 "UV-Prune": video tokens scored
 *                by the change across early target layers of their cosine
 *                similarity to the text tokens, summed over the text; top-K.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless a parameter says otherwise.  Sizes
 *     and strides are in ELEMENTS of the pointed-to type.  The caller owns all
 *     buffers; the library never allocates or frees device memory and keeps no
 *     state between calls (apart from a per-device property cache).
 *   - Everything is enqueued on `stream` (a hipStream_t passed as void*; NULL
 *     is the default stream).  Calls return without synchronising.
 *   - Arguments are validated on the host before anything is enqueued.  On a
 *     bad argument nothing is enqueued, a status is returned and
 *     svlm_last_error() gives a text (thread-local).  SVLM_E_HIP reports a
 *     launch error from the HIP runtime (including an earlier asynchronous
 *     fault surfacing at this launch).
 *   - A call whose launch would pass the dispatch limits (2^31 work-items
 *     along x, 2^16 workgroups along y and z) returns SVLM_E_UNSUPPORTED
 *     instead of a truncated grid.  The *_workspace() queries take any int
 *     sizes without overflow and return 0 for sizes that their call refuses.
 *   - Device data that the host cannot see (indices, lengths, scores) are
 *     preconditions, stated per call; kernels clamp them so that no access
 *     leaves the buffers, but results are unspecified when they are violated.
 *   - Only D in {64, 128} is supported; the innermost (D) dimension must be
 *     contiguous and every row 16-byte aligned (strides in multiples of 16
 *     bytes).
 *   - Operand types: SVLM_BF16 runs the tuned matrix-core kernels.  SVLM_F32
 *     (svlm_score, svlm_gather_kv, svlm_decode_attn[_indexed]) takes fp32
 *     q, k and v as given, for the tiny fp32 reference configuration: plain
 *     vector-ALU fp32 kernels with natural-base exp, correct at any size but
 *     not tuned for bandwidth.  Outputs are fp32 either way.
 *   - Selection, gather and acceptance are bit-deterministic; score and
 *     attention are run-to-run deterministic (fixed reduction order).
 *   - Calls on different streams may run concurrently if their workspaces
 *     differ.
 */
#ifndef SVLM_H
#define SVLM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SVLM_ABI_VERSION 4

enum svlm_status {
  SVLM_OK = 0,
  SVLM_E_INVALID = 1,     /* an argument is out of range, null or misaligned */
  SVLM_E_UNSUPPORTED = 2, /* a valid request this build does not implement (dtype, D, sizes) */
  SVLM_E_WORKSPACE = 3,   /* workspace missing or smaller than the *_workspace() size */
  SVLM_E_HIP = 4          /* the HIP runtime reported an error */
};

enum svlm_dtype { SVLM_BF16 = 0, SVLM_F32 = 1 };
enum svlm_agg { SVLM_AGG_QHEAD = 0, SVLM_AGG_KVHEAD = 1, SVLM_AGG_ALL = 2 };
enum svlm_verify_mode { SVLM_VERIFY_GREEDY = 0, SVLM_VERIFY_REJECT = 1 };

/* ABI version of the loaded library (SVLM_ABI_VERSION at build time). */
int svlm_abi_version(void);
/* Static text for a status code. */
const char* svlm_status_string(int status);
/* Thread-local text describing the last failure of a call on this thread. */
const char* svlm_last_error(void);

/* ------------------------------------------------------------------------
 * svlm_score - mean text-to-visual softmax attention of one layer.
 * [SpecVLM-5]; [StD-sel].
 *
 * For q head h (KV head g = h / (Hq/Hkv)), text query t at position
 * q_pos0 + t sees keys 0..q_pos0+t (causal) of k:
 *     P[t,h,n] = softmax_n(scale * <q_text[t,h], k[g,n]>)
 *     A[h,i]   = (1/T) * sum_t P[t,h,vis_start+i],   i < n_vis
 * The softmax runs over the whole visible range; visual columns are read
 * out of the normalised rows.  Aggregation `agg`: SVLM_AGG_QHEAD -> rows
 * [Hq][n_vis]; SVLM_AGG_KVHEAD -> mean over each group, [Hkv][n_vis];
 * SVLM_AGG_ALL -> mean over all q heads, [1][n_vis].  Then
 *     out = alpha * agg(A) + beta * out        (beta == 0: out is not read)
 * which lets several layers be averaged into one row set.
 *
 * q_text: [T][Hq][D] (dtype: SVLM_BF16 or SVLM_F32) with strides q_st (per
 *         text token) and q_sh (per head); D contiguous.
 * k:      [Hkv][n_ctx][D], same dtype, with strides k_sh, k_sn.
 * out:    fp32 rows, contiguous [rows][n_vis].
 * ws:     svlm_score_workspace(T, Hq, Hkv, q_pos0, n_vis) bytes (per-split row
 *         statistics and per-head score rows; with SVLM_F32 only the row
 *         log-sum-exps, which fit in the same size).
 * Requires 1 <= T <= 128, scale > 0, q_pos0 + T <= n_ctx, 0 <= vis_start, vis_start + n_vis
 * <= q_pos0 + 1 (every visual key visible to every text query), n_vis <= 2^18,
 * and ((T-1)*q_st + D)*2 and (n_ctx + 1024)*k_sn*2 below 2^31 (32-bit buffer
 * ranges; SVLM_E_UNSUPPORTED otherwise; the 32-bit limits apply to SVLM_BF16).
 * Computes QK^T on bf16 matrix cores with fp32 accumulation, in two passes
 * (row log-sum-exp, then normalised column sums); the score matrix is never
 * stored.  SVLM_F32 runs the same two passes in fp32 vector arithmetic.
 * ------------------------------------------------------------------------ */
size_t svlm_score_workspace(int T, int Hq, int Hkv, int q_pos0, int n_vis);
int svlm_score(const void* q_text, int64_t q_st, int64_t q_sh,
               const void* k, int64_t k_sh, int64_t k_sn,
               int dtype, int T, int n_ctx, int q_pos0, int vis_start, int n_vis,
               int Hq, int Hkv, int D, float scale, int agg,
               float alpha, float beta, float* out,
               void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_score_layers - svlm_score over `layers` layers in one call.
 * [SpecVLM-5]; [StD-sel] (the selection signal averaged over layers and
 * heads, or kept per layer).
 *
 * Layer l reads q_text + l*q_sl and k + l*k_sl (element strides, multiples
 * of 16 bytes, >= 0); every other argument is as for svlm_score, the same
 * for every layer.  Let R_l = agg(A_l), the rows svlm_score would form for
 * layer l (Hq, Hkv or 1 rows of n_vis).
 *   layer_mean = 1: out = alpha * (1/layers) * sum_l R_l + beta * out,
 *                   rows as for one layer (agg SVLM_AGG_KVHEAD or
 *                   SVLM_AGG_ALL; SVLM_AGG_QHEAD is SVLM_E_UNSUPPORTED).
 *   layer_mean = 0: out[l] = alpha * R_l + beta * out[l], out is
 *                   [layers][rows][n_vis].
 * With layers == 1 it is svlm_score (bit for bit, either layer_mean).
 * The layers share the launches: the key splits are planned over all of
 * them (at least four rounds of workgroups over the chip, whole rounds
 * preferred), so each workgroup covers more keys than in a one-layer call
 * and the results differ from per-layer svlm_score calls by fp32
 * reordering only.
 * ws: svlm_score_layers_workspace(layers, T, Hq, Hkv, q_pos0, n_vis) bytes
 *     (the per-layer statistics and group rows of every layer).
 * Errors as svlm_score; layers < 1 or layer_mean outside {0, 1} is
 * SVLM_E_INVALID; sizes whose launches or workspace exceed the limits are
 * SVLM_E_UNSUPPORTED.
 * ------------------------------------------------------------------------ */
size_t svlm_score_layers_workspace(int layers, int T, int Hq, int Hkv, int q_pos0, int n_vis);
int svlm_score_layers(const void* q_text, int64_t q_st, int64_t q_sh, int64_t q_sl,
                      const void* k, int64_t k_sh, int64_t k_sn, int64_t k_sl, int layers,
                      int dtype, int T, int n_ctx, int q_pos0, int vis_start, int n_vis,
                      int Hq, int Hkv, int D, float scale, int agg, int layer_mean,
                      float alpha, float beta, float* out,
                      void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_select - two-stage visual token selection, one row at a time.
 * [SpecVLM-5] (stages i and ii); [SpecVLM-A]; [StD-sel] for top_p >= 1.
 *
 * Each row holds n_vis = F*H*W fp32 scores s in [0, 1] (precondition),
 * token n = f*H*W + y*W + x (frame-major raster order).
 * Order: score descending, then index ascending.  Mass of a token:
 * floor(s * 2^40) as an exact integer; row total Q; target
 * ceil(double(Q) * top_p) in IEEE round-to-nearest double arithmetic.
 * Stage I keeps the shortest top prefix whose mass reaches the target,
 * truncated to `budget` tokens (top_p >= 1: the top `budget`; top_p <= 0:
 * none).  k1 = its size.  Stage II walks the other n_rem = n_vis - k1 tokens
 * in raster order and keeps the ones at ranks floor((2j+1)*n_rem/(2m)),
 * j < m = budget - k1 (one constant stride with centred phase, so each frame
 * gets its share spread evenly over its H x W grid).
 *
 * scores:   [R] rows with stride row_stride.
 * kept:     [R][budget] int32, ascending token indices (output).
 * n_stage1: [R] int32 k1 (output).  tag: [R][n_vis] uint8 or NULL
 *           (0 dropped, 1 stage I, 2 stage II).
 * ws:       svlm_select_workspace(R, n_vis, budget, top_p) bytes, 16-byte
 *           aligned (caller-owned, device memory).  It is 0 except for pure
 *           top-K (top_p >= 1) on rows longer than 32768 tokens, which are
 *           split into segments whose top-K candidates a second pass
 *           reduces; the result is identical.  With tag != NULL that form is
 *           not used and ws is ignored.  A workspace that is needed but
 *           missing or short is SVLM_E_WORKSPACE.
 * Requires 0 <= budget <= n_vis <= 2^18.
 * ------------------------------------------------------------------------ */
size_t svlm_select_workspace(int R, int n_vis, int budget, double top_p);
int svlm_select(const float* scores, int64_t row_stride, int R, int F, int H, int W,
                double top_p, int budget, int32_t* kept, int32_t* n_stage1, uint8_t* tag,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_gather_kv - compact the kept KV rows into a draft cache.
 * [StD-sel] ("dual-module architecture": the draft reads only selected KV).
 *
 * For every KV head g:
 *   dst[g, j]         = src[g, idx[g*idx_sh + j]],   j < n_idx
 *   dst[g, n_idx + j] = src[g, tail_start + j],      j < n_tail
 * (the tail carries the always-kept text rows).  Applied to K and V alike.
 * src: [Hkv][n_src][D] with strides s_sh, s_sn; dst: strides d_sh, d_sn.
 * dtype SVLM_BF16 or SVLM_F32 (2- or 4-byte elements; a bit-exact copy).
 * idx_sh = 0: one list for all heads; otherwise per-head lists.
 * Indices outside [0, n_src) are a precondition violation; such rows are
 * written as zeros.  Requires tail_start + n_tail <= n_src.  With
 * n_idx + n_tail == 0 nothing is done (pointers may be NULL).
 * ------------------------------------------------------------------------ */
int svlm_gather_kv(const void* k_src, const void* v_src, int64_t s_sh, int64_t s_sn, int n_src,
                   const int32_t* idx, int64_t idx_sh, int n_idx, int tail_start, int n_tail,
                   void* k_dst, void* v_dst, int64_t d_sh, int64_t d_sn,
                   int Hkv, int D, int dtype, void* stream);

/* ------------------------------------------------------------------------
 * svlm_decode_attn - split-K grouped-query decode attention, draft or verify.
 * [StD-dec] (sparse draft over the kept KV, one query; dense verify of the
 * gamma+1 newest tokens in one pass over the full KV); SpecVLM
 * technology-transfer listing, section 4 (decode is bound by loading the KV
 * cache every step).
 *
 * For batch b, query i < nq and q head h (g = h / (Hq/Hkv)), keys
 * n < L(b,i) with L = kv_len[b] - nq + i + 1 if causal_tail else kv_len[b]:
 *   out[b,i,h] = sum_n softmax_n(scale*<q[b,i,h], k[b,g,n]>) * v[b,g,n]
 *   lse[b,i,h] = log sum_n exp(scale*<q[b,i,h], k[b,g,n]>)   (natural log)
 * q:   [B][nq][Hq][D] (dtype), batch stride q_sb, the rest contiguous.
 * k,v: [B][Hkv][max_kv_len][D] (dtype) with strides kv_sb, kv_sh, kv_sn;
 *      kv_sb = 0 shares one cache among the batch entries.
 * kv_len: [B] int32 on the device; precondition nq <= kv_len[b] <=
 *         max_kv_len (values are clamped into [0, max_kv_len]).
 * out: [B][nq][Hq][D] fp32 contiguous; lse: [B][nq][Hq] fp32 or NULL.
 * num_splits: key-range splits per (batch, KV head); 0 picks one for the
 *   chip, or takes SVLM_NUM_SPLITS from the environment when that holds a
 *   positive integer (read once per process; the *_workspace() queries use
 *   the same rule).  With more than one split the partial (max, sum, output)
 *   states go to ws and are merged in a fixed order.
 * ws: svlm_decode_attn_workspace(batch, nq, Hq, Hkv, D, max_kv_len, num_splits)
 *   bytes (0 when one split suffices); no initial contents are needed.  Two
 *   calls that overlap in time must not share a workspace.  SVLM_F32 uses no
 *   workspace (ws may be NULL).
 * Requires scale > 0, nq*Hq*D*2 < 2^31, and one key split's rows times
 * kv_sn*2 below 2^31 bytes (always true when (max_kv_len + 576)*kv_sn*2 <
 * 2^31; SVLM_E_UNSUPPORTED otherwise).
 * SVLM_BF16 works in bf16 matrix-core products with fp32 accumulation; the
 * softmax weights enter the value product as a bf16 hi + lo pair, so the
 * output keeps fp32-level accuracy.  SVLM_F32: fp32 vector arithmetic, one
 * wave per output row.
 * ------------------------------------------------------------------------ */
size_t svlm_decode_attn_workspace(int batch, int nq, int Hq, int Hkv, int D, int max_kv_len,
                                  int num_splits);
int svlm_decode_attn(const void* q, int64_t q_sb,
                     const void* k, const void* v, int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                     const int32_t* kv_len, int max_kv_len,
                     int dtype, int batch, int nq, int Hq, int Hkv, int D, float scale,
                     int causal_tail, float* out, float* lse,
                     int num_splits, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_decode_attn_noalloc - svlm_decode_attn for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and results, with the
 * split-K partial state kept in a static device array of
 * SVLM_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends.  The call allocates nothing.
 *
 * Arguments are svlm_decode_attn's without the workspace.  A call whose
 * svlm_decode_attn_workspace(...) size exceeds SVLM_NOALLOC_SCRATCH_BYTES
 * returns SVLM_E_UNSUPPORTED before enqueueing anything (16 MiB covers dense
 * verify of 10 queries over 141194 keys at 28 q / 4 KV heads, which needs
 * about 8 MB).  The scratch needs no initial contents.  All calls on one
 * device share its scratch: calls that may overlap in time on one device
 * (different streams, or graph replays running concurrently) race and must
 * not be issued.  The array's device address is looked up once per device
 * (hipGetSymbolAddress) on the first call with that device current; a failure
 * there is SVLM_E_HIP.
 * ------------------------------------------------------------------------ */
#define SVLM_NOALLOC_SCRATCH_BYTES (16u << 20)
int svlm_decode_attn_noalloc(const void* q, int64_t q_sb,
                             const void* k, const void* v, int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                             const int32_t* kv_len, int max_kv_len,
                             int dtype, int batch, int nq, int Hq, int Hkv, int D, float scale,
                             int causal_tail, float* out, float* lse, int num_splits, void* stream);

/* ------------------------------------------------------------------------
 * svlm_decode_attn_indexed - svlm_decode_attn over keys named by an index
 * list, read in place from the full cache (the gather fused into the draft).
 * [StD-sel] ("dual-module architecture": the sparse draft reads only the
 * selected KV, per layer and head); [StD-dec].
 *
 * Key position n < n_idx[b] of batch b and KV head g is cache row
 *   r = kv_idx[b * idx_sb + g * idx_sh + n]
 * of k, v: [B][Hkv][kv_rows][D] bf16 with strides kv_sb, kv_sh, kv_sn.
 * idx_sh = 0: one list for all heads; idx_sb = 0: one list for all batch
 * entries.  List (b, g) has n_idx[b * n_sb + g * n_sh] entries (device
 * int32): n_sh = 0 gives one length per batch entry, n_sh = 1 and
 * n_sb = Hkv ragged per-head lengths (the per-layer, per-head selection of
 * [StD-sel]).  The attention is svlm_decode_attn's with k[b,g,n] replaced
 * by row r and kv_len by the list's length (precondition
 * nq <= length <= max_n_idx; causal_tail applies to the last nq positions of
 * each list).  Indices are a precondition in [0, kv_rows); one outside
 * reads a zero row (the result is then undefined) and never reads memory
 * outside the cache.  Requires kv_rows * kv_sn * 2 < 2^31 (SVLM_BF16).
 * ws: svlm_decode_attn_indexed_workspace(...) bytes, same rules as above.
 * ------------------------------------------------------------------------ */
size_t svlm_decode_attn_indexed_workspace(int batch, int nq, int Hq, int Hkv, int D, int max_n_idx,
                                          int num_splits);
int svlm_decode_attn_indexed(const void* q, int64_t q_sb,
                             const void* k, const void* v, int64_t kv_sb, int64_t kv_sh, int64_t kv_sn,
                             int kv_rows, const int32_t* kv_idx, int64_t idx_sb, int64_t idx_sh,
                             const int32_t* n_idx, int64_t n_sb, int64_t n_sh, int max_n_idx,
                             int dtype, int batch, int nq, int Hq, int Hkv, int D, float scale,
                             int causal_tail, float* out, float* lse,
                             int num_splits, void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_uvprune_score - UV-Prune score of every video token (an alternative
 * to svlm_score's attention signal that needs no attention matrix).
 * [PVLM-UV] ParallelVLM notes, method section 1 ("UV-Prune").
 *
 * With S^l_ij the cosine similarity of video token i and text token j at
 * target layer l (a zero vector's similarities are 0):
 *   dS_i = sum_j sum_{l=1..L} (S^l_ij - S^(l-1)_ij) = sum_j (S^L_ij - S^0_ij)
 *   out[i] = out_scale * dS_i + out_offset
 * so only the hidden states of layers 0 and L are read.  dS lies in
 * [-2 n_text, 2 n_text]; out_scale = 1/(4 n_text), out_offset = 1/2 maps it
 * monotonically into [0, 1] for svlm_select with top_p >= 1 (top-K).
 * v0, vL: [n_vis][d] bf16 video hidden states of layers 0 and L, row stride
 *         v_sn; x0, xL: [n_text][d] bf16 text hidden states, row stride x_sn.
 * out: [n_vis] fp32.  ws: svlm_uvprune_workspace(n_text, d) bytes.
 * Requires d % 8 == 0, d <= 16384, strides multiples of 8 and >= d,
 * 16-byte aligned pointers.  fp32 accumulation; deterministic.
 * ------------------------------------------------------------------------ */
size_t svlm_uvprune_workspace(int n_text, int d);
int svlm_uvprune_score(const void* v0, const void* vL, int64_t v_sn, int n_vis,
                       const void* x0, const void* xL, int64_t x_sn, int n_text, int d,
                       int dtype, float out_scale, float out_offset, float* out,
                       void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_verify - acceptance of gamma drafted tokens.
 * SVLM_VERIFY_GREEDY [StD-dec]: a_i = argmax target[b,i,:] (lowest index on
 *   ties); n = length of the longest prefix with draft_tok[b,j] == a_j;
 *   next_tok = a_n (a correction when n < gamma, the bonus token when
 *   n == gamma).  target holds logits [B][gamma+1][V].
 * SVLM_VERIFY_REJECT [PVLM-PD], standard speculative sampling: target holds
 *   probabilities p [B][gamma+1][V], draft_prob q [B][gamma][V], u
 *   [B][gamma+1] uniforms in [0,1).  Token i is accepted iff
 *   u_i * q_i(d_i) <= p_i(d_i) (exact fp64 product); at the first rejection
 *   n = i and next_tok is drawn from max(0, p_i - q_i) (formed in fp32);
 *   if all are accepted n = gamma and next_tok is drawn from p_gamma.  The
 *   draw is a fixed-point inverse CDF with u_gamma: m_v = floor(w_v*2^40),
 *   W = sum m_v, t = min(floor(double(u)*double(W)), W-1), token = least v
 *   with m_0+..+m_v > t.  If W == 0 the draw uses p_i instead, then
 *   argmax p_i.
 * n_accept, next_tok: [B] int32 outputs.  Requires 1 <= gamma, 1 <= V,
 * draft tokens in [0, V) (clamped otherwise), probabilities in [0, 1].
 * ws: svlm_verify_workspace(batch, gamma, V) bytes, zero-filled before its
 *   first use.  Its first 256 KB are arrival counters, one per sequence
 *   index: the call is one launch whose last workgroup per sequence to finish
 *   its vocabulary chunk reduces the chunk results (stored after the
 *   counters), and it leaves the counters zero again, so one workspace, big
 *   enough for the largest call, serves later calls of any shape without
 *   clearing.  Calls that share a workspace must not overlap in time.
 * ------------------------------------------------------------------------ */
size_t svlm_verify_workspace(int batch, int gamma, int V);
int svlm_verify(int mode, int batch, int gamma, int V, const int32_t* draft_tok,
                const float* target, const float* draft_prob, const float* u,
                int32_t* n_accept, int32_t* next_tok,
                void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * svlm_stream_read - measurement helper (not a step of the path): reads
 * `bytes` of src once, in the decode-attention kernel's access pattern (1 KB
 * LDS-DMA transfers per wave, nontemporal, 16 KB in flight per wave, four
 * waves per workgroup), split over `workgroups` contiguous ranges of whole
 * KB, and writes one float per workgroup to sink (device, `workgroups`
 * floats): the float at byte 4096 * (ceil(ceil(n / 1024) / 4) - 1) of its
 * n-byte range (the start of the first wave's last transfer).  Its time is
 * the achievable streaming rate of a launch of that size, the reference
 * beside the HBM peak for the attention calls.  bytes = 0 launches one empty
 * workgroup: the floor of a dependent launch.  src 16-byte aligned.
 * ------------------------------------------------------------------------ */
int svlm_stream_read(const void* src, int64_t bytes, int workgroups, float* sink, void* stream);

/* ------------------------------------------------------------------------
 * svlm_debug_flags - device preconditions violated since the last call.
 * For callers debugging their inputs: a library built with -DSVLM_DEBUG
 * (libsvlm_debug.so beside libsvlm.so) checks, inside the kernels, the
 * device-side preconditions stated per call above and, beside the clamping
 * every build does, sets one bit per kind of violation:
 *   SVLM_DBG_KV_LEN       an attention length (kv_len, or an index list's
 *                         length) outside [nq, max_kv_len]
 *   SVLM_DBG_KV_INDEX     an attention index-list entry outside [0, kv_rows)
 *   SVLM_DBG_GATHER_INDEX a gather index outside [0, n_src)
 *   SVLM_DBG_DRAFT_TOKEN  a draft token outside [0, V)
 *   SVLM_DBG_PROB_RANGE   a target or draft probability read by the
 *                         rejection test outside [0, 1] (or NaN)
 *   SVLM_DBG_SCORE_RANGE  a selection score outside [0, 1] (or NaN)
 * *flags receives the bits set since the previous call, which clears them.
 * Call it when the work to inspect has completed (the copy of the flags
 * synchronises with the default stream only).  Without SVLM_DEBUG it stores
 * 0 and returns SVLM_E_UNSUPPORTED; it launches nothing either way.
 * ------------------------------------------------------------------------ */
enum svlm_debug_flag {
  SVLM_DBG_KV_LEN = 1u,
  SVLM_DBG_KV_INDEX = 2u,
  SVLM_DBG_GATHER_INDEX = 4u,
  SVLM_DBG_DRAFT_TOKEN = 8u,
  SVLM_DBG_PROB_RANGE = 16u,
  SVLM_DBG_SCORE_RANGE = 32u
};
int svlm_debug_flags(unsigned* flags);

#ifdef __cplusplus
}
#endif

#endif /* SVLM_H */
