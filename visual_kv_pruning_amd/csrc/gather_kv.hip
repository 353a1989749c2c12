// svlm_gather_kv: compact the kept KV rows (kept visual tokens, then the
// always-kept text tail) into the draft cache.  Sparse-to-Dense explainer,
// technical summary, "dual-module architecture": the sparse draft reads only
// the selected KV, which cuts the draft stage's I/O.
//
// Pure copy: every destination row is one coalesced run of 16-byte loads and
// stores (D = 128 bf16 -> 16 lanes per row, 16 rows per 256-thread block).
#include "svlm_internal.h"

namespace svlm {
namespace {

struct GatherArgs {
  const uint16_t* src[2];
  uint16_t* dst[2];
  int64_t s_sh, s_sn, d_sh, d_sn;
  int n_src;
  const int32_t* idx;
  int64_t idx_sh;
  int n_idx, tail_start, n_tail;
};

template <int D>
__global__ __launch_bounds__(256) void gather_rows(GatherArgs a) {
  constexpr int CH = D / 8;            // 16-byte chunks per row
  constexpr int RPB = 256 / CH;        // rows per block
  const int t = threadIdx.x;
  const int j = blockIdx.x * RPB + t / CH;
  const int ch = t % CH;
  const int g = blockIdx.y;
  const int which = blockIdx.z;        // 0: K, 1: V
  if (j >= a.n_idx + a.n_tail) return;
  int srow;
  if (j < a.n_idx) srow = a.idx[(int64_t)g * a.idx_sh + j];
  else srow = a.tail_start + (j - a.n_idx);
  u32x4 val = {0u, 0u, 0u, 0u};
  if (srow >= 0 && srow < a.n_src)
    val = *(const u32x4*)(a.src[which] + (int64_t)g * a.s_sh + (int64_t)srow * a.s_sn + ch * 8);
  *(u32x4*)(a.dst[which] + (int64_t)g * a.d_sh + (int64_t)j * a.d_sn + ch * 8) = val;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" int svlm_gather_kv(const void* k_src, const void* v_src, int64_t s_sh, int64_t s_sn, int n_src,
                              const int32_t* idx, int64_t idx_sh, int n_idx, int tail_start, int n_tail,
                              void* k_dst, void* v_dst, int64_t d_sh, int64_t d_sn, int Hkv, int D, int dtype,
                              void* stream) {
  if (dtype != SVLM_BF16) return fail(SVLM_E_UNSUPPORTED, "svlm_gather_kv: only SVLM_BF16 is supported");
  if (D != 64 && D != 128) return fail(SVLM_E_UNSUPPORTED, "svlm_gather_kv: D must be 64 or 128 (got %d)", D);
  if (n_idx < 0 || n_tail < 0 || Hkv < 1 || n_src < 0) return fail(SVLM_E_INVALID, "svlm_gather_kv: negative size");
  if (n_idx + n_tail == 0) return SVLM_OK;  // nothing to copy
  if (!k_src || !v_src || !k_dst || !v_dst) return fail(SVLM_E_INVALID, "svlm_gather_kv: null K/V pointer");
  if (n_idx > 0 && !idx) return fail(SVLM_E_INVALID, "svlm_gather_kv: null index list");
  if (idx_sh < 0) return fail(SVLM_E_INVALID, "svlm_gather_kv: idx_sh must be >= 0");
  if (tail_start < 0 || (int64_t)tail_start + n_tail > n_src)
    return fail(SVLM_E_INVALID, "svlm_gather_kv: tail [%d, %d) outside the %d source rows", tail_start,
                tail_start + n_tail, n_src);
  if (!aligned16(k_src) || !aligned16(v_src) || !aligned16(k_dst) || !aligned16(v_dst))
    return fail(SVLM_E_INVALID, "svlm_gather_kv: K/V pointers must be 16-byte aligned");
  if (s_sn < D || d_sn < D || s_sn % 8 || d_sn % 8 || s_sh % 8 || d_sh % 8 || s_sh < 0 || d_sh < 0)
    return fail(SVLM_E_INVALID, "svlm_gather_kv: strides must be multiples of 8 elements, row strides >= D");
  const int n = n_idx + n_tail;
  GatherArgs a;
  a.src[0] = (const uint16_t*)k_src;
  a.src[1] = (const uint16_t*)v_src;
  a.dst[0] = (uint16_t*)k_dst;
  a.dst[1] = (uint16_t*)v_dst;
  a.s_sh = s_sh;
  a.s_sn = s_sn;
  a.d_sh = d_sh;
  a.d_sn = d_sn;
  a.n_src = n_src;
  a.idx = idx;
  a.idx_sh = idx_sh;
  a.n_idx = n_idx;
  a.tail_start = tail_start;
  a.n_tail = n_tail;
  const int rpb = 256 / (D / 8);
  dim3 grid((unsigned)((n + rpb - 1) / rpb), (unsigned)Hkv, 2);
  if (D == 128) gather_rows<128><<<grid, 256, 0, (hipStream_t)stream>>>(a);
  else gather_rows<64><<<grid, 256, 0, (hipStream_t)stream>>>(a);
  return check_launch("svlm_gather_kv");
}
