// svlm_stream_read: a measurement helper, not a step of the path.  It reads a
// buffer once from HBM the way the decode-attention kernel reads its keys and
// values (1 KB LDS-DMA transfers per wave, nontemporal, a private ring of 16 KB
// in flight per wave, four waves per workgroup, about one workgroup per
// compute unit) and does nothing else, so its time is what this chip gives a
// launch of that many bytes in that pattern: the achievable reference beside
// the 8 TB/s peak for the attention calls.  With zero bytes it is one empty
// workgroup, the per-launch floor of a dependent launch.
#include "svlm_internal.h"

namespace svlm {
namespace {

constexpr int kSrWaves = 4;
constexpr int kSrSlots = 16;  // 1 KB transfers in flight per wave

struct StreamArgs {
  const unsigned char* src;
  int64_t bytes;
  int64_t per_wg;  // bytes per workgroup, a multiple of 1 KB
  float* sink;
};

__global__ __launch_bounds__(64 * kSrWaves, 1) void stream_read(StreamArgs a) {
  __shared__ __align__(16) unsigned char ring[kSrWaves][kSrSlots][1024];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t begin = (int64_t)blockIdx.x * a.per_wg;
  const int64_t n = a.bytes - begin < a.per_wg ? a.bytes - begin : a.per_wg;
  const int nt0 = (int)((n + 1023) / 1024);
  const int last0 = (nt0 + kSrWaves - 1) / kSrWaves - 1;  // wave 0's last transfer
  if (n > 0) {
    // descriptor over exactly this workgroup's bytes: transfers past its end read zeros
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)(a.src + begin), (short)0, (int)n, kBufferFlags);
    const int nt = (int)((n + 1023) / 1024);      // 1 KB transfers of this workgroup
    const int mine = (nt - wave + kSrWaves - 1) / kSrWaves;   // transfers wave, wave + 4, ...
    auto issue = [&](int i) {
      const int slot = i % kSrSlots;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)&ring[wave][slot][0], 16, lane * 16,
          (i * kSrWaves + wave) * 1024, 0, kNT);
    };
    int i = 0;
    for (; i < mine && i < kSrSlots; ++i) issue(i);
    for (int j = kSrSlots; j < mine; ++j) {
      wait_vmcnt<kSrSlots - 1>();  // the oldest transfer has landed: its slot is free
      issue(j);
    }
    wait_vmcnt<0>();
  }
  // the first word of wave 0's last transfer (workgroup byte 4096 * last0), so
  // the reads have an observable use
  __syncthreads();
  if (threadIdx.x == 0) a.sink[blockIdx.x] = (n > 0) ? *(const float*)&ring[0][last0 % kSrSlots][0] : 0.f;
}

}  // namespace
}  // namespace svlm

using namespace svlm;

extern "C" int svlm_stream_read(const void* src, int64_t bytes, int workgroups, float* sink, void* stream) {
  if (bytes < 0 || workgroups < 1) return fail(SVLM_E_INVALID, "svlm_stream_read: bytes >= 0, workgroups >= 1");
  if (!sink || (bytes > 0 && !src)) return fail(SVLM_E_INVALID, "svlm_stream_read: null pointer");
  if (bytes > 0 && !aligned16(src)) return fail(SVLM_E_INVALID, "svlm_stream_read: src must be 16-byte aligned");
  StreamArgs a;
  a.src = (const unsigned char*)src;
  a.bytes = bytes;
  const int64_t per = (bytes + workgroups - 1) / workgroups;
  a.per_wg = (per + 1023) / 1024 * 1024;
  if (a.per_wg > INT32_MAX) return fail(SVLM_E_UNSUPPORTED, "svlm_stream_read: more than 2^31 bytes per workgroup");
  a.sink = sink;
  const int64_t blocks = bytes > 0 ? (bytes + a.per_wg - 1) / a.per_wg : 1;
  if (!grid_fits(blocks, 64 * kSrWaves))
    return fail(SVLM_E_UNSUPPORTED, "svlm_stream_read: %d workgroups exceed the launch limit", workgroups);
  const unsigned grid = (unsigned)blocks;
  stream_read<<<grid, 64 * kSrWaves, 0, (hipStream_t)stream>>>(a);
  return check_launch("svlm_stream_read");
}
