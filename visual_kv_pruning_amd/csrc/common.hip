// Host-side status reporting and device queries shared by the libsvlm entry points.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <vector>

#include "svlm_internal.h"

namespace svlm {

static thread_local char g_last_error[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(SVLM_E_HIP, "%s: HIP error %d (%s)", what, (int)e, hipGetErrorString(e));
  return SVLM_OK;
}

int num_cus() {
  static std::mutex mu;
  static std::vector<int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  if ((int)cache.size() <= dev) cache.resize(dev + 1, 0);
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

}  // namespace svlm

extern "C" int svlm_abi_version(void) { return SVLM_ABI_VERSION; }

extern "C" const char* svlm_status_string(int status) {
  switch (status) {
    case SVLM_OK: return "SVLM_OK";
    case SVLM_E_INVALID: return "SVLM_E_INVALID: invalid argument";
    case SVLM_E_UNSUPPORTED: return "SVLM_E_UNSUPPORTED: unsupported dtype or shape";
    case SVLM_E_WORKSPACE: return "SVLM_E_WORKSPACE: workspace missing or too small";
    case SVLM_E_HIP: return "SVLM_E_HIP: HIP runtime error";
    default: return "unknown svlm status";
  }
}

extern "C" const char* svlm_last_error(void) { return svlm::g_last_error; }

extern "C" int svlm_debug_flags(unsigned* flags) {
  if (!flags) return svlm::fail(SVLM_E_INVALID, "svlm_debug_flags: null pointer");
  *flags = 0;
#ifdef SVLM_DEBUG
  using namespace svlm;
  bool (*const take[])(unsigned*) = {debug_take_decode_attn, debug_take_f32_path, debug_take_gather,
                                     debug_take_select, debug_take_verify};
  unsigned all = 0;
  for (auto t : take) {
    unsigned v = 0;
    if (!t(&v)) return fail(SVLM_E_HIP, "svlm_debug_flags: reading the device flags failed");
    all |= v;
  }
  *flags = all;
  return SVLM_OK;
#else
  return svlm::fail(SVLM_E_UNSUPPORTED, "svlm_debug_flags: this library was built without SVLM_DEBUG");
#endif
}
