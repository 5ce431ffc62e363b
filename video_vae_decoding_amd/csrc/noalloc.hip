// The allocation-free single causal conv: wanvae_causal_conv3d with its workspace in a
// fixed device array of the library instead of memory the call allocates or the caller
// brings. For callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it).
//
// The array is file-scope device memory; each GPU the library runs on holds its own copy
// until the process ends. Its address on a device comes from hipGetSymbolAddress, taken once
// per device on that device's first call and kept; only that address is ever handed to the
// kernels. Calls that overlap in time on one device share the array and race: a caller must
// order them (one stream, or events). Nothing in the array needs to start at zero: the conv
// writes the repacked weights, the bias, the layout-converted frames and every split-K
// partial before it reads them.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "internal.h"

namespace wanvae {
namespace {

constexpr size_t kScratchBytes = (size_t)128 << 20;  // 128 MiB

__device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// The device address of this device's copy of the array (looked up once per device).
int scratch_ptr(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return report(WANVAE_EHIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return report(WANVAE_EHIP, "device index beyond the scratch table");
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      char buf[256];
      snprintf(buf, sizeof buf, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
      return report(WANVAE_EHIP, buf);
    }
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return WANVAE_OK;
}

}  // namespace
}  // namespace wanvae

using namespace wanvae;

extern "C" {

int wanvae_causal_conv3d_noalloc(const void* x, const void* cache, int64_t B, int64_t Cin, int64_t t, int64_t h,
                                 int64_t w, int64_t n_cache, const wanvae_tensor* weight, const wanvae_tensor* bias,
                                 int32_t layout, int32_t dtype, void* y, int32_t y_dtype, void* cache_out,
                                 void* stream) {
  size_t need = 0;
  if (int rc = conv_plan(x, cache, B, Cin, t, h, w, n_cache, weight, bias, layout, dtype, y, y_dtype, cache_out,
                         &need))
    return rc;
  if (need > kScratchBytes) {
    char buf[256];
    snprintf(buf, sizeof buf, "the conv needs %zu bytes of scratch; the fixed scratch holds %zu", need, kScratchBytes);
    return report(WANVAE_EWORKSPACE, buf);
  }
  void* ws = nullptr;
  if (int rc = scratch_ptr(&ws)) return rc;
  return conv_enqueue(x, cache, B, Cin, t, h, w, n_cache, weight, bias, layout, dtype, y, y_dtype, cache_out, ws,
                      (hipStream_t)stream);
}

}  // extern "C"
