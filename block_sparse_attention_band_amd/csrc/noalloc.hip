// prism_estimate_noalloc: the estimator for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation). Its workspace is this file's device array
// `scratch` instead of a caller's buffer; everything else is prism_estimate.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// address on a device is looked up once per device (hipGetSymbolAddress with
// that device current) and only that address is handed to the kernels. Each
// device holds its own copy for the life of the process, and every call on a
// device shares it: calls that overlap on one device race. No kernel relies
// on the array's earlier contents (every workspace byte a call reads, the
// same call wrote first), so nothing is cleared between calls.
#include <mutex>

#include "prism_kernels.h"

namespace {

constexpr size_t kScratchBytes = PRISM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch`, per device, once looked up

hipError_t scratch_address(int dev, void **out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" int prism_estimate_noalloc(const prism_tensor_t *q, const prism_tensor_t *k, const prism_cfg_t *cfg,
                                      prism_mask_t *mask_out, void *stream) {
  prism_workspace_layout_t L;
  const int st = prism::check_estimate_call(q, k, cfg, mask_out, &L);
  if (st) return st;
  if (L.total_bytes > kScratchBytes) return PRISM_ERR_SCRATCH;
  hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  void *ws = nullptr;
  if (prism::stream_device(s, &dev) != hipSuccess || scratch_address(dev, &ws) != hipSuccess) return PRISM_ERR_LAUNCH;
  return prism::enqueue_estimate(q, k, cfg, mask_out, L, ws, s);
}
