// Device queries the launchers need, cached per device: the one piece of
// state the library keeps between calls (written once per device, then
// read-only).
#include <mutex>

#include "prism_kernels.h"

namespace prism {
namespace {
constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
int g_cus[kMaxDevices];
hipError_t g_err[kMaxDevices];

// resident workgroups per CU of a kernel, by kernel (a few dozen at most)
struct Occ {
  const void *f;
  int threads, per_cu;
};
std::mutex g_occ_mu;
Occ g_occ[128];
int g_nocc = 0;
}  // namespace

hipError_t stream_device(hipStream_t s, int *dev) {
  if (s == nullptr) return hipGetDevice(dev);
  return hipStreamGetDevice(s, dev);
}

hipError_t stream_capturing(hipStream_t s, bool *capturing) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  const hipError_t e = hipStreamIsCapturing(s, &st);
  *capturing = st != hipStreamCaptureStatusNone;
  return e;
}

hipError_t device_cu_count(int dev, int *cus) {
  if (dev < 0 || dev >= kMaxDevices) return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
  });
  *cus = g_cus[dev];
  return g_err[dev];
}

hipError_t kernel_occupancy(const void *f, int threads, int *per_cu) {
  std::lock_guard<std::mutex> lock(g_occ_mu);
  for (int i = 0; i < g_nocc; ++i)
    if (g_occ[i].f == f && g_occ[i].threads == threads) {
      *per_cu = g_occ[i].per_cu;
      return hipSuccess;
    }
  const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(per_cu, f, threads, 0);
  if (e == hipSuccess && g_nocc < 128) g_occ[g_nocc++] = Occ{f, threads, *per_cu};
  return e;
}

}  // namespace prism
