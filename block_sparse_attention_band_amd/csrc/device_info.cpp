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
}  // namespace

hipError_t stream_device(hipStream_t s, int *dev) {
  if (s == nullptr) return hipGetDevice(dev);
  return hipStreamGetDevice(s, dev);
}

hipError_t device_cu_count(int dev, int *cus) {
  if (dev < 0 || dev >= kMaxDevices) return hipDeviceGetAttribute(cus, hipDeviceAttributeMultiprocessorCount, dev);
  std::call_once(g_once[dev], [dev] {
    g_err[dev] = hipDeviceGetAttribute(&g_cus[dev], hipDeviceAttributeMultiprocessorCount, dev);
  });
  *cus = g_cus[dev];
  return g_err[dev];
}

}  // namespace prism
