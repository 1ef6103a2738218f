// Library-wide host helpers: error strings, version, device check.
#include "isd_common.hpp"

#include <atomic>
#include <cstring>

extern "C" {

const char* isd_strerror(int code) {
  switch (code) {
    case ISD_OK:
      return "success";
    case ISD_E_INVALID:
      return "invalid argument (null pointer, size, stride or alignment)";
    case ISD_E_UNSUPPORTED:
      return "unsupported dtype, head_dim, rank, stride or shape";
    case ISD_E_WORKSPACE:
      return "workspace missing, misaligned or too small";
    case ISD_E_LAUNCH:
      return "kernel launch failed";
    case ISD_E_DEVICE:
      return "current device is not a gfx950 GPU";
    default:
      return "unknown error code";
  }
}

int isd_version(void) { return 104; }

// Per-device facts, looked up once: 0 unknown, else 1 + CU count for a
// gfx950 device, or -1 for any other device.
static std::atomic<int> g_device_info[64];

static int device_info(void) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return -1;
  int info = g_device_info[dev].load(std::memory_order_relaxed);
  if (info == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
    info = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 + prop.multiProcessorCount : -1;
    g_device_info[dev].store(info, std::memory_order_relaxed);
  }
  return info;
}

// 0 if the current HIP device is a gfx950, else ISD_E_DEVICE.
int isd_check_device_internal(void) { return device_info() > 0 ? ISD_OK : ISD_E_DEVICE; }

// Compute units of the current device (gfx950 only; 256 if unknown).
int isd_device_cus_internal(void) {
  const int info = device_info();
  return info > 1 ? info - 1 : 256;
}

}  // extern "C"
