// Library-wide host helpers: error strings, version, device check.
#include "isd_common.hpp"

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

int isd_version(void) { return 100; }

// 0 if the current HIP device is a gfx950, else ISD_E_DEVICE. Cached per device.
int isd_check_device_internal(void) {
  static int cached[64];  // 0 unknown, 1 gfx950, 2 other
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return ISD_E_DEVICE;
  if (cached[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return ISD_E_DEVICE;
    cached[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  return cached[dev] == 1 ? ISD_OK : ISD_E_DEVICE;
}

}  // extern "C"
