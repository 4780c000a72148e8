// Host-side pieces of the library shared by its entry points: the device
// check, the aliasing test and the status strings.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "fa2.h"
#include "fa2_host.h"

namespace fa2_host {

namespace {

// Per-device verdict on whether the device is gfx950 (0 unknown, 1 yes,
// 2 no) and its compute-unit count, both cached on first use.
constexpr int kMaxDevices = 64;
std::atomic<int> g_device_ok[kMaxDevices];
std::atomic<int> g_device_cus[kMaxDevices];

}  // namespace

int check_device(int* n_cu) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return FA2_ERR_NO_DEVICE;
  }
  int verdict = g_device_ok[dev].load(std::memory_order_acquire);
  if (verdict == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return FA2_ERR_NO_DEVICE;
    }
    verdict = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_device_cus[dev].store(prop.multiProcessorCount > 0 ? prop.multiProcessorCount : 1,
                            std::memory_order_relaxed);
    g_device_ok[dev].store(verdict, std::memory_order_release);
  }
  *n_cu = g_device_cus[dev].load(std::memory_order_relaxed);
  return verdict == 1 ? FA2_OK : FA2_ERR_NO_DEVICE;
}

}  // namespace fa2_host

extern "C" int fa2_supported(int D, int dtype) {
  return (D == 64 || D == 128 || D == 256) && (dtype == FA2_F16 || dtype == FA2_BF16);
}

extern "C" const char* fa2_status_string(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL: return "a tensor pointer is NULL";
    case FA2_ERR_SHAPE:
      return "B, H and S must be >= 1, B and H <= 65535, B*H*S*D elements (and their bytes) "
             "within int64, the grid within 2^31 workgroups, and 256 rows of a K or V "
             "sequence stride within 2^31 bytes";
    case FA2_ERR_HEADDIM: return "head dimension must be 64, 128 or 256";
    case FA2_ERR_DTYPE: return "dtype must be FA2_F16 or FA2_BF16";
    case FA2_ERR_ALIGN: return "q, k, v and o must be 16-byte aligned and lse 4-byte aligned";
    case FA2_ERR_SCALE: return "scale must be finite (FP8 descales finite and > 0)";
    case FA2_ERR_NO_DEVICE: return "no current HIP device, or it is not a gfx950 (MI355X)";
    case FA2_ERR_LAUNCH: return "the HIP runtime reported an error at kernel launch";
    case FA2_ERR_ALIAS: return "o or lse overlaps q, k, v or each other (or the workspace overlaps any of them)";
    case FA2_ERR_STRIDE:
      return "strides must be in [0, 2^40] and multiples of 8, sequence strides >= D, and o's "
             "rows must not overlap";
    case FA2_ERR_SCRATCH:
      return "the call needs more scratch than the no-allocation entry point's fixed "
             "FA2_SCRATCH_BYTES; pass a workspace to fa2_fwd_splitkv instead";
    case FA2_ERR_WORKSPACE:
      return "the workspace is NULL, not 16-byte aligned, or smaller than fa2_splitkv_workspace_bytes";
    default: return "unknown fa2 status";
  }
}
