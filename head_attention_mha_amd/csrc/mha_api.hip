// C ABI: the per-device architecture check and the status/version entry
// points. The operations themselves are in mha_fwd.hip, mha_splitkv.hip and
// mha_bwd.hip; declarations and contracts are in include/mha.h.
#include "mha_common.hpp"

#include <atomic>
#include <cstring>

namespace mha_host {

namespace {
// Per-device cache: 0 = unknown, 1 = gfx950, 2 = other architecture.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];
}  // namespace

mha_status_t check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MHA_ERR_DEVICE;
  }
  if (dev < kMaxDevices) {
    const int cached = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (cached == 1) return MHA_OK;
    if (cached == 2) return MHA_ERR_UNSUPPORTED;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_DEVICE;
  }
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? MHA_OK : MHA_ERR_UNSUPPORTED;
}

}  // namespace mha_host

extern "C" {

const char* mha_status_string(int status) {
  switch (status) {
    case MHA_OK:
      return "ok";
    case MHA_ERR_INVALID_ARG:
      return "invalid argument";
    case MHA_ERR_UNSUPPORTED:
      return "unsupported (head dim must be 64 or 128, at most 8 query rows for the split-KV "
             "forward; device must be gfx950)";
    case MHA_ERR_DEVICE:
      return "no usable HIP device";
    case MHA_ERR_LAUNCH:
      return "kernel launch failed";
    case MHA_ERR_SCRATCH_TOO_SMALL:
      return "the problem's split workspace exceeds the fixed scratch of mha_fwd_splitkv_noalloc "
             "(MHA_NOALLOC_SCRATCH_BYTES); use mha_fwd_splitkv with a workspace";
    default:
      return "unknown status";
  }
}

int mha_abi_version(void) { return MHA_ABI_VERSION; }

}  // extern "C"
