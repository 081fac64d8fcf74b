// C ABI of the fused attention forward: argument validation, per-device
// architecture check, template dispatch and launch. Declarations and the
// contract of every entry point are in include/mha.h.
#include "../../include/mha.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "mha_fwd_kernel.hpp"

namespace {

// Per-device cache: 0 = unknown, 1 = gfx950, 2 = other architecture.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// [p, p+n) and [q, q+m) overlap (empty ranges never overlap).
bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

// Pure host-side checks; no HIP call. Returns MHA_OK if the call is valid
// and `*empty` tells whether there is nothing to compute.
mha_status_t validate(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int d, int causal, float scale, int dtype,
                      bool* empty) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return MHA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_FP16 && dtype != MHA_DTYPE_BF16) return MHA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MHA_ERR_INVALID_ARG;
  if (d <= 0) return MHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;

  const size_t es = 2;
  const size_t nq = (size_t)B * Nq * H * d;
  const size_t nk = (size_t)B * Nk * H * d;
  const size_t nl = (size_t)B * H * Nq;
  *empty = (nl == 0);
  if (*empty) return MHA_OK;
  if (Nk < 1) return MHA_ERR_INVALID_ARG;  // softmax over no keys is undefined

  if (!q || !k || !v || !o || !lse) return MHA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return MHA_ERR_INVALID_ARG;
  // Index arithmetic in the kernel: tokens*H*d offsets are 64-bit; the grid
  // and per-head token counts must fit 31 bits.
  const long long n_qtiles = ((long long)Nq + mha::kBQ - 1) / mha::kBQ;
  if ((long long)B * H * n_qtiles > 0x7fffffffLL) return MHA_ERR_INVALID_ARG;

  if (overlap(o, nq * es, q, nq * es) || overlap(o, nq * es, k, nk * es) ||
      overlap(o, nq * es, v, nk * es) || overlap(lse, nl * 4, q, nq * es) ||
      overlap(lse, nl * 4, k, nk * es) || overlap(lse, nl * 4, v, nk * es) ||
      overlap(lse, nl * 4, o, nq * es))
    return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

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

template <typename T, int D, bool C>
mha_status_t launch(const mha::Params& p, hipStream_t stream) {
  void* args[] = {const_cast<mha::Params*>(&p)};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_fwd_kernel<T, D, C>),
                                       dim3(p.n_blocks), dim3(mha::kThreads), args, 0, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

template <typename T>
mha_status_t dispatch_d(const mha::Params& p, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch<T, 64, true>(p, s) : launch<T, 64, false>(p, s);
  return causal ? launch<T, 128, true>(p, s) : launch<T, 128, false>(p, s);
}

}  // namespace

extern "C" {

mha_status_t mha_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                     int H, int Nq, int Nk, int d, int causal, float scale, void* stream,
                     int dtype) {
  bool empty = false;
  mha_status_t st = validate(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, &empty);
  if (st != MHA_OK || empty) return st;
  st = check_device();
  if (st != MHA_OK) return st;

  mha::Params p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.defer_raw = mha::kDeferLog2 / p.scale_log2;
  p.n_qtiles = (Nq + mha::kBQ - 1) / mha::kBQ;
  p.n_blocks = B * H * p.n_qtiles;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MHA_DTYPE_BF16) return dispatch_d<mha::BF16>(p, d, causal != 0, s);
  return dispatch_d<mha::F16>(p, d, causal != 0, s);
}

const char* mha_status_string(int status) {
  switch (status) {
    case MHA_OK:
      return "ok";
    case MHA_ERR_INVALID_ARG:
      return "invalid argument";
    case MHA_ERR_UNSUPPORTED:
      return "unsupported (head dim must be 64 or 128; device must be gfx950)";
    case MHA_ERR_DEVICE:
      return "no usable HIP device";
    case MHA_ERR_LAUNCH:
      return "kernel launch failed";
    default:
      return "unknown status";
  }
}

int mha_abi_version(void) { return MHA_ABI_VERSION; }

}  // extern "C"
