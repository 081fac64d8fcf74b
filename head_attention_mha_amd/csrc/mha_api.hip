// C ABI of the fused attention forward and backward: argument validation,
// per-device architecture check, template dispatch and launch. Declarations
// and the contract of every entry point are in include/mha.h.
#include "../../include/mha.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "mha_bwd_kernel.hpp"
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

// Host-side checks of an mha_bwd call. `*empty_q`: no query rows (dQ and D
// have no elements); `*empty_k`: no key rows (dK and dV have no elements).
mha_status_t validate_bwd(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* delta, int B, int H, int Nq, int Nk, int d, int causal,
                          float scale, int dtype, bool* empty_q, bool* empty_k) {
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
  *empty_q = (nl == 0);
  *empty_k = (nk == 0);
  if (*empty_q && *empty_k) return MHA_OK;
  if (!*empty_q && Nk < 1) return MHA_ERR_INVALID_ARG;  // softmax over no keys

  if (!*empty_q) {
    if (!q || !o || !dout || !lse || !dq || !delta) return MHA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(o, 16) || !aligned(dout, 16) || !aligned(dq, 16) ||
        !aligned(lse, 4) || !aligned(delta, 4))
      return MHA_ERR_INVALID_ARG;
  }
  if (!*empty_k) {
    if (!k || !v || !dk || !dv) return MHA_ERR_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(dk, 16) || !aligned(dv, 16))
      return MHA_ERR_INVALID_ARG;
  }
  // grid sizes of the three kernels must fit 31 bits
  const long long nqb = ((long long)Nq + mha::bwd::kBQ - 1) / mha::bwd::kBQ;
  const long long nkb = ((long long)Nk + mha::bwd::kBKV - 1) / mha::bwd::kBKV;
  if ((long long)B * H * nqb > 0x7fffffffLL || (long long)B * H * nkb > 0x7fffffffLL ||
      (long long)nl > 0x7fffffffLL)
    return MHA_ERR_INVALID_ARG;

  // every output is disjoint from every other buffer
  const void* in[6] = {q, k, v, o, dout, lse};
  const size_t in_n[6] = {nq * es, nk * es, nk * es, nq * es, nq * es, nl * 4};
  void* out[4] = {dq, dk, dv, delta};
  const size_t out_n[4] = {nq * es, nk * es, nk * es, nl * 4};
  for (int a = 0; a < 4; ++a) {
    for (int b = 0; b < 6; ++b)
      if (overlap(out[a], out_n[a], in[b], in_n[b])) return MHA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 4; ++b)
      if (overlap(out[a], out_n[a], out[b], out_n[b])) return MHA_ERR_INVALID_ARG;
  }
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

template <typename T, int D, bool C>
mha_status_t launch_bwd(const mha::BwdParams& pd, const mha::BwdParams& pq,
                        const mha::BwdParams& pk, bool run_q, bool run_k, hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (run_q) {
    void* a0[] = {const_cast<mha::BwdParams*>(&pd)};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_bwd_delta_kernel<T, D>),
                        dim3(pd.n_blocks), dim3(mha::bwd::kThreads), a0, 0, stream);
    if (e == hipSuccess) {
      void* a1[] = {const_cast<mha::BwdParams*>(&pq)};
      e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_bwd_dq_kernel<T, D, C>),
                          dim3(pq.n_blocks), dim3(mha::bwd::kThreads), a1, 0, stream);
    }
  }
  if (e == hipSuccess && run_k) {
    void* a2[] = {const_cast<mha::BwdParams*>(&pk)};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_bwd_dkdv_kernel<T, D, C>),
                        dim3(pk.n_blocks), dim3(mha::bwd::kThreads), a2, 0, stream);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

template <typename T>
mha_status_t dispatch_bwd(const mha::BwdParams& pd, const mha::BwdParams& pq,
                          const mha::BwdParams& pk, bool run_q, bool run_k, int d, bool causal,
                          hipStream_t s) {
  if (d == 64)
    return causal ? launch_bwd<T, 64, true>(pd, pq, pk, run_q, run_k, s)
                  : launch_bwd<T, 64, false>(pd, pq, pk, run_q, run_k, s);
  return causal ? launch_bwd<T, 128, true>(pd, pq, pk, run_q, run_k, s)
                : launch_bwd<T, 128, false>(pd, pq, pk, run_q, run_k, s);
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

mha_status_t mha_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                     const float* lse, void* dq, void* dk, void* dv, float* delta, int B, int H,
                     int Nq, int Nk, int d, int causal, float scale, void* stream, int dtype) {
  bool empty_q = false, empty_k = false;
  mha_status_t st = validate_bwd(q, k, v, o, dout, lse, dq, dk, dv, delta, B, H, Nq, Nk, d,
                                 causal, scale, dtype, &empty_q, &empty_k);
  if (st != MHA_OK || (empty_q && empty_k)) return st;
  st = check_device();
  if (st != MHA_OK) return st;

  mha::BwdParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<const uint16_t*>(o);
  p.dout = static_cast<const uint16_t*>(dout);
  p.lse = lse;
  p.dq = static_cast<uint16_t*>(dq);
  p.dk = static_cast<uint16_t*>(dk);
  p.dv = static_cast<uint16_t*>(dv);
  p.delta = delta;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;

  mha::BwdParams pd = p, pq = p, pk = p;
  const long long n_rows = (long long)B * H * Nq;
  const int rows_per_block = mha::bwd::kThreads / (d / 8);
  pd.n_tiles = 0;
  pd.n_blocks = (int)((n_rows + rows_per_block - 1) / rows_per_block);
  pq.n_tiles = (Nq + mha::bwd::kBQ - 1) / mha::bwd::kBQ;
  pq.n_blocks = B * H * pq.n_tiles;
  pk.n_tiles = (Nk + mha::bwd::kBKV - 1) / mha::bwd::kBKV;
  pk.n_blocks = B * H * pk.n_tiles;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool run_q = !empty_q, run_k = !empty_k;
  if (dtype == MHA_DTYPE_BF16)
    return dispatch_bwd<mha::BF16>(pd, pq, pk, run_q, run_k, d, causal != 0, s);
  return dispatch_bwd<mha::F16>(pd, pq, pk, run_q, run_k, d, causal != 0, s);
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
