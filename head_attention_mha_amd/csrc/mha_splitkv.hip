// C ABI of the split-over-keys forward, with a caller workspace or with the
// library's fixed scratch array: template dispatch and launch of the partial
// and merge kernels (contract in include/mha.h; argument checks in
// mha_validate.hpp).
#include "mha_common.hpp"
#include "mha_split_kernel.hpp"

#include <atomic>
#include <mutex>

using namespace mha_host;

namespace {

// Workspace of mha_fwd_splitkv_noalloc: one fixed array per GPU in device
// memory, held until the process ends. In host code its name is only a
// host-side stand-in; host code uses the device address that
// hipGetSymbolAddress returns for it, looked up once per device.
static __device__ __align__(256) unsigned char scratch[MHA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxScratchDevices];
std::mutex g_scratch_mu;

// Device address of the current device's scratch array.
mha_status_t scratch_of_current_device(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return MHA_ERR_DEVICE;
  }
  if (dev >= kMaxScratchDevices) return MHA_ERR_UNSUPPORTED;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
        (void)hipGetLastError();
        return MHA_ERR_DEVICE;
      }
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return MHA_OK;
}

using mha::split::kMaxSplits;
using mha::split::kSplitAlign;  // keys per split: a multiple of the partial kernel's block at d = 64

int split_len(int Nk, int n_splits) {
  const long long per = ((long long)Nk + n_splits - 1) / n_splits;
  return (int)(((per + kSplitAlign - 1) / kSplitAlign) * kSplitAlign);
}

template <typename T, int D, int NQ, bool C>
mha_status_t launch_split(const mha::SplitParams& p, hipStream_t stream) {
  void* args[] = {const_cast<mha::SplitParams*>(&p)};
  hipError_t e = hipLaunchKernel(
      reinterpret_cast<const void*>(&mha::mha_split_partial_kernel<T, D, NQ, C>),
      dim3(p.B * p.H * p.n_splits), dim3(mha::split::kThreads), args, 0, stream);
  if (e == hipSuccess) {
    const int rows = p.B * p.H * p.Nq;  // one workgroup per row
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_split_merge_kernel<T, D>),
                        dim3(rows), dim3(mha::split::kThreads), args, 0, stream);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

template <typename T, int D, bool C>
mha_status_t dispatch_split_nq(const mha::SplitParams& p, hipStream_t s) {
  if (p.Nq <= 1) return launch_split<T, D, 1, C>(p, s);
  if (p.Nq <= 2) return launch_split<T, D, 2, C>(p, s);
  if (p.Nq <= 4) return launch_split<T, D, 4, C>(p, s);
  return launch_split<T, D, 8, C>(p, s);
}

template <typename T>
mha_status_t dispatch_split(const mha::SplitParams& p, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? dispatch_split_nq<T, 64, true>(p, s) : dispatch_split_nq<T, 64, false>(p, s);
  return causal ? dispatch_split_nq<T, 128, true>(p, s) : dispatch_split_nq<T, 128, false>(p, s);
}

// Launch of the partial and merge kernels for a validated call whose
// workspace is (o_part, lse_part).
mha_status_t run_split(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                       int H, int Nq, int Nk, int d, int causal, float scale, int n_splits,
                       float* o_part, float* lse_part, void* stream, int dtype) {
  mha::SplitParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.o_part = o_part;
  p.lse_part = lse_part;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.n_splits = n_splits;
  p.split_len = split_len(Nk, n_splits);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MHA_DTYPE_BF16) return dispatch_split<mha::BF16>(p, d, causal != 0, s);
  return dispatch_split<mha::F16>(p, d, causal != 0, s);
}

}  // namespace

extern "C" {

int mha_fwd_splitkv_splits(int B, int H, int Nq, int Nk) {
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1) return 1;
  // about 2048 workgroups in flight, each split at least one 256-key block
  const long long bh = (long long)B * H;
  long long n = (2048 + bh - 1) / bh;
  const long long max_by_keys = ((long long)Nk + kSplitAlign - 1) / kSplitAlign;
  if (n > max_by_keys) n = max_by_keys;
  if (n > kMaxSplits) n = kMaxSplits;
  return n < 1 ? 1 : (int)n;
}

mha_status_t mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse,
                             int B, int H, int Nq, int Nk, int d, int causal, float scale,
                             int n_splits, float* o_part, float* lse_part, void* stream,
                             int dtype) {
  bool empty = false;
  mha_status_t st = validate_splitkv(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, n_splits,
                                     o_part, lse_part, dtype, &empty);
  if (st != MHA_OK || empty) return st;
  st = check_device();
  if (st != MHA_OK) return st;
  return run_split(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, n_splits, o_part, lse_part,
                   stream, dtype);
}

mha_status_t mha_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Nq, int Nk, int d, int causal,
                                     float scale, int n_splits, void* stream, int dtype) {
  bool empty = false;
  mha_status_t st = validate_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale,
                                             n_splits, dtype, MHA_NOALLOC_SCRATCH_BYTES, &empty);
  if (st != MHA_OK || empty) return st;
  st = check_device();
  if (st != MHA_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != MHA_OK) return st;
  // partial outputs first, the partial LSEs after them (256-byte aligned)
  float* o_part = static_cast<float*>(ws);
  float* lse_part = reinterpret_cast<float*>(static_cast<unsigned char*>(ws) +
                                             splitkv_opart_bytes(B, H, Nq, d, n_splits));
  return run_split(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, n_splits, o_part, lse_part,
                   stream, dtype);
}

}  // extern "C"
