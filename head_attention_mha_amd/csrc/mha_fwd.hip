// C ABI of the fused attention forward: template dispatch and launch of
// mha_fwd_kernel (contract in include/mha.h).
#include "mha_common.hpp"
#include "mha_fwd_kernel.hpp"

using namespace mha_host;

namespace {

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
  mha_status_t st = validate_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, mha::kBQ,
                                 &empty);
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

}  // extern "C"
