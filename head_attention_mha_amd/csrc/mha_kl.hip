// C ABI of the fused attention KL divergence: template dispatch and launch
// of mha_kl_kernel (contract in include/mha.h; argument checks in
// mha_validate.hpp).
#include "mha_common.hpp"
#include "mha_kl_kernel.hpp"

using namespace mha_host;

namespace {

template <typename T, int D, bool C>
mha_status_t launch_kl(const mha::KlParams& p, hipStream_t stream) {
  void* args[] = {const_cast<mha::KlParams*>(&p)};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_kl_kernel<T, D, C>),
                                       dim3(p.n_blocks), dim3(mha::kl::kThreads), args, 0, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

template <typename T>
mha_status_t dispatch_kl(const mha::KlParams& p, int d, bool causal, hipStream_t s) {
  if (d == 64) return causal ? launch_kl<T, 64, true>(p, s) : launch_kl<T, 64, false>(p, s);
  return causal ? launch_kl<T, 128, true>(p, s) : launch_kl<T, 128, false>(p, s);
}

}  // namespace

extern "C" {

mha_status_t mha_kl_fwd(const void* q1, const void* k1, const void* q2, const void* k2,
                        float* kl, float* lse1, float* lse2, int B, int H, int Nq, int Nk,
                        int d, int causal, float scale, void* stream, int dtype) {
  bool empty = false;
  mha_status_t st = validate_kl(q1, k1, q2, k2, kl, lse1, lse2, B, H, Nq, Nk, d, causal, scale,
                                dtype, &empty);
  if (st != MHA_OK || empty) return st;
  st = check_device();
  if (st != MHA_OK) return st;

  mha::KlParams p;
  p.q1 = static_cast<const uint16_t*>(q1);
  p.k1 = static_cast<const uint16_t*>(k1);
  p.q2 = static_cast<const uint16_t*>(q2);
  p.k2 = static_cast<const uint16_t*>(k2);
  p.kl = kl;
  p.lse1 = lse1;
  p.lse2 = lse2;
  p.B = B;
  p.H = H;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.defer_raw = mha::kDeferLog2 / p.scale_log2;
  p.n_tiles = (Nq + mha::kl::kBQ - 1) / mha::kl::kBQ;
  p.n_blocks = B * H * p.n_tiles;

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MHA_DTYPE_BF16) return dispatch_kl<mha::BF16>(p, d, causal != 0, s);
  return dispatch_kl<mha::F16>(p, d, causal != 0, s);
}

}  // extern "C"
