// C ABI of the output projection after attention: dispatch and launch of
// mha_proj_kernel (contract in include/mha.h; argument checks in
// mha_validate.hpp).
#include "mha_common.hpp"
#include "mha_proj_kernel.hpp"

using namespace mha_host;

namespace {

template <typename T>
mha_status_t launch_proj(const mha::ProjParams& p, hipStream_t stream) {
  void* args[] = {const_cast<mha::ProjParams*>(&p)};
  const hipError_t e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_proj_kernel<T>),
                                       dim3(p.n_tiles), dim3(mha::proj::kThreads), args, 0, stream);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

}  // namespace

extern "C" {

mha_status_t mha_out_proj(const void* o, const void* w, const void* bias, void* y, int B, int Nq,
                          int H, int d, int E, void* stream, int dtype) {
  bool empty = false;
  mha_status_t st = validate_proj(o, w, bias, y, B, Nq, H, d, E, dtype, &empty);
  if (st != MHA_OK || empty) return st;
  st = check_device();
  if (st != MHA_OK) return st;

  mha::ProjParams p;
  p.x = static_cast<const uint16_t*>(o);
  p.w = static_cast<const uint16_t*>(w);
  p.bias = static_cast<const uint16_t*>(bias);
  p.y = static_cast<uint16_t*>(y);
  p.M = B * Nq;
  p.N = E;
  p.K = H * d;
  p.tiles_n = (E + mha::proj::kBN - 1) / mha::proj::kBN;
  p.n_tiles = p.tiles_n * ((p.M + mha::proj::kBM - 1) / mha::proj::kBM);

  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == MHA_DTYPE_BF16) return launch_proj<mha::BF16>(p, s);
  return launch_proj<mha::F16>(p, s);
}

}  // extern "C"
