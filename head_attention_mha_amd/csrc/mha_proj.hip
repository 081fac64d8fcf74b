// C ABI of the output projection after attention: validation, dispatch and
// launch of mha_proj_kernel (contract in include/mha.h).
#include "mha_common.hpp"
#include "mha_proj_kernel.hpp"

using namespace mha_host;

namespace {

mha_status_t validate_proj(const void* o, const void* w, const void* bias, void* y, int B,
                           int Nq, int H, int d, int E, int dtype, bool* empty) {
  if (B < 0 || Nq < 0 || H < 0 || d < 0 || E < 0) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_FP16 && dtype != MHA_DTYPE_BF16) return MHA_ERR_INVALID_ARG;
  const long long M = (long long)B * Nq, K = (long long)H * d;
  *empty = (M == 0 || E == 0);
  if (*empty) return MHA_OK;
  if (K == 0) return MHA_ERR_INVALID_ARG;
  if (K % mha::proj::kBK != 0 || E % 4 != 0) return MHA_ERR_UNSUPPORTED;
  if (M > 0x7fffffffLL || K > (1LL << 24)) return MHA_ERR_INVALID_ARG;
  const long long tiles = ((M + mha::proj::kBM - 1) / mha::proj::kBM) *
                          (((long long)E + mha::proj::kBN - 1) / mha::proj::kBN);
  if (tiles > 0x7fffffffLL) return MHA_ERR_INVALID_ARG;
  if (!o || !w || !y) return MHA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || !aligned(w, 16) || !aligned(y, 16) || (bias && !aligned(bias, 8)))
    return MHA_ERR_INVALID_ARG;
  const size_t es = 2;
  const size_t n_o = (size_t)M * K * es, n_w = (size_t)E * K * es, n_y = (size_t)M * E * es;
  const size_t n_b = bias ? (size_t)E * es : 0;
  if (overlap(y, n_y, o, n_o) || overlap(y, n_y, w, n_w) || overlap(y, n_y, bias, n_b))
    return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

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
