// C ABI of the attention backward: template dispatch and launch of the dQ
// kernel (which also forms D) and the dK/dV kernel (contract in
// include/mha.h; argument checks in mha_validate.hpp).
#include "mha_bwd_kernel.hpp"
#include "mha_common.hpp"

using namespace mha_host;

namespace {

template <typename T, int D, bool C>
mha_status_t launch_bwd(const mha::BwdParams& pq, const mha::BwdParams& pk, bool run_q, bool run_k,
                        hipStream_t stream) {
  hipError_t e = hipSuccess;
  if (run_q) {
    // dQ and D (the dK/dV kernel, launched after it on the same stream,
    // reads D)
    void* a1[] = {const_cast<mha::BwdParams*>(&pq)};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_bwd_dq_kernel<T, D, C>),
                        dim3(pq.n_blocks), dim3(mha::bwd::kThreads), a1, 0, stream);
  }
  if (e == hipSuccess && run_k) {
    void* a2[] = {const_cast<mha::BwdParams*>(&pk)};
    if constexpr (D == 128) {
      // producer/consumer wave pairs: two waves per SIMD
      e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_bwd_dkdv_pair_kernel<T, D, C>),
                          dim3(pk.n_blocks), dim3(2 * mha::bwd::kThreads), a2, 0, stream);
    } else {
      e = hipLaunchKernel(reinterpret_cast<const void*>(&mha::mha_bwd_dkdv_kernel<T, D, C>),
                          dim3(pk.n_blocks), dim3(mha::bwd::kThreads), a2, 0, stream);
    }
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return MHA_ERR_LAUNCH;
  }
  return MHA_OK;
}

template <typename T>
mha_status_t dispatch_bwd(const mha::BwdParams& pq, const mha::BwdParams& pk, bool run_q, bool run_k,
                          int d, bool causal, hipStream_t s) {
  if (d == 64)
    return causal ? launch_bwd<T, 64, true>(pq, pk, run_q, run_k, s)
                  : launch_bwd<T, 64, false>(pq, pk, run_q, run_k, s);
  return causal ? launch_bwd<T, 128, true>(pq, pk, run_q, run_k, s)
                : launch_bwd<T, 128, false>(pq, pk, run_q, run_k, s);
}

}  // namespace

extern "C" {

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

  mha::BwdParams pq = p, pk = p;
  pq.n_tiles = (Nq + mha::bwd::kBQ - 1) / mha::bwd::kBQ;
  pq.n_blocks = B * H * pq.n_tiles;
  pk.n_tiles = (Nk + mha::bwd::kBKV - 1) / mha::bwd::kBKV;
  pk.n_blocks = B * H * pk.n_tiles;

  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool run_q = !empty_q, run_k = !empty_k;
  if (dtype == MHA_DTYPE_BF16)
    return dispatch_bwd<mha::BF16>(pq, pk, run_q, run_k, d, causal != 0, s);
  return dispatch_bwd<mha::F16>(pq, pk, run_q, run_k, d, causal != 0, s);
}

}  // extern "C"
