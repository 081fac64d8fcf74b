// Host-side helpers shared by the C-ABI entry points: pointer checks,
// forward argument validation and the per-device architecture check.
#pragma once

#include "../../include/mha.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstddef>
#include <cstdint>

namespace mha_host {

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// [p, p+n) and [q, q+m) overlap (empty ranges never overlap).
inline bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + m && b < a + n;
}

// Host-side checks of a forward call (no HIP call). Returns MHA_OK if the
// call is valid and `*empty` tells whether there is nothing to compute;
// rows_per_block is the launch's query rows per workgroup (grid limit).
inline mha_status_t validate_fwd(const void* q, const void* k, const void* v, void* o,
                                 float* lse, int B, int H, int Nq, int Nk, int d, int causal,
                                 float scale, int dtype, int rows_per_block, bool* empty) {
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
  const long long n_qtiles = ((long long)Nq + rows_per_block - 1) / rows_per_block;
  if ((long long)B * H * n_qtiles > 0x7fffffffLL) return MHA_ERR_INVALID_ARG;

  if (overlap(o, nq * es, q, nq * es) || overlap(o, nq * es, k, nk * es) ||
      overlap(o, nq * es, v, nk * es) || overlap(lse, nl * 4, q, nq * es) ||
      overlap(lse, nl * 4, k, nk * es) || overlap(lse, nl * 4, v, nk * es) ||
      overlap(lse, nl * 4, o, nq * es))
    return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

// MHA_OK if the current HIP device is a gfx950 (cached per device),
// MHA_ERR_UNSUPPORTED for another architecture, MHA_ERR_DEVICE without one.
mha_status_t check_device();

}  // namespace mha_host
