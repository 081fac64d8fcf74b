// Host-side argument checks of every C-ABI entry point (contracts in
// include/mha.h): pointers, sizes, flags and the limits the kernels' index
// arithmetic needs. Plain C++ with no HIP dependency, so the same code also
// builds on its own for host-only test programs (e.g. under AddressSanitizer
// and UndefinedBehaviorSanitizer). No function here makes a HIP call.
#pragma once

#include "../../include/mha.h"
#include "mha_tiles.hpp"

#include <cmath>
#include <cstddef>
#include <cstdint>
#include <initializer_list>

namespace mha_host {

inline bool aligned(const void* p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

// [p, p+n) and [q, q+m) overlap (empty ranges never overlap); no sum that
// could wrap past the end of the address space is formed.
inline bool overlap(const void* p, size_t n, const void* q, size_t m) {
  if (n == 0 || m == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a <= b ? b - a < n : a - b < m;
}

// Element counts and grid sizes are products of int arguments. They are
// formed with overflow checks: `*out` = the product of the non-negative
// factors, false if it exceeds `limit` (nothing overflows on the way).
inline bool product(long long* out, std::initializer_list<long long> factors, long long limit) {
  long long r = 1;
  for (long long f : factors) {
    if (f == 0) {
      *out = 0;
      return true;
    }
  }
  for (long long f : factors) {
    if (f < 0 || r > limit / f) return false;
    r *= f;
  }
  *out = r;
  return true;
}
// No tensor the kernels address exceeds 2^60 elements; grids stay below 2^31
// workgroups.
constexpr long long kMaxElems = 1LL << 60;
constexpr long long kMaxGrid = 0x7fffffffLL;

// The kernels address a workgroup's tile of up to 256 token rows through one
// buffer resource with 32-bit byte offsets and range: 256 rows of H*d
// two-byte elements must span at most 4 GiB, i.e. H*d <= 2^23 elements per
// token row. Larger rows would wrap the offsets, so they are rejected.
constexpr long long kMaxRowElems = 1LL << 23;

inline bool row_fits(int H, int d) { return (long long)H * d <= kMaxRowElems; }

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
  if (!row_fits(H, d)) return MHA_ERR_INVALID_ARG;

  long long nl = 0, nq = 0, nk = 0, grid = 0;
  if (!product(&nl, {B, H, Nq}, kMaxElems)) return MHA_ERR_INVALID_ARG;
  *empty = (nl == 0);
  if (*empty) return MHA_OK;
  if (Nk < 1) return MHA_ERR_INVALID_ARG;  // softmax over no keys is undefined
  if (!product(&nq, {B, Nq, H, d}, kMaxElems) || !product(&nk, {B, Nk, H, d}, kMaxElems))
    return MHA_ERR_INVALID_ARG;

  if (!q || !k || !v || !o || !lse) return MHA_ERR_INVALID_ARG;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return MHA_ERR_INVALID_ARG;
  // Index arithmetic in the kernel: tokens*H*d offsets to a tile's first row
  // are 64-bit, offsets within a tile 32-bit (row_fits above); the grid and
  // per-head token counts must fit 31 bits.
  const long long n_qtiles = ((long long)Nq + rows_per_block - 1) / rows_per_block;
  if (!product(&grid, {B, H, n_qtiles}, kMaxGrid)) return MHA_ERR_INVALID_ARG;
  const size_t es = 2;

  if (overlap(o, nq * es, q, nq * es) || overlap(o, nq * es, k, nk * es) ||
      overlap(o, nq * es, v, nk * es) || overlap(lse, nl * 4, q, nq * es) ||
      overlap(lse, nl * 4, k, nk * es) || overlap(lse, nl * 4, v, nk * es) ||
      overlap(lse, nl * 4, o, nq * es))
    return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

// Host-side checks of an mha_fwd_splitkv call, apart from its workspace.
inline mha_status_t validate_splitkv_args(const void* q, const void* k, const void* v, void* o,
                                          float* lse, int B, int H, int Nq, int Nk, int d,
                                          int causal, float scale, int n_splits, int dtype,
                                          bool* empty) {
  bool e = false;
  mha_status_t st = validate_fwd(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale, dtype, 1, &e);
  if (st != MHA_OK) return st;
  if (n_splits < 1 || n_splits > mha::split::kMaxSplits) return MHA_ERR_INVALID_ARG;
  *empty = e;
  if (e) return MHA_OK;
  if (Nq > mha::split::kMaxNq) return MHA_ERR_UNSUPPORTED;
  long long g1 = 0, g2 = 0, n_opl = 0;
  if (!product(&g1, {B, H, n_splits}, kMaxGrid) || !product(&g2, {B, H, Nq}, kMaxGrid) ||
      (long long)Nk + mha::split::kSplitAlign > kMaxGrid)
    return MHA_ERR_INVALID_ARG;
  if (!product(&n_opl, {n_splits, B, H, Nq, d}, kMaxElems)) return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

// Bytes of the split-KV workspace: the partial outputs [n_splits, B, H, Nq, d]
// fp32, padded to 256 bytes, then the partial LSEs [n_splits, B, H, Nq] fp32.
// Valid for sizes validate_splitkv_args accepted.
inline size_t splitkv_opart_bytes(int B, int H, int Nq, int d, int n_splits) {
  const size_t n = (size_t)n_splits * B * H * Nq * d * 4;
  return (n + 255) / 256 * 256;
}
inline size_t splitkv_workspace_bytes(int B, int H, int Nq, int d, int n_splits) {
  return splitkv_opart_bytes(B, H, Nq, d, n_splits) + (size_t)n_splits * B * H * Nq * 4;
}

// Host-side checks of an mha_fwd_splitkv call with a caller workspace.
inline mha_status_t validate_splitkv(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Nq, int Nk, int d, int causal,
                                     float scale, int n_splits, float* o_part, float* lse_part,
                                     int dtype, bool* empty) {
  mha_status_t st = validate_splitkv_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale,
                                          n_splits, dtype, empty);
  if (st != MHA_OK || *empty) return st;
  if (!o_part || !lse_part || !aligned(o_part, 16) || !aligned(lse_part, 4))
    return MHA_ERR_INVALID_ARG;
  // sizes below are bounded by the products validate_splitkv_args checked
  const size_t es = 2;
  const size_t nq = (size_t)B * Nq * H * d;
  const size_t nk = (size_t)B * Nk * H * d;
  const size_t nl = (size_t)B * H * Nq;
  const size_t n_op = (size_t)n_splits * nl * d * 4, n_lp = (size_t)n_splits * nl * 4;
  const void* bufs[5] = {q, k, v, o, lse};
  const size_t sizes[5] = {nq * es, nk * es, nk * es, nq * es, nl * 4};
  for (int i = 0; i < 5; ++i)
    if (overlap(o_part, n_op, bufs[i], sizes[i]) || overlap(lse_part, n_lp, bufs[i], sizes[i]))
      return MHA_ERR_INVALID_ARG;
  if (overlap(o_part, n_op, lse_part, n_lp)) return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

// Host-side checks of an mha_fwd_splitkv_noalloc call: as mha_fwd_splitkv's,
// and the workspace must fit the library's fixed scratch of `scratch_bytes`
// (MHA_ERR_SCRATCH_TOO_SMALL otherwise).
inline mha_status_t validate_splitkv_noalloc(const void* q, const void* k, const void* v,
                                             void* o, float* lse, int B, int H, int Nq, int Nk,
                                             int d, int causal, float scale, int n_splits,
                                             int dtype, size_t scratch_bytes, bool* empty) {
  mha_status_t st = validate_splitkv_args(q, k, v, o, lse, B, H, Nq, Nk, d, causal, scale,
                                          n_splits, dtype, empty);
  if (st != MHA_OK || *empty) return st;
  if (splitkv_workspace_bytes(B, H, Nq, d, n_splits) > scratch_bytes)
    return MHA_ERR_SCRATCH_TOO_SMALL;
  return MHA_OK;
}

// Host-side checks of an mha_bwd call. `*empty_q`: no query rows (dQ and D
// have no elements); `*empty_k`: no key rows (dK and dV have no elements).
inline mha_status_t validate_bwd(const void* q, const void* k, const void* v, const void* o,
                          const void* dout, const float* lse, void* dq, void* dk, void* dv,
                          float* delta, int B, int H, int Nq, int Nk, int d, int causal,
                          float scale, int dtype, bool* empty_q, bool* empty_k) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return MHA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_FP16 && dtype != MHA_DTYPE_BF16) return MHA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MHA_ERR_INVALID_ARG;
  if (d <= 0) return MHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  if (!row_fits(H, d)) return MHA_ERR_INVALID_ARG;

  long long nql = 0, nkl = 0, nll = 0;
  if (!product(&nql, {B, Nq, H, d}, kMaxElems) || !product(&nkl, {B, Nk, H, d}, kMaxElems) ||
      !product(&nll, {B, H, Nq}, kMaxElems))
    return MHA_ERR_INVALID_ARG;
  const size_t es = 2;
  const size_t nq = (size_t)nql, nk = (size_t)nkl, nl = (size_t)nll;
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
  long long g1 = 0, g2 = 0;
  if (!product(&g1, {B, H, nqb}, kMaxGrid) || !product(&g2, {B, H, nkb}, kMaxGrid) ||
      nll > kMaxGrid)
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

// Host-side checks of an mha_kl_fwd call; `*empty`: no query rows.
inline mha_status_t validate_kl(const void* q1, const void* k1, const void* q2, const void* k2,
                         float* kl, float* lse1, float* lse2, int B, int H, int Nq, int Nk,
                         int d, int causal, float scale, int dtype, bool* empty) {
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0) return MHA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_FP16 && dtype != MHA_DTYPE_BF16) return MHA_ERR_INVALID_ARG;
  if (!std::isfinite(scale) || !(scale > 0.f)) return MHA_ERR_INVALID_ARG;
  if (d <= 0) return MHA_ERR_INVALID_ARG;
  if (d != 64 && d != 128) return MHA_ERR_UNSUPPORTED;
  if (!row_fits(H, d)) return MHA_ERR_INVALID_ARG;
  long long nll = 0, nql = 0, nkl = 0, grid = 0;
  if (!product(&nll, {B, H, Nq}, kMaxElems)) return MHA_ERR_INVALID_ARG;
  *empty = (nll == 0);
  if (*empty) return MHA_OK;
  if (Nk < 1) return MHA_ERR_INVALID_ARG;  // a softmax over no keys is undefined
  if (!product(&nql, {B, Nq, H, d}, kMaxElems) || !product(&nkl, {B, Nk, H, d}, kMaxElems))
    return MHA_ERR_INVALID_ARG;
  const size_t es = 2;
  const size_t nq = (size_t)nql, nk = (size_t)nkl, nl = (size_t)nll;
  if (!q1 || !k1 || !q2 || !k2 || !kl || !lse1 || !lse2) return MHA_ERR_INVALID_ARG;
  if (!aligned(q1, 16) || !aligned(k1, 16) || !aligned(q2, 16) || !aligned(k2, 16) ||
      !aligned(kl, 4) || !aligned(lse1, 4) || !aligned(lse2, 4))
    return MHA_ERR_INVALID_ARG;
  const long long n_qtiles = ((long long)Nq + mha::kl::kBQ - 1) / mha::kl::kBQ;
  if (!product(&grid, {B, H, n_qtiles}, kMaxGrid)) return MHA_ERR_INVALID_ARG;
  const void* in[4] = {q1, k1, q2, k2};
  const size_t in_n[4] = {nq * es, nk * es, nq * es, nk * es};
  float* out[3] = {kl, lse1, lse2};
  for (int a = 0; a < 3; ++a) {
    for (int b = 0; b < 4; ++b)
      if (overlap(out[a], nl * 4, in[b], in_n[b])) return MHA_ERR_INVALID_ARG;
    for (int b = a + 1; b < 3; ++b)
      if (overlap(out[a], nl * 4, out[b], nl * 4)) return MHA_ERR_INVALID_ARG;
  }
  return MHA_OK;
}

// Host-side checks of an mha_out_proj call; `*empty`: nothing to write.
inline mha_status_t validate_proj(const void* o, const void* w, const void* bias, void* y, int B,
                           int Nq, int H, int d, int E, int dtype, bool* empty) {
  if (B < 0 || Nq < 0 || H < 0 || d < 0 || E < 0) return MHA_ERR_INVALID_ARG;
  if (dtype != MHA_DTYPE_FP16 && dtype != MHA_DTYPE_BF16) return MHA_ERR_INVALID_ARG;
  const long long M = (long long)B * Nq, K = (long long)H * d;
  *empty = (M == 0 || E == 0);
  if (*empty) return MHA_OK;
  if (K == 0) return MHA_ERR_INVALID_ARG;
  // a stage's 256 rows of K elements span at most 4 GiB (32-bit offsets)
  if (M > kMaxGrid || K > kMaxRowElems) return MHA_ERR_INVALID_ARG;
  if (K % mha::proj::kBK != 0 || E % 4 != 0) return MHA_ERR_UNSUPPORTED;
  long long tiles = 0, n_ol = 0, n_wl = 0, n_yl = 0;
  if (!product(&tiles, {(M + mha::proj::kBM - 1) / mha::proj::kBM,
                        ((long long)E + mha::proj::kBN - 1) / mha::proj::kBN}, kMaxGrid) ||
      !product(&n_ol, {M, K}, kMaxElems) || !product(&n_wl, {E, K}, kMaxElems) ||
      !product(&n_yl, {M, E}, kMaxElems))
    return MHA_ERR_INVALID_ARG;
  if (!o || !w || !y) return MHA_ERR_INVALID_ARG;
  if (!aligned(o, 16) || !aligned(w, 16) || !aligned(y, 16) || (bias && !aligned(bias, 8)))
    return MHA_ERR_INVALID_ARG;
  const size_t es = 2;
  const size_t n_o = (size_t)n_ol * es, n_w = (size_t)n_wl * es, n_y = (size_t)n_yl * es;
  const size_t n_b = bias ? (size_t)E * es : 0;
  if (overlap(y, n_y, o, n_o) || overlap(y, n_y, w, n_w) || overlap(y, n_y, bias, n_b))
    return MHA_ERR_INVALID_ARG;
  return MHA_OK;
}

}  // namespace mha_host
