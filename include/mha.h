/*
 * mha.h -- C ABI of the fused multi-head attention forward (whole, or split
 * over the keys for decoding), its backward, the fused attention KL
 * divergence and the output projection, for AMD MI355X (gfx950 / CDNA4).
 *
 * The operation (per batch b and head h) is
 *
 *     O = softmax(scale * Q K^T  [+ causal mask]) V
 *     LSE_i = ln( sum_j exp(scale * q_i . k_j) )   over the visible keys j
 *
 * - the attention formula: "CANN ops-transformer" article, section 1 (the MHA
 *   formula softmax(QK^T / sqrt(d_k)) V), and "SparkAttention", MHA-Forward
 *   passage (Eq. 1: per head, heads split the embedding);
 * - the fused, tiled evaluation that never writes the Nq x Nk score matrix to
 *   memory and writes O once: "SparkAttention", Fig. 6 passage (steps 1-4 and
 *   the final write-back), and the FlashAttention long-sequence post,
 *   "Attention parallelism" (row blocks per worker);
 * - LSE = m + log l with m the running row max and l the running row sum:
 *   "StreamKL", Methodology section 1 (online formulation) and section 2 (the
 *   stored LSE from which P = exp(S - LSE) is regenerated);
 * - causal: key j is visible to query i iff j <= i (top-left aligned, also
 *   when Nq != Nk): "SparkAttention", Transformer data-flow passage (Fig. 1),
 *   the masked decoder attention, read inclusively. Whole key tiles past the
 *   causal frontier are skipped: "StreamKL", Methodology section 1.
 */
#ifndef MHA_MI355X_H
#define MHA_MI355X_H

/* Symbols the library exports (it is built with hidden default visibility). */
#if defined(__GNUC__)
#define MHA_API __attribute__((visibility("default")))
#else
#define MHA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum {
  MHA_OK = 0,
  MHA_ERR_INVALID_ARG = 1, /* a null/misaligned/overlapping pointer, a bad size, flag or scale */
  MHA_ERR_UNSUPPORTED = 2, /* valid but not implemented: head dim other than 64/128, device not gfx950 */
  MHA_ERR_DEVICE = 3,      /* no usable HIP device (e.g. a host without a GPU) */
  MHA_ERR_LAUNCH = 4,      /* the kernel launch itself failed */
  MHA_ERR_SCRATCH_TOO_SMALL = 5 /* mha_fwd_splitkv_noalloc: the problem's workspace exceeds
                                   MHA_NOALLOC_SCRATCH_BYTES */
} mha_status_t;

/* Element type of Q, K, V and O (LSE is always fp32). */
typedef enum { MHA_DTYPE_FP16 = 0, MHA_DTYPE_BF16 = 1 } mha_dtype_t;

/*
 * mha_fwd -- fused attention forward: writes O and LSE.
 *
 * Arguments
 *   q      device pointer, [B, Nq, H, d] row-major, element type `dtype`
 *   k, v   device pointers, [B, Nk, H, d] row-major, element type `dtype`
 *   o      device pointer, [B, Nq, H, d] row-major, element type `dtype`
 *          (written; each element is the fp32 result rounded to nearest even)
 *   lse    device pointer, [B, H, Nq] fp32 (written; natural log)
 *   B, H   batch size and number of heads, >= 0
 *   Nq, Nk query and key/value sequence lengths, >= 0; Nk >= 1 whenever
 *          B*H*Nq > 0 (a softmax over no keys is undefined)
 *   d      head dimension: 64 or 128
 *   causal 0 or 1 (1: key j visible to query i iff j <= i)
 *   scale  softmax scale applied to q.k, finite and > 0 (typically 1/sqrt(d)).
 *          The definition itself admits any finite scale; the restriction
 *          to scale > 0 is this implementation's: the kernels defer the
 *          rescale of O while a row's running maximum of the raw scores q.k
 *          grows by less than a fixed margin, which assumes exp(scale * x)
 *          increases with x.
 *   stream hipStream_t to enqueue on, passed as void*; NULL = default stream
 *   dtype  MHA_DTYPE_FP16 or MHA_DTYPE_BF16
 *
 * Layout: the [S, H*D] per-sequence layout of the CANN article, section 1,
 * with a leading batch dimension; no strides other than these.
 *
 * Ownership and execution: every pointer belongs to the caller and must stay
 * valid until the enqueued work completes. The library allocates nothing,
 * keeps no workspace and retains no pointer. q, k and v are only read; o and
 * lse are overwritten entirely. The call enqueues one kernel on `stream` and
 * returns without synchronising. It is reentrant; calls on one stream run in
 * order, calls on different streams that write the same o/lse race.
 *
 * Requirements checked before anything is enqueued (violations return
 * MHA_ERR_INVALID_ARG and write nothing): q, k, v, o non-null and 16-byte
 * aligned, lse non-null and 4-byte aligned (null is accepted only for a
 * tensor with zero elements); o and lse must not overlap each other or any
 * input; H*d <= 2^23 (a workgroup addresses 256 token rows with 32-bit byte
 * offsets); fewer than 2^31 workgroups (B*H*ceil(Nq/256)); no tensor above
 * 2^60 elements. Sizes are multiplied with overflow checks, so any int
 * arguments are safe to pass. An empty problem (B*H*Nq == 0) returns MHA_OK
 * and enqueues nothing.
 *
 * Errors are reported only through the return value: nothing is printed,
 * nothing aborts, no C++ exception crosses this boundary. A fault inside the
 * kernel (e.g. a pointer to too small a buffer) surfaces at the caller's next
 * synchronisation of `stream`.
 */
MHA_API mha_status_t mha_fwd(const void* q, const void* k, const void* v, void* o,
                             float* lse, int B, int H, int Nq, int Nk, int d, int causal,
                             float scale, void* stream, int dtype);

/*
 * mha_fwd_splitkv -- the same forward (O and LSE, as mha_fwd) for few query
 * rows, split over the keys: for decoding (one or a few new tokens per
 * sequence against a long key/value cache).
 *
 * Workgroup (b, h, s) computes the softmax over the keys of split s,
 * [s*L, (s+1)*L) with L = n_splits-th of Nk rounded up to 256 keys, giving a
 * normalised partial O_s and its LSE_s per query row; a second kernel merges
 * a row's splits with LSE = log sum_s exp(LSE_s) and
 * O = sum_s exp(LSE_s - LSE) O_s ("StreamKL", Methodology section 3: keys
 * split across thread blocks when NQ is small; the LSE as in its section 1).
 * The result equals mha_fwd's up to rounding.
 *
 * Arguments: as for mha_fwd, plus
 *   n_splits  number of key splits, 1 .. 256 (mha_fwd_splitkv_splits gives
 *             a default); splits past the last key compute nothing
 *   o_part    device pointer, fp32, n_splits*B*H*Nq*d elements, 16-byte
 *             aligned: the caller's workspace for the partial outputs,
 *             layout [n_splits, B, H, Nq, d] (overwritten)
 *   lse_part  device pointer, fp32, n_splits*B*H*Nq elements, 4-byte
 *             aligned: workspace for the partial LSEs, [n_splits, B, H, Nq]
 *             (overwritten; -inf where a split has no visible key)
 * Supported: Nq <= 8 (larger Nq returns MHA_ERR_UNSUPPORTED: use mha_fwd).
 *
 * Ownership and execution: as for mha_fwd; the library allocates nothing,
 * the workspace belongs to the caller and may be reused once the enqueued
 * work has completed (calls on one stream may share it). Two kernels are
 * enqueued on `stream`. The workspace must not overlap any other argument
 * (checked: MHA_ERR_INVALID_ARG). Other errors as for mha_fwd.
 */
MHA_API mha_status_t mha_fwd_splitkv(const void* q, const void* k, const void* v, void* o,
                                     float* lse, int B, int H, int Nq, int Nk, int d,
                                     int causal, float scale, int n_splits, float* o_part,
                                     float* lse_part, void* stream, int dtype);

/*
 * mha_fwd_splitkv_noalloc -- mha_fwd_splitkv without a workspace argument and
 * without any allocation, for callers that cannot allocate device memory:
 * code being captured into a HIP graph, tight serving loops, and harnesses
 * that forbid hipMalloc during a step.
 *
 * The partial outputs and LSEs go to a scratch array the library holds in
 * device memory: one per GPU, MHA_NOALLOC_SCRATCH_BYTES bytes, kept from the
 * library's first use of that device until the process ends. The call
 * allocates nothing (no hipMalloc/hipFree, no allocating
 * library routine): its first call on a device only looks up the array's
 * device address. The workspace a call needs,
 *     n_splits*B*H*Nq*d*4 bytes (rounded up to 256) + n_splits*B*H*Nq*4 bytes,
 * must fit: larger problems return MHA_ERR_SCRATCH_TOO_SMALL and enqueue
 * nothing (use mha_fwd_splitkv with a workspace of their own). E.g. at the
 * default n_splits, B=1, H=32, Nq=1, Nk=32768, d=128 needs 1.1 MB.
 *
 * Arguments, results and other errors: as for mha_fwd_splitkv, without
 * o_part and lse_part. The kernels overwrite every workspace entry they
 * read, so nothing carries over from the previous call.
 *
 * Concurrency: every call on one GPU uses that GPU's one scratch array.
 * Calls that may run at the same time on one GPU (on different streams, or
 * from different host threads onto different streams) race on it and give
 * undefined results; calls on one stream run in order and are safe.
 */
#define MHA_NOALLOC_SCRATCH_BYTES (16u << 20)
MHA_API mha_status_t mha_fwd_splitkv_noalloc(const void* q, const void* k, const void* v,
                                             void* o, float* lse, int B, int H, int Nq, int Nk,
                                             int d, int causal, float scale, int n_splits,
                                             void* stream, int dtype);

/*
 * Suggested n_splits for mha_fwd_splitkv: enough splits for about 2048
 * workgroups, each split at least 256 keys, at most 256 splits; 1 for
 * invalid sizes. Pure host function.
 */
MHA_API int mha_fwd_splitkv_splits(int B, int H, int Nq, int Nk);

/*
 * mha_kl_fwd -- fused attention KL divergence: writes KL(P1 || P2) per query
 * row and the two LSEs.
 *
 *     P_t = softmax(scale * Q_t K_t^T  [+ causal mask]),  t = 1, 2
 *     KL_i = sum_j P1_ij (log P1_ij - log P2_ij)
 *     LSE_t,i = ln( sum_j exp(scale * q_t,i . k_t,j) )  over the visible keys
 *
 * computed in one pass over the keys with five running scalars per row
 * (m1, m2, l1, l2, acc) and KL = acc / l1 + LSE2 - LSE1, never writing either
 * Nq x Nk matrix ("StreamKL", Methodology section 1; P1 is the fixed
 * distribution of its standard distillation setting). LSE1 and LSE2 are what
 * a backward would regenerate the distributions from (its section 2).
 *
 * Arguments
 *   q1, q2      device pointers, [B, Nq, H, d], element type `dtype`
 *   k1, k2      device pointers, [B, Nk, H, d], element type `dtype`
 *   kl          device pointer, [B, H, Nq] fp32 (written; natural log units)
 *   lse1, lse2  device pointers, [B, H, Nq] fp32 (written; natural log)
 *   B, H, Nq, Nk, d, causal, scale, stream, dtype  as for mha_fwd (one scale
 *               and one mask for both distributions)
 *
 * Ownership, execution and errors: as for mha_fwd (one kernel enqueued; the
 * library allocates nothing; kl, lse1 and lse2 must not overlap each other
 * or any input).
 */
MHA_API mha_status_t mha_kl_fwd(const void* q1, const void* k1, const void* q2,
                                const void* k2, float* kl, float* lse1, float* lse2, int B,
                                int H, int Nq, int Nk, int d, int causal, float scale,
                                void* stream, int dtype);

/*
 * mha_out_proj -- output projection after attention: Y = concat_heads(O) W^T
 * (+ bias).
 *
 * "SparkAttention", MHA-Forward passage (Eq. 1): the heads' outputs are
 * concatenated and multiplied by the output weight. O as written by mha_fwd,
 * [B, Nq, H, d], is already that concatenation when read as
 * [B*Nq, H*d], so no reshuffle is needed:
 *
 *     Y[t, e] = sum_{h, c} O[t, h, c] W[e, h*d + c]  (+ bias[e]),  t < B*Nq
 *
 * Arguments
 *   o      device pointer, [B, Nq, H, d], element type `dtype`, 16-byte aligned
 *   w      device pointer, [E, H*d] (one output feature per row),
 *          `dtype`, 16-byte aligned
 *   bias   device pointer, [E], `dtype`, 8-byte aligned; or NULL for none
 *   y      device pointer, [B, Nq, E], `dtype` (written; fp32 accumulation
 *          rounded to nearest even), 16-byte aligned
 *   B, Nq, H, d, E  sizes, >= 0; H*d at most 2^23 (32-bit offsets within
 *                   a 256-row tile) and B*Nq below 2^31 (else
 *                   MHA_ERR_INVALID_ARG); H*d a multiple of 64 and E of 4
 *                   (else MHA_ERR_UNSUPPORTED)
 *   stream, dtype   as for mha_fwd
 *
 * Ownership, execution and errors: as for mha_fwd (one kernel enqueued; the
 * library allocates nothing; y must not overlap o, w or bias). An empty
 * problem (B*Nq == 0 or E == 0) returns MHA_OK and enqueues nothing.
 */
MHA_API mha_status_t mha_out_proj(const void* o, const void* w, const void* bias, void* y,
                                  int B, int Nq, int H, int d, int E, void* stream, int dtype);

/*
 * mha_bwd -- attention backward: writes dQ, dK, dV and D.
 *
 * With P = exp(scale * Q K^T - LSE) (masked like the forward), regenerated
 * tile by tile from the forward's LSE ("StreamKL", Methodology section 2),
 * and D_i = sum_c dO_ic O_ic (the per-row term of the "SparkAttention"
 * backward passage, there called dPsum, written as rowsum(dO o O)):
 *
 *     dV = P^T dO,  dP = dO V^T,  dS = P o (dP - D),
 *     dQ = scale * dS K,  dK = scale * dS^T Q
 *
 * ("SparkAttention", backward passage: dV, dP, dS, dQ and dK per key block;
 * the FlashAttention long-sequence post, "Attention parallelism": backward
 * workers own blocks of keys). Keys no query sees (causal, key >= Nq) get
 * dK = dV = 0.
 *
 * Arguments
 *   q, o, dout  device pointers, [B, Nq, H, d], element type `dtype`: the
 *               forward's inputs Q and output O, and dL/dO
 *   k, v        device pointers, [B, Nk, H, d], element type `dtype`
 *   lse         device pointer, [B, H, Nq] fp32: the forward's LSE (natural log)
 *   dq          device pointer, [B, Nq, H, d], `dtype` (written)
 *   dk, dv      device pointers, [B, Nk, H, d], `dtype` (written)
 *   delta       device pointer, [B, H, Nq] fp32 (written: D, computed from
 *               the o and dout given; the dQ and dK/dV kernels read it)
 *   B, H, Nq, Nk, d, causal, scale, stream, dtype
 *               as for mha_fwd, and equal to the forward's
 * Each result element is the fp32 accumulation rounded to nearest even.
 *
 * Ownership and execution: as for mha_fwd. The library allocates nothing;
 * `delta` is the caller's buffer for the one intermediate the kernels share.
 * q, k, v, o, dout and lse are only read; dq, dk, dv and delta are
 * overwritten entirely. The call enqueues three kernels on `stream` (D, then
 * dQ, then dK/dV; only dK/dV when Nq == 0) and returns without
 * synchronising.
 *
 * Requirements checked before anything is enqueued (violations return
 * MHA_ERR_INVALID_ARG and write nothing): every pointer of a tensor with
 * elements non-null; element-type pointers 16-byte aligned, fp32 pointers
 * 4-byte aligned; dq, dk, dv and delta disjoint from each other and from
 * every input; Nk >= 1 when B*H*Nq > 0. B*H == 0 (or Nq == Nk == 0) returns
 * MHA_OK and enqueues nothing. Errors as for mha_fwd.
 */
MHA_API mha_status_t mha_bwd(const void* q, const void* k, const void* v, const void* o,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             float* delta, int B, int H, int Nq, int Nk, int d, int causal,
                             float scale, void* stream, int dtype);

/* Static, human-readable text for a status code (never NULL). */
MHA_API const char* mha_status_string(int status);

/* ABI version of this header; bumped on any incompatible change. */
#define MHA_ABI_VERSION 1
MHA_API int mha_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MHA_MI355X_H */
