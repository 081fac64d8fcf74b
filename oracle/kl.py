"""fp64 CPU oracle for the attention KL divergence ("StreamKL").

TEST INFRASTRUCTURE ONLY, like the rest of the oracle: only the tests and the
bench's cpu_baseline leg may import it; it shares no code with the HIP
kernels or their C-ABI library.

Two attention distributions over the same keys ("StreamKL", problem
statement: one attention distribution is trained to match another by
minimising their KL divergence), per batch b, head h and query row i:

    S1 = scale * Q1 K1^T,   S2 = scale * Q2 K2^T      (same causal mask)
    P_t = softmax_rows(S_t),  LSE_t = log sum_j exp(S_t,ij)
    KL_i = sum_j P1_ij (log P1_ij - log P2_ij)         (KL(P1 || P2))

with log P_t,ij = S_t,ij - LSE_t,i, so masked keys (P1 = 0) contribute
nothing and no log of an underflowed probability is taken (the page computes
its log ratios from logit differences and the LSEs for the same reason,
"StreamKL", section 3, numerical stability). P1 is the fixed distribution in
the page's standard distillation setting (its backward setting 1), hence the
direction KL(P1 || P2).

The page's online form (Methodology section 1) is the same quantity:
KL_i = acc_i / l1_i + LSE2_i - LSE1_i with acc_i = sum_j exp(S1_ij - m1_i)
(S1_ij - S2_ij); `kl_online_terms` evaluates those terms directly (all keys at
once, fp64) so a pin can check the identity.

Layouts: Q1, Q2 [B, Nq, H, d]; K1, K2 [B, Nk, H, d]; KL, LSE1, LSE2
[B, H, Nq]. Inputs float64; outputs float64, unrounded.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_probs, causal_visible, scores

__all__ = ["attention_kl", "kl_online_terms"]


def attention_kl(q1, k1, q2, k2, causal: bool, scale: float, rows=None):
    """(KL, LSE1, LSE2), each [B, H, n], for query ``rows`` (default all)."""
    q1, k1, q2, k2 = (np.asarray(x, np.float64) for x in (q1, k1, q2, k2))
    B, Nq, H, d = q1.shape
    if q2.shape != q1.shape or k1.shape[0] != B or k1.shape[2:] != (H, d) or k2.shape != k1.shape:
        raise ValueError("q1, k1, q2, k2 shapes disagree")
    Nk = k1.shape[1]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    KL = np.empty((B, H, len(rows)))
    L1 = np.empty((B, H, len(rows)))
    L2 = np.empty((B, H, len(rows)))
    vis = causal_visible(rows, Nk) if causal else np.ones((len(rows), Nk), bool)
    for b in range(B):
        for h in range(H):
            P1, lse1 = attention_probs(q1, k1, causal, scale, b, h, rows)
            _, lse2 = attention_probs(q2, k2, causal, scale, b, h, rows)
            S1 = scores(q1[b, rows, h, :], k1[b, :, h, :], scale)
            S2 = scores(q2[b, rows, h, :], k2[b, :, h, :], scale)
            log_ratio = np.where(vis, (S1 - lse1[:, None]) - (S2 - lse2[:, None]), 0.0)
            KL[b, h] = (P1 * log_ratio).sum(axis=1)
            L1[b, h] = lse1
            L2[b, h] = lse2
    return KL, L1, L2


def kl_online_terms(q1, k1, q2, k2, causal: bool, scale: float, b: int, h: int):
    """(m1, l1, m2, l2, acc) of the page's online form for one (b, h), every
    key at once: m_t the row max of S_t, l_t = sum_j exp(S_t - m_t) and
    acc = sum_j exp(S1 - m1) (S1 - S2) over the visible keys."""
    q1, k1, q2, k2 = (np.asarray(x, np.float64) for x in (q1, k1, q2, k2))
    Nq, Nk = q1.shape[1], k1.shape[1]
    S1 = scores(q1[b, :, h, :], k1[b, :, h, :], scale)
    S2 = scores(q2[b, :, h, :], k2[b, :, h, :], scale)
    vis = causal_visible(np.arange(Nq), Nk) if causal else np.ones((Nq, Nk), bool)
    S1m = np.where(vis, S1, -np.inf)
    S2m = np.where(vis, S2, -np.inf)
    m1, m2 = S1m.max(axis=1), S2m.max(axis=1)
    E1 = np.exp(S1m - m1[:, None])
    E2 = np.exp(S2m - m2[:, None])
    acc = (E1 * np.where(vis, S1 - S2, 0.0)).sum(axis=1)
    return m1, E1.sum(axis=1), m2, E2.sum(axis=1), acc
