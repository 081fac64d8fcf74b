"""fp64 CPU oracle for the attention backward (gradients of the forward).

TEST INFRASTRUCTURE ONLY, like the forward oracle: only the tests may import
it; it shares no code with the HIP kernels or their C-ABI library.

The pages describe a fused backward that recomputes the forward tile by tile
from the stored LSE ("StreamKL", Methodology §2: P = exp(S - LSE)), uses a
per-row term they call dPsum to form dS ("SparkAttention", backward passage
and its Eq. 4, whose body the page does not print), accumulates dK and dV per
key block and adds dQ across blocks ("SparkAttention" backward passage; the
FlashAttention long-sequence post, "Attention parallelism"). None of them
prints the gradient formulas, so this oracle is the plain definition: the
derivative of the forward

    S = scale * Q K^T (masked: -inf where key j > query i when causal)
    P = softmax_rows(S),   O = P V

for a loss whose gradient with respect to O is dO. With everything
materialised, per (batch, head):

    dV = P^T dO                      (O is linear in V)
    dP = dO V^T                      (gradient with respect to P)
    D_i = sum_j P_ij dP_ij           (the row term; equals sum_c dO_ic O_ic)
    dS = P o (dP - D)                (softmax Jacobian applied row by row)
    dQ = scale * dS K,   dK = scale * dS^T Q

D is what the SparkAttention page calls dPsum (read as this row sum; the page
does not print it). Masked entries have P = 0, so they contribute nothing.

Layouts as in the forward oracle: Q, dO, dQ [B, Nq, H, d]; K, V, dK, dV
[B, Nk, H, d]; D [B, H, Nq]. Inputs are float64 arrays; outputs stay float64.

Pinned by the ``-m "not gpu"`` tests against central finite differences of the
(separately pinned) forward oracle, PyTorch CPU float64 autograd through its
scaled-dot-product attention, closed forms and a hand-worked example.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_probs

__all__ = [
    "grad_v",
    "grad_p",
    "softmax_grad",
    "grad_q",
    "grad_k",
    "attention_bwd",
]


def grad_v(P: np.ndarray, do_bh: np.ndarray) -> np.ndarray:
    """dV = P^T dO for one (b, h): P [n, Nk], dO [n, d] -> [Nk, d]."""
    return P.T @ np.asarray(do_bh, np.float64)


def grad_p(do_bh: np.ndarray, v_bh: np.ndarray) -> np.ndarray:
    """dP = dO V^T for one (b, h): dO [n, d], V [Nk, d] -> [n, Nk]."""
    return np.asarray(do_bh, np.float64) @ np.asarray(v_bh, np.float64).T


def softmax_grad(P: np.ndarray, dP: np.ndarray):
    """(dS, D): dS = P o (dP - D) with D_i = sum_j P_ij dP_ij, row by row.

    The derivative of a row softmax: dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik).
    D is the per-row term of the SparkAttention backward ("dPsum")."""
    D = (P * dP).sum(axis=1)
    return P * (dP - D[:, None]), D


def grad_q(dS: np.ndarray, k_bh: np.ndarray, scale: float) -> np.ndarray:
    """dQ = scale * dS K for one (b, h): dS [n, Nk], K [Nk, d] -> [n, d]."""
    return float(scale) * (dS @ np.asarray(k_bh, np.float64))


def grad_k(dS: np.ndarray, q_bh: np.ndarray, scale: float) -> np.ndarray:
    """dK = scale * dS^T Q for one (b, h): dS [n, Nk], Q [n, d] -> [Nk, d]."""
    return float(scale) * (dS.T @ np.asarray(q_bh, np.float64))


def attention_bwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                  causal: bool, scale: float):
    """(dQ, dK, dV, D) in float64 for the whole problem.

    Every query row is used (dK and dV sum over all of them)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    B, Nq, H, d = q.shape
    if k.shape[0] != B or k.shape[2:] != (H, d) or v.shape != k.shape or do.shape != q.shape:
        raise ValueError("q, k, v, do shapes disagree")
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    D = np.empty((B, H, Nq), np.float64)
    for b in range(B):
        for h in range(H):
            P, _ = attention_probs(q, k, causal, scale, b, h)
            dv[b, :, h, :] = grad_v(P, do[b, :, h, :])
            dP = grad_p(do[b, :, h, :], v[b, :, h, :])
            dS, D[b, h, :] = softmax_grad(P, dP)
            dq[b, :, h, :] = grad_q(dS, k[b, :, h, :], scale)
            dk[b, :, h, :] = grad_k(dS, q[b, :, h, :], scale)
    return dq, dk, dv, D
