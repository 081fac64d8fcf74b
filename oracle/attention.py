"""fp64 CPU oracle for the fused multi-head attention forward.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or run
this module: only the tests, the smoke check in ``__graft_entry__`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the HIP
kernels or their C-ABI library.

What it computes (per batch b and head h):

    S = scale * Q_bh K_bh^T                   (Nq x Nk, materialised)
    S[i, j] = -inf where j > i   (causal only; key j visible iff j <= i)
    m_i = max_j S_ij,  E = exp(S - m),  l_i = sum_j E_ij,  P = E / l
    O_bh = P V_bh
    LSE_i = m_i + ln(l_i)

Sources:
  * the attention formula softmax(Q K^T / sqrt(d_k)) V -- "CANN ops-transformer"
    article, section 1 (the MHA formula), and "SparkAttention", MHA-Forward
    passage (Eq. 1, per head, heads split the embedding);
  * the three materialising steps (S to memory, P to memory, O = P V) --
    "SparkAttention", the traditional MHA-Forward computation (its Section 2.3);
  * LSE = m + log l and P = exp(S - LSE) -- "StreamKL", Methodology §1 (online
    formulation, LSE_t = m_t + log l_t) and §2 (recomputation from the LSE);
  * the causal mask -- "SparkAttention", Transformer data-flow passage (Fig. 1):
    the masked decoder attention lets a token attend only to the tokens before
    it. Read inclusively (a token also sees itself), top-left aligned even when
    Nq != Nk.

Layouts (the pages fix only [S, H*D] per sequence, CANN article §1):
Q, O are [B, Nq, H, d]; K, V are [B, Nk, H, d]; LSE is [B, H, Nq]. Inputs are
float64 arrays (the caller widens the fp16/bf16 bits exactly); outputs stay
float64, unrounded.

Every function here is pinned by the ``-m "not gpu"`` tests against hand-worked
examples, closed forms, a library routine and a brute-force evaluator.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "scores",
    "causal_visible",
    "softmax_rows",
    "weighted_values",
    "log_sum_exp",
    "attention_probs",
    "attention_fwd",
    "attention_fwd_bruteforce",
]


def scores(q_bh: np.ndarray, k_bh: np.ndarray, scale: float) -> np.ndarray:
    """S = scale * Q K^T for one (b, h): q_bh [n, d], k_bh [Nk, d] -> [n, Nk].

    "CANN ops-transformer" §1 formula; "SparkAttention" first unfused step."""
    return float(scale) * (np.asarray(q_bh, np.float64) @ np.asarray(k_bh, np.float64).T)


def causal_visible(rows: np.ndarray, Nk: int) -> np.ndarray:
    """Boolean [len(rows), Nk]: key j visible to query row i iff j <= i.

    "SparkAttention", Fig. 1 passage (masked decoder attention), read
    inclusively and top-left aligned."""
    rows = np.asarray(rows)
    return np.arange(Nk)[None, :] <= rows[:, None]


def softmax_rows(S: np.ndarray):
    """Row softmax of a (possibly -inf masked) score matrix.

    Returns (P, m, l) with m the row max, l = sum_j exp(S_ij - m_i) and
    P = exp(S - m) / l. "SparkAttention" second unfused step; m and l are the
    two running scalars of "StreamKL" §1."""
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    l = E.sum(axis=1)
    P = E / l[:, None]
    return P, m, l


def weighted_values(P: np.ndarray, v_bh: np.ndarray) -> np.ndarray:
    """O = P V for one (b, h): P [n, Nk], v_bh [Nk, d] -> [n, d].

    "SparkAttention" third unfused step (read P and V, compute O)."""
    return P @ np.asarray(v_bh, np.float64)


def log_sum_exp(m: np.ndarray, l: np.ndarray) -> np.ndarray:
    """LSE = m + ln(l) with the natural log ("StreamKL" §1, LSE_t = m_t + log l_t)."""
    return m + np.log(l)


def attention_probs(q: np.ndarray, k: np.ndarray, causal: bool, scale: float,
                    b: int, h: int, rows: np.ndarray | None = None):
    """P and LSE for one (b, h) and a set of query rows (all rows by default)."""
    Nq, Nk = q.shape[1], k.shape[1]
    if rows is None:
        rows = np.arange(Nq)
    S = scores(q[b, rows, h, :], k[b, :, h, :], scale)
    if causal:
        S[~causal_visible(rows, Nk)] = -np.inf
    P, m, l = softmax_rows(S)
    return P, log_sum_exp(m, l)


def attention_fwd(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                  scale: float, rows: np.ndarray | None = None):
    """O [B, n, H, d] and LSE [B, H, n] (float64) for query ``rows``.

    ``rows`` defaults to every query row. Each row is computed from the plain
    definition; the subset only bounds memory (rows are independent, as the
    FlashAttention long-sequence post notes for its row-block workers)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, H, d = q.shape
    Bk, Nk, Hk, dk = k.shape
    if (Bk, Hk, dk) != (B, H, d) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    if rows is None:
        rows = np.arange(Nq)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((B, len(rows), H, d), np.float64)
    LSE = np.empty((B, H, len(rows)), np.float64)
    for b in range(B):
        for h in range(H):
            P, lse = attention_probs(q, k, causal, scale, b, h, rows)
            O[b, :, h, :] = weighted_values(P, v[b, :, h, :])
            LSE[b, h, :] = lse
    return O, LSE


def attention_fwd_bruteforce(q, k, v, causal: bool, scale: float):
    """Element-by-element evaluation for tiny shapes (pure Python, math.fsum).

    Reads the flat C-order buffers through the layout formula
    index(b, n, h, c) = ((b*N + n)*H + h)*d + c, so it checks the layout
    reading independently of NumPy's reshapes."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, H, d = q.shape
    Nk = k.shape[1]
    qf, kf, vf = q.ravel().tolist(), k.ravel().tolist(), v.ravel().tolist()

    def qi(b, n, h, c):
        return qf[((b * Nq + n) * H + h) * d + c]

    def ki(b, n, h, c):
        return kf[((b * Nk + n) * H + h) * d + c]

    def vi(b, n, h, c):
        return vf[((b * Nk + n) * H + h) * d + c]

    O = [0.0] * (B * Nq * H * d)
    LSE = [0.0] * (B * H * Nq)
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(Nk) if (not causal) or j <= i]
                s = {j: scale * math.fsum(qi(b, i, h, c) * ki(b, j, h, c) for c in range(d))
                     for j in keys}
                smax = max(s.values())
                w = {j: math.exp(s[j] - smax) for j in keys}
                den = math.fsum(w.values())
                for c in range(d):
                    num = math.fsum(w[j] * vi(b, j, h, c) for j in keys)
                    O[((b * Nq + i) * H + h) * d + c] = num / den
                LSE[(b * H + h) * Nq + i] = smax + math.log(den)
    return (np.array(O).reshape(B, Nq, H, d), np.array(LSE).reshape(B, H, Nq))
