"""fp64 CPU oracle for the split-over-keys forward and its merge.

TEST INFRASTRUCTURE ONLY, like the rest of the oracle: only the tests may
import it; it shares no code with the HIP kernels or their C-ABI library.

"StreamKL" (Methodology section 3) splits the keys of a row over several
workers when there are few query rows (decoding) and merges their partial
results; the merge rests on the LSE of the online formulation (its
section 1: LSE = m + log l, P = exp(S - LSE)). For a partition of the keys
into blocks K_1 .. K_n and one query row:

    O_s   = softmax over the visible keys of K_s, applied to their V rows
    LSE_s = log sum_{j in K_s, visible} exp(S_j)     (-inf if none visible)
    LSE   = log sum_s exp(LSE_s)
    O     = sum_s exp(LSE_s - LSE) O_s

which equals the softmax over all keys (the definition in attention.py):
exp(LSE_s - LSE) is the share of block s in the row's normaliser. The page
prints neither formula; this is the plainest reading of "merge the partial
results by their LSE".

Pinned by the ``-m "not gpu"`` tests against the unsplit oracle (any
partition, causal and not), a one-block partition, blocks with no visible
key, and planted mistakes.
"""
from __future__ import annotations

import numpy as np

from .attention import attention_probs, log_sum_exp, scores, softmax_rows, weighted_values

__all__ = ["split_partials", "merge_splits", "attention_fwd_split"]


def split_partials(q, k, v, causal: bool, scale: float, bounds):
    """Per-block (O_s [n, B, Nq, H, d], LSE_s [n, B, H, Nq]) for key blocks
    [bounds[s], bounds[s+1]). A query row with no visible key in a block gets
    O_s = 0 and LSE_s = -inf."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Nq, H, d = q.shape
    n = len(bounds) - 1
    O = np.zeros((n, B, Nq, H, d))
    L = np.full((n, B, H, Nq), -np.inf)
    rows = np.arange(Nq)
    for s in range(n):
        a, e = int(bounds[s]), int(bounds[s + 1])
        if e <= a:
            continue
        # rows that see at least one key of the block: all, or i >= a (causal)
        seen = rows[rows >= a] if causal else rows
        if len(seen) == 0:
            continue
        for b in range(B):
            for h in range(H):
                # scores against keys a..e-1 only
                kb = k[:, a:e]
                vb = v[:, a:e]
                if causal:
                    P, lse = _causal_block(q, kb, scale, b, h, seen, a)
                else:
                    P, lse = attention_probs(q, kb, False, scale, b, h, seen)
                O[s, b, seen, h, :] = weighted_values(P, vb[b, :, h, :])
                L[s, b, h, seen] = lse
    return O, L


def _causal_block(q, kb, scale, b, h, rows, a):
    """P and LSE of ``rows`` against a key block starting at key a, causal:
    key a + t is visible to row i iff a + t <= i."""
    S = scores(q[b, rows, h, :], kb[b, :, h, :], scale)
    visible = (a + np.arange(kb.shape[1]))[None, :] <= rows[:, None]
    S[~visible] = -np.inf
    P, m, l = softmax_rows(S)
    return P, log_sum_exp(m, l)


def merge_splits(O_parts, LSE_parts):
    """Merge per-block partial results: (O [B, Nq, H, d], LSE [B, H, Nq])."""
    O_parts = np.asarray(O_parts, np.float64)
    LSE_parts = np.asarray(LSE_parts, np.float64)
    M = LSE_parts.max(axis=0)                      # [B, H, Nq]
    w = np.exp(LSE_parts - M[None])                # exp(-inf) = 0 for empty blocks
    total = w.sum(axis=0)
    LSE = M + np.log(total)
    share = w / total[None]                        # exp(LSE_s - LSE)
    # share is [n, B, H, Nq]; O_parts is [n, B, Nq, H, d]
    O = np.einsum("sbhn,sbnhc->bnhc", share, O_parts)
    return O, LSE


def attention_fwd_split(q, k, v, causal: bool, scale: float, bounds):
    """The forward computed block by block and merged (O, LSE)."""
    O_parts, L_parts = split_partials(q, k, v, causal, scale, bounds)
    return merge_splits(O_parts, L_parts)
