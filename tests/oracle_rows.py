"""The fp64 oracle over many query rows, in row chunks that bound its memory.

Rows are independent (each query row's softmax and output depend only on
that row's scores), so evaluating the oracle on row chunks and concatenating
is the same computation; the chunk only caps the size of the materialised
score matrix (chunk x Nk per head)."""
from __future__ import annotations

import numpy as np

import oracle


def attention_fwd_rows(q, k, v, causal: bool, scale: float, rows=None, chunk: int = 2048):
    """oracle.attention_fwd over ``rows`` (default: all), ``chunk`` rows per call."""
    Nq = q.shape[1]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    Os, Ls = [], []
    for r0 in range(0, len(rows), chunk):
        O, L = oracle.attention_fwd(q, k, v, causal, scale, rows=rows[r0:r0 + chunk])
        Os.append(O)
        Ls.append(L)
    if not Os:
        B, _, H, d = q.shape
        return np.empty((B, 0, H, d)), np.empty((B, H, 0))
    return np.concatenate(Os, axis=1), np.concatenate(Ls, axis=2)
