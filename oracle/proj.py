"""fp64 CPU oracle for the output projection after attention (head concat,
then a linear map).

TEST INFRASTRUCTURE ONLY, like the rest of the oracle: only the tests and the
bench's cpu_baseline leg may import it; it shares no code with the HIP
kernels or their C-ABI library.

"SparkAttention" (MHA-Forward passage, Eq. 1): the heads' outputs are
concatenated and multiplied by an output weight matrix W_O. With the
attention output O laid out [B, Nq, H, d], the concatenation of a token's
heads is its row of O seen as [B*Nq, H*d], so

    Y[t, e] = sum_{h, c} O[t, h, c] * W[e, h*d + c]  (+ bias[e])

with W stored [E, H*d] (one output feature per row, the usual linear-layer
layout). `out_proj` is that definition with a matrix product as its step;
`out_proj_by_heads` writes the same map as a sum of per-head products
(sum_h O_h W_h^T), which a pin compares against it.
"""
from __future__ import annotations

import numpy as np

__all__ = ["out_proj", "out_proj_by_heads", "out_proj_bruteforce"]


def out_proj(o, w, bias=None):
    """Y [B, Nq, E] = concat_heads(O) W^T (+ bias), float64."""
    o = np.asarray(o, np.float64)
    w = np.asarray(w, np.float64)
    B, Nq, H, d = o.shape
    if w.shape[1] != H * d:
        raise ValueError("W must be [E, H*d]")
    y = o.reshape(B * Nq, H * d) @ w.T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)[None, :]
    return y.reshape(B, Nq, w.shape[0])


def out_proj_by_heads(o, w, bias=None):
    """The same map as a sum over heads of O_h W_h^T, W_h = W[:, h*d:(h+1)*d]."""
    o = np.asarray(o, np.float64)
    w = np.asarray(w, np.float64)
    B, Nq, H, d = o.shape
    y = np.zeros((B, Nq, w.shape[0]))
    for h in range(H):
        y += o[:, :, h, :] @ w[:, h * d:(h + 1) * d].T
    if bias is not None:
        y = y + np.asarray(bias, np.float64)
    return y


def out_proj_bruteforce(o, w, bias=None):
    """Element by element (pure Python, math.fsum) for tiny shapes."""
    import math
    o = np.asarray(o, np.float64)
    w = np.asarray(w, np.float64)
    B, Nq, H, d = o.shape
    E = w.shape[0]
    y = np.empty((B, Nq, E))
    for b in range(B):
        for t in range(Nq):
            for e in range(E):
                terms = [o[b, t, h, c] * w[e, h * d + c] for h in range(H) for c in range(d)]
                if bias is not None:
                    terms.append(float(bias[e]))
                y[b, t, e] = math.fsum(terms)
    return y
