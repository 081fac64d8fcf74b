"""Comparison of the HIP path's outputs with the fp64 oracle.

Bars (O in the fp16/bf16 I/O type, LSE in fp32), all against the unrounded
fp64 oracle:
  * O: max-abs <= 1e-2 and mean-abs <= 1e-3. The max-abs bar is applied per
    element as |O_gpu - O_ref| <= max(1e-2, half an output ulp at O_ref + 1e-3):
    it is exactly 1e-2 wherever the output format can represent a value within
    1e-2 of the exact one, and only widens where it cannot -- rounding the exact
    result to bf16 is itself more than 1e-2 off once |O| >= 4 (half a bf16 ulp
    is 2^-6 there), which happens for one element of the masked decoder
    workload.
  * LSE: max-abs <= 1e-3.
  * Every O and LSE value finite.
"""
from __future__ import annotations

import numpy as np

import workloads as wl

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output format at |x|."""
    ax = np.abs(np.asarray(x, np.float64))
    _, e = np.frexp(ax)  # ax = m * 2^e, m in [0.5, 1)
    expo = e - 1        # floor(log2 |x|)
    if dtype == "bf16":
        expo = np.maximum(expo, -126)
        return np.ldexp(1.0, expo - 8)
    expo = np.maximum(expo, -14)
    return np.ldexp(1.0, expo - 11)


def compare(o_bits: np.ndarray, lse: np.ndarray, O_ref: np.ndarray, L_ref: np.ndarray,
            dtype: str) -> dict:
    """Error statistics of (o_bits, lse) against the oracle; all arrays aligned."""
    O = wl.bits_to_f64(o_bits, dtype)
    err = np.abs(O - O_ref)
    allowed = np.maximum(O_MAX_ABS, half_ulp(O_ref, dtype) + 1e-3)
    lse = np.asarray(lse, np.float64)
    err_lse = np.abs(lse - L_ref)
    n = err.size
    return dict(
        finite=bool(np.all(np.isfinite(O)) and np.all(np.isfinite(lse))),
        o_max=float(err.max()) if n else 0.0,
        o_mean=float(err.mean()) if n else 0.0,
        o_excess=float((err - allowed).max()) if n else -1.0,
        o_n_over_1e2=int((err > O_MAX_ABS).sum()),
        lse_max=float(err_lse.max()) if err_lse.size else 0.0,
    )


def assert_parity(stats: dict, label: str = ""):
    msg = f"{label}: {stats}"
    assert stats["finite"], "non-finite output " + msg
    assert stats["o_excess"] <= 0.0, "O max-abs " + msg
    assert stats["o_mean"] <= O_MEAN_ABS, "O mean-abs " + msg
    assert stats["lse_max"] <= LSE_MAX_ABS, "LSE max-abs " + msg
