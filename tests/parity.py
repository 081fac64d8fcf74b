"""Comparison of the HIP path's outputs with the fp64 oracle.

Bars (O in the fp16/bf16 I/O type, LSE in fp32), all against the unrounded
fp64 oracle, exactly as stated for the forward:
  * O: max-abs <= 1e-2 and mean-abs <= 1e-3;
  * LSE: max-abs <= 1e-3;
  * every O and LSE value finite.

The max-abs bar on O is flat. The only elements allowed above it are those
where the output format itself cannot come within 1e-2 of the exact value:
the element's rounding floor |nearest representable value - O_ref| exceeds
1e-2 (bf16 keeps 8 significant bits, so half an ulp is 2^-6 once |O| >= 4).
Such an element may be off by at most the largest floor among the compared
elements, i.e. the GPU must return the representable value nearest to the
exact one there. ``report`` states, per comparison, the max-abs error against
1e-2, the floor and where each occurs, and how many elements sit above the
gate (all of them at the format's floor when the comparison passes).
"""
from __future__ import annotations

import numpy as np

import workloads as wl

O_MAX_ABS = 1e-2
O_MEAN_ABS = 1e-3
LSE_MAX_ABS = 1e-3

# significant bits and smallest normal exponent of the 16-bit output formats
_FORMAT = {"bf16": (8, -126), "fp16": (11, -14)}


def rounding_floor(x: np.ndarray, dtype: str) -> np.ndarray:
    """|x - nearest value of the output format| per element, in fp64.

    With p significant bits, the spacing of the format at |x| in
    [2^e, 2^(e+1)) is 2^(e - p + 1) (2^(emin - p + 1) below the normal
    range); x is a fraction of that power of two away from a multiple of it.
    Computed directly from x (no double rounding through fp32)."""
    p, emin = _FORMAT[dtype]
    x = np.asarray(x, np.float64)
    _, e = np.frexp(np.abs(x))        # |x| = m * 2^e, m in [0.5, 1)
    expo = np.maximum(e - 1, emin)    # floor(log2 |x|), clamped at the subnormals
    u = np.ldexp(1.0, expo - p + 1)   # spacing of the format at |x|
    return np.abs(x - np.rint(x / u) * u)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half the spacing of the output format at |x| (the floor's upper bound)."""
    p, emin = _FORMAT[dtype]
    _, e = np.frexp(np.abs(np.asarray(x, np.float64)))
    return np.ldexp(1.0, np.maximum(e - 1, emin) - p)


def _at(flat_index: int, shape, rows):
    idx = list(np.unravel_index(int(flat_index), shape))
    if rows is not None and len(shape) == 4:
        idx[1] = int(np.asarray(rows)[idx[1]])
    return tuple(int(i) for i in idx)


def compare(o_bits: np.ndarray, lse: np.ndarray, O_ref: np.ndarray, L_ref: np.ndarray,
            dtype: str, rows=None) -> dict:
    """Error statistics of (o_bits, lse) against the oracle; arrays aligned.

    O arrays are [B, n, H, d] and LSE [B, H, n]; ``rows`` (optional) maps the
    n compared rows back to query indices for the reported positions, which
    are (b, row, h, c) for O and (b, h, row) for LSE."""
    O = wl.bits_to_f64(o_bits, dtype)
    O_ref = np.asarray(O_ref, np.float64)
    err = np.abs(O - O_ref)
    floor = rounding_floor(O_ref, dtype)
    lse = np.asarray(lse, np.float64)
    err_lse = np.abs(lse - L_ref)
    n = err.size
    st = dict(finite=bool(np.all(np.isfinite(O)) and np.all(np.isfinite(lse))), n=int(n))
    if n:
        i = int(np.nanargmax(err)) if np.isfinite(err).any() else 0
        j = int(np.argmax(floor))
        over = err > O_MAX_ABS
        st.update(
            o_max=float(err.max()), o_max_at=_at(i, err.shape, rows),
            o_mean=float(err.mean()),
            floor=float(floor[np.unravel_index(j, floor.shape)]), floor_at=_at(j, floor.shape, rows),
            o_n_over=int(over.sum()),
            # every element above the gate is one the format cannot bring
            # within 1e-2, and is no further off than the comparison's floor
            o_over_at_floor=bool(np.all(floor[over] > O_MAX_ABS)
                                 and np.all(err[over] <= floor.max())),
        )
    else:
        st.update(o_max=0.0, o_max_at=None, o_mean=0.0, floor=0.0, floor_at=None, o_n_over=0,
                  o_over_at_floor=True)
    if err_lse.size:
        k = int(np.nanargmax(err_lse)) if np.isfinite(err_lse).any() else 0
        kk = np.unravel_index(k, err_lse.shape)
        kat = tuple(int(t) for t in kk)
        if rows is not None and err_lse.ndim == 3:
            kat = (kat[0], kat[1], int(np.asarray(rows)[kat[2]]))
        st.update(lse_max=float(err_lse.max()), lse_max_at=kat)
    else:
        st.update(lse_max=0.0, lse_max_at=None)
    return st


def passes(st: dict) -> bool:
    return (st["finite"]
            and (st["o_max"] <= O_MAX_ABS or (st["o_n_over"] > 0 and st["o_over_at_floor"]))
            and st["o_mean"] <= O_MEAN_ABS and st["lse_max"] <= LSE_MAX_ABS)


def report(st: dict, label: str = "") -> str:
    """One line: max-abs against the flat gate, the floor and their positions."""
    over = ""
    if st["o_n_over"]:
        over = (f"; {st['o_n_over']} element(s) over 1e-2, "
                + ("all at the format's rounding floor" if st["o_over_at_floor"]
                   else "NOT explained by the rounding floor"))
    return (f"{label}: O max-abs {st['o_max']:.3e} vs 1e-2 at {st['o_max_at']} "
            f"(floor {st['floor']:.3e} at {st['floor_at']}{over}); "
            f"O mean-abs {st['o_mean']:.3e} vs 1e-3; LSE max-abs {st['lse_max']:.3e} vs 1e-3 "
            f"at {st['lse_max_at']}; finite {st['finite']}; {st['n']} elements")


def assert_parity(stats: dict, label: str = ""):
    msg = report(stats, label)
    assert stats["finite"], "non-finite output " + msg
    assert stats["o_max"] <= O_MAX_ABS or stats["o_over_at_floor"], "O max-abs " + msg
    assert stats["o_mean"] <= O_MEAN_ABS, "O mean-abs " + msg
    assert stats["lse_max"] <= LSE_MAX_ABS, "LSE max-abs " + msg
