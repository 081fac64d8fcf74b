"""Reference gradients and per-element error bounds for the attention backward.

The reference values are the fp64 oracle's (oracle.backward's steps, applied
per (batch, head) and per block of query rows). The bar is a per-element
bound derived from the arithmetic of a backward that, like the HIP kernels,

  * recomputes S = Q K^T and dP = dO V^T with fp32 accumulation of exact
    products of the 16-bit inputs (at most d terms),
  * forms P = exp2(S * scale*log2(e) - LSE*log2(e)) in fp32 from the LSE it is
    given, and D_i = sum_c dO_ic O_ic in fp32 from the O it is given,
  * rounds P and dS = P (dP - D) to the 16-bit I/O type as MFMA operands,
  * accumulates dV = P^T dO, dQ = dS K and dK = dS^T Q in fp32 (at most
    Nq or Nk terms), scales dQ and dK by the fp32 scale, and rounds every
    output to the I/O type (round to nearest even).

With u the unit roundoff of the I/O type (2^-8 bf16, 2^-11 fp16), a its
absolute floor (half the smallest subnormal step: 2^-25 for fp16, nothing
for bf16) and g_n = n * 2^-24 the worst-case relative error of an fp32 sum of
n terms, each inexact step contributes its standard first-order bound:

  dS_r:  E_ij = u|dS_ij| + a + (1+u) [ e_ij P_ij (|dP_ij - D_i| + dd_ij + dD_i)
                                        + P_ij (dd_ij + dD_i) + 2^-23 |dS_ij| ]
  dV:    u|dV| + a + (1+u) [ ((u + (1+u) e + g_Nq) o P)^T |dO| + a sum_i |dO_i| ]
  dQ:    u|dQ| + a + (1+u) scale [ E |K| + g_Nk |dS| |K| ] + 2^-24 |dQ|
  dK:    u|dK| + a + (1+u) scale [ E^T |Q| + g_Nq |dS|^T |Q| ] + 2^-24 |dK|
  D:     dD_i = sum_c |dO_ic| |O_in,ic - O_ic| + g_d sum_c |dO_ic O_in,ic| + 2^-24 |D_i|

where e_ij bounds the relative error of P (the LSE it was given, off by
dL_i = |LSE_in,i - LSE_i|; the fp32 score sum, off by ds_ij = g_d (|Q||K|^T)_ij
in raw units; fp32 rounding of the exponent's terms; one ulp of exp2):
e_ij = 1.01 (scale ds_ij + dL_i) + 2^-22 (2 + |S_ij| + |LSE_i|) with S the
scaled score, and
dd_ij = g_d (|dO||V|^T)_ij bounds the fp32 error of dP. Second-order terms
are covered by a 25% margin (BOUND_MARGIN). The input deviations |O_in - O|
and |LSE_in - LSE| are those of the inputs the test hands the kernel; with
the oracle's own O and LSE rounded to the I/O type and fp32 they are known
exactly here.

A statistical bar sits beside it: the RMS of the error over a tensor stays
below 4u times the RMS of the reference. Independent roundings of the two
operands of every product and of the output give an expected RMS error near
u/sqrt(3) * sqrt(2) ~ 0.8u of the reference's RMS, so 4u leaves a margin of
five while a systematic slip (a dropped term, a wrong row term) of a percent
of the signal fails it. Where the reference is identically zero (one key:
P = 1 and dS = 0 exactly) there is no signal to be relative to, and the
element bound alone applies.
"""
from __future__ import annotations

import numpy as np

import oracle
import oracle.backward as ob

BOUND_MARGIN = 1.25
RMS_FACTOR = 4.0
CHUNK_ROWS = 1024


def unit_roundoff(dtype: str) -> tuple[float, float]:
    """(u, a): unit roundoff and absolute floor of the 16-bit I/O type."""
    if dtype == "bf16":
        return 2.0 ** -8, 0.0
    if dtype == "fp16":
        return 2.0 ** -11, 2.0 ** -25
    raise ValueError(dtype)


def head_reference(qh, kh, vh, doh, oh_in, lh_in, causal: bool, scale: float, dtype: str,
                   rows=None, cols=None) -> dict:
    """Reference values and bounds for one (batch, head).

    qh, doh, oh_in: [Nq, d]; kh, vh: [Nk, d]; lh_in: [Nq] (all float64: the
    exact values of what the kernel is given). ``rows`` selects the query rows
    whose dQ and D are checked, ``cols`` the keys whose dK and dV are
    checked (default: all). Every query row still enters dK and dV.
    """
    u, a = unit_roundoff(dtype)
    Nq, d = qh.shape
    Nk = kh.shape[0]
    rows = np.arange(Nq) if rows is None else np.asarray(rows, np.int64)
    cols = np.arange(Nk) if cols is None else np.asarray(cols, np.int64)
    row_pos = {int(r): n for n, r in enumerate(rows)}
    g_d, g_q, g_k = d * 2.0 ** -24, Nq * 2.0 ** -24, Nk * 2.0 ** -24
    aK, aQ, aV, adO = np.abs(kh), np.abs(qh), np.abs(vh), np.abs(doh)

    out = {k: np.zeros((len(rows), d)) for k in ("dq", "dq_bound")}
    out.update({k: np.zeros((len(cols), d)) for k in ("dk", "dk_bound", "dv", "dv_bound")})
    out.update({k: np.zeros(len(rows)) for k in ("D", "D_bound")})
    for r0 in range(0, Nq, CHUNK_ROWS):
        rc = np.arange(r0, min(Nq, r0 + CHUNK_ROWS))
        # causal: keys past the block's last row have P = 0 and dS = 0 exactly
        # (in the kernel too), so they are left out
        nk = min(Nk, int(rc[-1]) + 1) if causal else Nk
        kc, vc, aKc, aVc = kh[:nk], vh[:nk], aK[:nk], aV[:nk]
        # the oracle's forward and backward steps for these rows
        P, lse = oracle.attention_probs(qh[None, :, None, :], kc[None, :, None, :], causal, scale,
                                        0, 0, rc)
        O = oracle.weighted_values(P, vc)
        dP = ob.grad_p(doh[rc], vc)
        dS, D = ob.softmax_grad(P, dP)
        # input deviations of the rows
        dL = np.abs(lh_in[rc] - lse)
        dD = ((adO[rc] * np.abs(oh_in[rc] - O)).sum(1)
              + g_d * np.abs(doh[rc] * oh_in[rc]).sum(1) + 2.0 ** -24 * np.abs(D))

        def terms(ri, cj):
            """e and E on the block (rows rc[ri], keys cj)."""
            r = rc[ri]
            Pb, dPb, dSb = P[np.ix_(ri, cj)], dP[np.ix_(ri, cj)], dS[np.ix_(ri, cj)]
            Sb = np.abs(oracle.scores(qh[r], kc[cj], scale))
            ds = g_d * (aQ[r] @ aKc[cj].T)
            dd = g_d * (adO[r] @ aVc[cj].T)
            Db, dDb = D[ri][:, None], dD[ri][:, None]
            e = 1.01 * (scale * ds + dL[ri][:, None]) + 2.0 ** -22 * (2 + Sb + np.abs(lse[ri])[:, None])
            E = (u * np.abs(dSb) + a + (1 + u) * (e * Pb * (np.abs(dPb - Db) + dd + dDb)
                                                  + Pb * (dd + dDb) + 2.0 ** -23 * np.abs(dSb)))
            return e, E

        all_rows = np.arange(len(rc))
        # keys: dV, dK over this block of rows
        ci = np.nonzero(cols < nk)[0]
        cc = cols[ci]
        ec, Ec = terms(all_rows, cc)
        Pc, dSc = P[:, cc], dS[:, cc]
        out["dv"][ci] += ob.grad_v(Pc, doh[rc])
        out["dk"][ci] += ob.grad_k(dSc, qh[rc], scale)
        out["dv_bound"][ci] += ((u + (1 + u) * ec + g_q) * Pc).T @ adO[rc]
        out["dv_bound"] += a * adO[rc].sum(0)
        out["dk_bound"][ci] += scale * (Ec.T @ aQ[rc] + g_q * np.abs(dSc).T @ aQ[rc])
        # rows: dQ and D of the selected rows in this block
        sel = np.array([n for n, r in enumerate(rc) if int(r) in row_pos], np.int64)
        if len(sel):
            pos = [row_pos[int(rc[n])] for n in sel]
            if len(cc) == nk and np.array_equal(cc, np.arange(nk)):
                Er = Ec[sel]
            else:
                Er = terms(sel, np.arange(nk))[1]
            out["dq"][pos] = ob.grad_q(dS[sel], kc, scale)
            out["dq_bound"][pos] = scale * (Er @ aKc + g_k * np.abs(dS[sel]) @ aKc)
            out["D"][pos] = D[sel]
            out["D_bound"][pos] = dD[sel]
    for g in ("dq", "dk"):
        out[g + "_bound"] = (u * np.abs(out[g]) + a + (1 + u) * out[g + "_bound"]
                             + 2.0 ** -24 * np.abs(out[g]))
    out["dv_bound"] = u * np.abs(out["dv"]) + a + (1 + u) * out["dv_bound"]
    return out


def compare_head(ref: dict, got: dict) -> dict:
    """Error statistics of one head's kernel results against ``ref``.

    ``got`` holds dq [len(rows), d], dk and dv [len(cols), d] and D [len(rows)]
    as float64 (the exact values of the kernel's outputs)."""
    st = {}
    for g in ("dq", "dk", "dv", "D"):
        err = np.abs(got[g] - ref[g])
        bound = BOUND_MARGIN * ref[g + "_bound"]
        st[g] = dict(
            finite=bool(np.all(np.isfinite(got[g]))),
            max_err=float(err.max()) if err.size else 0.0,
            worst_ratio=float((err / np.maximum(bound, 1e-300)).max()) if err.size else 0.0,
            rms_err=float(np.sqrt((err ** 2).mean())) if err.size else 0.0,
            rms_ref=float(np.sqrt((ref[g] ** 2).mean())) if err.size else 0.0,
        )
    return st


def merge_stats(stats: list[dict]) -> dict:
    """Combine per-head statistics (max of maxima, RMS over heads)."""
    out = {}
    for g in ("dq", "dk", "dv", "D"):
        s = [x[g] for x in stats]
        out[g] = dict(
            finite=all(x["finite"] for x in s),
            max_err=max(x["max_err"] for x in s),
            worst_ratio=max(x["worst_ratio"] for x in s),
            rms_err=float(np.sqrt(np.mean([x["rms_err"] ** 2 for x in s]))),
            rms_ref=float(np.sqrt(np.mean([x["rms_ref"] ** 2 for x in s]))),
        )
    return out


def assert_bwd_parity(st: dict, dtype: str, label: str = ""):
    u, _ = unit_roundoff(dtype)
    for g in ("dq", "dk", "dv", "D"):
        s = st[g]
        msg = f"{label} {g}: {s}"
        assert s["finite"], "non-finite " + msg
        assert s["worst_ratio"] <= 1.0, "element bound " + msg
        if g != "D" and s["rms_ref"] > 0.0:
            assert s["rms_err"] <= RMS_FACTOR * u * s["rms_ref"], "RMS bar " + msg
