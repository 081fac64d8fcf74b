"""The backward's parity bar, checked on the CPU before any kernel runs.

tests/parity_bwd.py derives a per-element bound (and an RMS bar) for a
backward that rounds where the HIP kernels round. Here a float32 NumPy model
of exactly those rounding points -- P and dS rounded to the 16-bit type as
MFMA operands, fp32 sums, 16-bit outputs -- must pass the bar (the bound is
not too tight), and the same model with a planted mistake of the kind a
kernel can make must fail it (the bound is not too loose). The model is test
code only; it shares nothing with the HIP kernels and is not the oracle.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import workloads as wl
from parity_bwd import assert_bwd_parity, compare_head, head_reference, merge_stats

LOG2E = 1.4426950408889634


def _rt(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 to the 16-bit type and back (exact widening)."""
    return wl.bits_to_f32(wl.round_bits(x32, dtype), dtype)


def model_head(q, k, v, do, o_in, l_in, causal, scale, dtype, mistake=None):
    """fp32 model of one head's backward; all arrays float32, returns float64."""
    f32 = np.float32
    Nq, Nk = q.shape[0], k.shape[0]
    c = f32(f32(scale) * f32(LOG2E))
    s = q @ k.T
    arg = s * c - (l_in * f32(LOG2E))[:, None]
    P = np.exp2(arg).astype(f32)
    vis = np.ones((Nq, Nk), bool)
    if causal:
        vis = np.arange(Nk)[None, :] <= np.arange(Nq)[:, None]
    if mistake == "drop last key":
        vis[:, Nk - 1] = False
    P = np.where(vis, P, f32(0))
    D = (do * o_in).sum(1, dtype=f32)
    if mistake == "no row term":
        D[:] = 0
    dP = do @ v.T
    dS = P * (dP - D[:, None])
    if mistake == "sign of dS":
        dS = -dS
    Pr, dSr = _rt(P, dtype), _rt(dS, dtype)
    if mistake == "P unrounded as bf16 of P^2":
        Pr = _rt(P * P, dtype)
    dv = Pr.T @ do
    dq = f32(scale) * (dSr @ k)
    dk = f32(scale) * (dSr.T @ q)
    if mistake == "dK scaled twice":
        dk = f32(scale) * dk
    if mistake == "dQ rows shifted":
        dq = np.roll(dq, 1, axis=0)
    return {g: _rt(x, dtype).astype(np.float64) for g, x in (("dq", dq), ("dk", dk), ("dv", dv))} | {
        "D": D.astype(np.float64)}


def run_case(B, H, Nq, Nk, d, dtype, causal, seed, mistake=None, std=1.0):
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed, std=std)
    gb = wl.random_grad(B, H, Nq, d, dtype, seed + 1000)
    q, k, v, do = (wl.bits_to_f64(x, dtype) for x in (qb, kb, vb, gb))
    scale = float(np.float32(1 / math.sqrt(d)))
    O, L = oracle.attention_fwd(q, k, v, causal, scale)
    o_in = wl.bits_to_f64(wl.round_bits(O.astype(np.float32), dtype), dtype)
    l_in = L.astype(np.float32).astype(np.float64)
    stats = []
    for b in range(B):
        for h in range(H):
            ref = head_reference(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], o_in[b, :, h],
                                 l_in[b, h], causal, scale, dtype)
            got = model_head(*(x.astype(np.float32) for x in (
                q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], o_in[b, :, h], l_in[b, h])),
                causal, scale, dtype, mistake)
            stats.append(compare_head(ref, got))
    return merge_stats(stats)


CASES = [
    (1, 2, 77, 131, 64, "bf16", False, 1),
    (1, 2, 131, 77, 128, "bf16", True, 2),
    (2, 1, 200, 200, 64, "fp16", True, 3),
    (1, 1, 1, 300, 128, "fp16", False, 4),
    (1, 1, 600, 600, 128, "bf16", True, 5),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "q{}k{}d{}{}{}".format(
    c[2], c[3], c[4], c[5], "c" if c[6] else ""))
def test_rounding_model_passes(case):
    st = run_case(*case)
    assert_bwd_parity(st, case[5], str(case))
    # the bound is not vacuous: the model's worst element uses a visible part of it
    assert max(st[g]["worst_ratio"] for g in ("dq", "dk", "dv")) > 1e-3


def test_rounding_model_passes_peaky_scores():
    st = run_case(1, 2, 96, 96, 64, "bf16", True, 9, std=2.0)
    assert_bwd_parity(st, "bf16", "peaky")


MISTAKES = ["drop last key", "no row term", "sign of dS", "P unrounded as bf16 of P^2",
            "dK scaled twice", "dQ rows shifted"]


@pytest.mark.parametrize("mistake", MISTAKES)
def test_planted_kernel_mistakes_fail(mistake):
    st = run_case(1, 2, 131, 77, 64, "bf16", False, 7, mistake=mistake)
    with pytest.raises(AssertionError):
        assert_bwd_parity(st, "bf16", mistake)
