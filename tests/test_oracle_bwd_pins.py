"""Pins of the fp64 backward oracle (CPU only).

The backward oracle (oracle/backward.py) is checked against things other
than itself:
  * central finite differences of the forward oracle (itself pinned in
    test_oracle_pins.py): d(sum dO o O)/dX for X in {Q, K, V};
  * PyTorch CPU float64 autograd through scaled_dot_product_attention;
  * closed forms: V constant over the keys gives dQ = dK = 0; Q = 0 gives
    uniform P and dV_j = sum over the rows that see key j of dO_i / |row i|;
  * the identity D_i = sum_c dO_ic O_ic;
  * a hand-worked example (tests/golden/bwd_worked_example.json).
Each planted mistake in a backward step fails at least one of them.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.backward as ob

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "bwd_worked_example.json")


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * std


def _problem(seed, B=1, H=2, Nq=5, Nk=6, d=4):
    q = _rand((B, Nq, H, d), seed)
    k = _rand((B, Nk, H, d), seed + 1)
    v = _rand((B, Nk, H, d), seed + 2)
    do = _rand((B, Nq, H, d), seed + 3)
    return q, k, v, do


def _loss(q, k, v, do, causal, scale):
    O, _ = oracle.attention_fwd(q, k, v, causal, scale)
    return float((O * do).sum())


def _fd_grad(q, k, v, do, causal, scale, which, eps=1e-5):
    """Central finite differences of sum(dO o O) with respect to one input."""
    args = [q.copy(), k.copy(), v.copy()]
    x = args[which]
    g = np.empty_like(x)
    for idx in np.ndindex(x.shape):
        old = x[idx]
        x[idx] = old + eps
        lp = _loss(*args, do, causal, scale)
        x[idx] = old - eps
        lm = _loss(*args, do, causal, scale)
        x[idx] = old
        g[idx] = (lp - lm) / (2 * eps)
    return g


def pin_finite_differences():
    ok = True
    for causal, (Nq, Nk) in ((False, (5, 6)), (True, (6, 6)), (True, (7, 4)), (False, (3, 8))):
        q, k, v, do = _problem(11 + Nq + Nk, Nq=Nq, Nk=Nk)
        dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, causal, 0.7)
        for which, g in ((0, dq), (1, dk), (2, dv)):
            ref = _fd_grad(q, k, v, do, causal, 0.7, which)
            ok &= bool(np.allclose(g, ref, rtol=1e-6, atol=1e-8))
    return ok


def pin_torch_autograd():
    torch = pytest.importorskip("torch")
    ok = True
    for causal in (False, True):
        q, k, v, do = _problem(5, B=2, H=3, Nq=7, Nk=7, d=8)
        dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, causal, 0.3)
        tq, tk, tv = (torch.tensor(x.transpose(0, 2, 1, 3), dtype=torch.float64, requires_grad=True)
                      for x in (q, k, v))
        out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=0.3)
        out.backward(torch.tensor(do.transpose(0, 2, 1, 3), dtype=torch.float64))
        for g, t in ((dq, tq), (dk, tk), (dv, tv)):
            ok &= bool(np.allclose(g, t.grad.numpy().transpose(0, 2, 1, 3), rtol=1e-10, atol=1e-12))
    return ok


def pin_constant_v():
    """V equal for every key: O does not depend on the scores, so dQ = dK = 0."""
    ok = True
    for causal in (False, True):
        q, k, _, do = _problem(21, Nq=6, Nk=6)
        v = np.broadcast_to(_rand((1, 1, 2, 4), 23), (1, 6, 2, 4)).copy()
        dq, dk, dv, _ = ob.attention_bwd(q, k, v, do, causal, 0.9)
        ok &= bool(np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12)
    return ok


def pin_uniform_scores():
    """Q = 0: P_ij = 1/n_i over the visible keys, so dV_j = sum_{i sees j} dO_i / n_i."""
    ok = True
    for causal in (False, True):
        Nq = Nk = 6
        _, k, v, do = _problem(31, Nq=Nq, Nk=Nk)
        q = np.zeros((1, Nq, 2, 4))
        _, _, dv, _ = ob.attention_bwd(q, k, v, do, causal, 0.5)
        ref = np.zeros_like(dv)
        for i in range(Nq):
            keys = range(i + 1) if causal else range(Nk)
            for j in keys:
                ref[:, j] += do[:, i] / len(keys)
        ok &= bool(np.allclose(dv, ref, rtol=1e-12, atol=1e-14))
    return ok


def pin_row_term_identity():
    """D_i = sum_j P_ij dP_ij equals sum_c dO_ic O_ic."""
    ok = True
    for causal in (False, True):
        q, k, v, do = _problem(41, Nq=7, Nk=7)
        _, _, _, D = ob.attention_bwd(q, k, v, do, causal, 0.6)
        O, _ = oracle.attention_fwd(q, k, v, causal, 0.6)
        ok &= bool(np.allclose(D, np.einsum("bnhc,bnhc->bhn", do, O), rtol=1e-12, atol=1e-14))
    return ok


def pin_worked_example():
    g = json.load(open(GOLDEN))
    arr = {n: np.array(g[n], np.float64) for n in ("q", "k", "v", "do", "dq", "dk", "dv", "D")}
    dq, dk, dv, D = ob.attention_bwd(arr["q"], arr["k"], arr["v"], arr["do"], g["causal"], g["scale"])
    return all(bool(np.allclose(x, arr[n], rtol=1e-14, atol=1e-15))
               for x, n in ((dq, "dq"), (dk, "dk"), (dv, "dv"), (D, "D")))


PINS = {
    "finite differences": pin_finite_differences,
    "torch autograd": pin_torch_autograd,
    "constant V": pin_constant_v,
    "uniform scores": pin_uniform_scores,
    "row term identity": pin_row_term_identity,
    "worked example": pin_worked_example,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    assert PINS[name](), name


def test_worked_example_by_hand():
    """The golden file's numbers, recomputed from its stated derivation."""
    g = json.load(open(GOLDEN))
    P = np.array([1 / 3, 2 / 3])
    assert np.allclose(np.array(g["dv"]).ravel(), P)
    assert math.isclose(g["dq"][0][0][0][0], (2 / 3) * math.log(2), rel_tol=1e-15)
    assert np.allclose(np.array(g["dk"]).ravel(), [-2 / 3, 2 / 3])


# ---------------------------------------------------- planted mistakes
def _m_grad_v_no_transpose(P, do):
    return np.resize(P @ np.asarray(do)[: P.shape[1]], (P.shape[1], np.asarray(do).shape[1]))


def _m_grad_v_reversed(P, do):
    return P.T @ np.asarray(do)[::-1]


def _m_grad_p_transposed_v(do, v):
    v = np.asarray(v)
    return np.asarray(do) @ v[::-1].T


def _m_softmax_grad_no_row_term(P, dP):
    return P * dP, (P * dP).sum(axis=1)


def _m_softmax_grad_wrong_axis(P, dP):
    D = (P * dP).sum(axis=0)
    return P * (dP - D[None, :]), (P * dP).sum(axis=1)


def _m_softmax_grad_sign(P, dP):
    D = (P * dP).sum(axis=1)
    return P * (D[:, None] - dP), D


def _m_grad_q_no_scale(dS, k, scale):
    return dS @ np.asarray(k)


def _m_grad_k_no_transpose(dS, q, scale):
    q = np.asarray(q)
    return float(scale) * np.resize(dS @ np.resize(q, (dS.shape[1], q.shape[1])), (dS.shape[1], q.shape[1]))


def _m_grad_k_scale_twice(dS, q, scale):
    return float(scale) ** 2 * (dS.T @ np.asarray(q))


MUTANTS = {
    "dV without the transpose of P": ("grad_v", _m_grad_v_no_transpose),
    "dV with dO rows reversed": ("grad_v", _m_grad_v_reversed),
    "dP with V rows reversed": ("grad_p", _m_grad_p_transposed_v),
    "dS without the row term": ("softmax_grad", _m_softmax_grad_no_row_term),
    "row term over the wrong axis": ("softmax_grad", _m_softmax_grad_wrong_axis),
    "dS sign flipped": ("softmax_grad", _m_softmax_grad_sign),
    "dQ without the scale": ("grad_q", _m_grad_q_no_scale),
    "dK without the transpose of dS": ("grad_k", _m_grad_k_no_transpose),
    "dK with the scale twice": ("grad_k", _m_grad_k_scale_twice),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(ob, attr, fn)
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake '{mutant}' passes every pin"
