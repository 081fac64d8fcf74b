"""Pins of the attention-KL oracle (CPU only).

oracle/kl.py is checked against: scipy's relative entropy of the two
softmax rows (a library routine on the materialised distributions),
PyTorch CPU float64 kl_div on the log-softmax rows, KL = 0 for identical
distributions, KL >= 0 (Gibbs), a two-key closed form, the page's online
form acc/l1 + LSE2 - LSE1, the causal mask (row 0 sees one key, so KL = 0),
and planted mistakes.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

import oracle
import oracle.kl as okl


def _problem(seed, B=2, H=2, Nq=6, Nk=9, d=4, std2=1.0):
    rng = np.random.default_rng(seed)
    q1 = rng.standard_normal((B, Nq, H, d))
    k1 = rng.standard_normal((B, Nk, H, d))
    q2 = q1 + std2 * rng.standard_normal((B, Nq, H, d))
    k2 = k1 + std2 * rng.standard_normal((B, Nk, H, d))
    return q1, k1, q2, k2


def _softmax(S):
    e = np.exp(S - S.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


def pin_scipy_rel_entr():
    from scipy.special import rel_entr
    ok = True
    for causal in (False, True):
        q1, k1, q2, k2 = _problem(1, Nq=9)
        KL, _, _ = okl.attention_kl(q1, k1, q2, k2, causal, 0.6)
        for b in range(2):
            for h in range(2):
                S1 = 0.6 * q1[b, :, h] @ k1[b, :, h].T
                S2 = 0.6 * q2[b, :, h] @ k2[b, :, h].T
                if causal:
                    m = np.triu(np.ones_like(S1, bool), 1)
                    S1[m] = -np.inf
                    S2[m] = -np.inf
                ref = rel_entr(_softmax(S1), _softmax(S2)).sum(axis=1)
                ok &= bool(np.allclose(KL[b, h], ref, rtol=1e-10, atol=1e-13))
    return ok


def pin_torch_kl_div():
    torch = pytest.importorskip("torch")
    q1, k1, q2, k2 = _problem(2, Nq=7, Nk=7, d=8)
    ok = True
    for causal in (False, True):
        KL, L1, L2 = okl.attention_kl(q1, k1, q2, k2, causal, 0.3)
        for b in range(2):
            for h in range(2):
                S1 = torch.tensor(0.3 * q1[b, :, h] @ k1[b, :, h].T)
                S2 = torch.tensor(0.3 * q2[b, :, h] @ k2[b, :, h].T)
                if causal:
                    m = torch.triu(torch.ones_like(S1, dtype=torch.bool), 1)
                    S1 = S1.masked_fill(m, -math.inf)
                    S2 = S2.masked_fill(m, -math.inf)
                lp1, lp2 = torch.log_softmax(S1, 1), torch.log_softmax(S2, 1)
                # kl_div(input=log P2, target=log P1, log_target) = P1 (log P1 - log P2)
                ref = torch.nn.functional.kl_div(lp2, lp1, reduction="none", log_target=True)
                ref = torch.nan_to_num(ref, nan=0.0).sum(1).numpy()
                ok &= bool(np.allclose(KL[b, h], ref, rtol=1e-10, atol=1e-13))
                ok &= bool(np.allclose(L1[b, h], torch.logsumexp(S1, 1).numpy(), rtol=1e-13))
                ok &= bool(np.allclose(L2[b, h], torch.logsumexp(S2, 1).numpy(), rtol=1e-13))
    return ok


def pin_identical_is_zero_and_gibbs():
    q1, k1, _, _ = _problem(3)
    KL, L1, L2 = okl.attention_kl(q1, k1, q1, k1, False, 0.5)
    ok = bool(np.abs(KL).max() < 1e-13 and np.allclose(L1, L2, rtol=1e-15))
    for seed in range(4, 9):
        q1, k1, q2, k2 = _problem(seed, std2=2.0)
        for causal in (False, True):
            KL, _, _ = okl.attention_kl(q1, k1, q2, k2, causal, 0.7)
            ok &= bool(KL.min() >= -1e-13)
    return ok


def pin_two_key_closed_form():
    """One row, two keys: P1 = (a, 1-a), P2 = (c, 1-c) from scores chosen by
    hand; KL = a ln(a/c) + (1-a) ln((1-a)/(1-c))."""
    q1 = np.array([[[[1.0]]]])
    k1 = np.array([[[[0.0]], [[1.0]]]])       # S1 = (0, 1)
    q2 = np.array([[[[2.0]]]])
    k2 = np.array([[[[0.5]], [[-0.5]]]])      # S2 = (1, -1)
    KL, L1, L2 = okl.attention_kl(q1, k1, q2, k2, False, 1.0)
    a = 1 / (1 + math.e)                      # P1(key 0)
    c = 1 / (1 + math.exp(-2))                # P2(key 0)
    want = a * math.log(a / c) + (1 - a) * math.log((1 - a) / (1 - c))
    return bool(math.isclose(KL[0, 0, 0], want, rel_tol=1e-14)
                and math.isclose(L1[0, 0, 0], math.log(1 + math.e), rel_tol=1e-15)
                and math.isclose(L2[0, 0, 0], math.log(math.e + math.exp(-1)), rel_tol=1e-15))


def pin_online_form():
    ok = True
    for causal in (False, True):
        q1, k1, q2, k2 = _problem(10, Nq=8, Nk=8, std2=1.5)
        KL, L1, L2 = okl.attention_kl(q1, k1, q2, k2, causal, 0.45)
        for b in range(2):
            for h in range(2):
                m1, l1, m2, l2, acc = okl.kl_online_terms(q1, k1, q2, k2, causal, 0.45, b, h)
                lse1, lse2 = m1 + np.log(l1), m2 + np.log(l2)
                ok &= bool(np.allclose(acc / l1 + lse2 - lse1, KL[b, h], rtol=1e-12, atol=1e-13))
                ok &= bool(np.allclose(lse1, L1[b, h], rtol=1e-14))
    return ok


def pin_causal_row_zero():
    q1, k1, q2, k2 = _problem(11, std2=2.0)
    KL, L1, _ = okl.attention_kl(q1, k1, q2, k2, True, 0.8)
    want_l1 = 0.8 * np.einsum("bhc,bhc->bh", q1[:, 0], k1[:, 0])
    return bool(np.abs(KL[:, :, 0]).max() < 1e-14 and np.allclose(L1[:, :, 0], want_l1, rtol=1e-14))


PINS = {
    "scipy rel_entr": pin_scipy_rel_entr,
    "torch kl_div": pin_torch_kl_div,
    "identical and Gibbs": pin_identical_is_zero_and_gibbs,
    "two-key closed form": pin_two_key_closed_form,
    "online form": pin_online_form,
    "causal row 0": pin_causal_row_zero,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    assert PINS[name](), name


def _m_reversed(q1, k1, q2, k2, causal, scale, rows=None):
    return _orig(q2, k2, q1, k1, causal, scale, rows)


def _m_no_lse(q1, k1, q2, k2, causal, scale, rows=None):
    KL, L1, L2 = _orig(q1, k1, q2, k2, causal, scale, rows)
    return KL - (L2 - L1), L1, L2


def _m_swapped_mask_direction(q1, k1, q2, k2, causal, scale, rows=None):
    if not causal:
        return _orig(q1, k1, q2, k2, causal, scale, rows)
    rev = lambda x: x[:, ::-1]
    KL, L1, L2 = _orig(rev(q1), rev(k1), rev(q2), rev(k2), causal, scale, rows)
    return KL[:, :, ::-1], L1[:, :, ::-1], L2[:, :, ::-1]


def _m_scale_dropped(q1, k1, q2, k2, causal, scale, rows=None):
    return _orig(q1, k1, q2, k2, causal, 1.0, rows)


_orig = okl.attention_kl
MUTANTS = {
    "KL(P2 || P1)": _m_reversed,
    "log ratio without the LSEs": _m_no_lse,
    "causal mask reversed": _m_swapped_mask_direction,
    "scale dropped": _m_scale_dropped,
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(okl, "attention_kl", MUTANTS[mutant])
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake '{mutant}' passes every pin"
