"""Pins of the fp64 oracle to things other than itself.

Each pin below checks the oracle against something the pages or mathematics
fix: hand-worked examples (tests/golden/worked_examples.json), closed forms,
a library routine (PyTorch's CPU float64 scaled_dot_product_attention and
logsumexp) and the pure-Python brute-force evaluator. ``test_planted_mistakes``
then plants plausible mistakes in the oracle's steps, one at a time, on the
CPU, and requires that at least one pin fails for each.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.attention as oa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")


# ----------------------------------------------------------------- pin checks
# Each returns True when the oracle passes it.

def pin_worked_examples() -> bool:
    ex = json.load(open(GOLDEN))["examples"]
    for e in ex:
        B, H, Nq, Nk, d = e["B"], e["H"], e["Nq"], e["Nk"], e["d"]
        q = np.array(e["q"]).reshape(B, Nq, H, d)
        k = np.array(e["k"]).reshape(B, Nk, H, d)
        v = np.array(e["v"]).reshape(B, Nk, H, d)
        with np.errstate(all="ignore"):
            O, L = oracle.attention_fwd(q, k, v, e["causal"], e["scale"])
        if not (np.all(np.isfinite(O)) and np.all(np.isfinite(L))):
            return False
        if np.abs(O.ravel() - np.array(e["o"])).max() > 1e-12:
            return False
        if np.abs(L.ravel() - np.array(e["lse"])).max() > 1e-12:
            return False
    return True


def test_bruteforce_matches_worked_examples():
    """The brute-force evaluator is pinned to the hand-worked values too."""
    for e in json.load(open(GOLDEN))["examples"]:
        B, H, Nq, Nk, d = e["B"], e["H"], e["Nq"], e["Nk"], e["d"]
        O, L = oracle.attention_fwd_bruteforce(np.array(e["q"]).reshape(B, Nq, H, d),
                                               np.array(e["k"]).reshape(B, Nk, H, d),
                                               np.array(e["v"]).reshape(B, Nk, H, d),
                                               e["causal"], e["scale"])
        np.testing.assert_allclose(O.ravel(), e["o"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(L.ravel(), e["lse"], rtol=0, atol=1e-12)


def _torch_ref(q, k, v, causal, scale):
    import torch
    qt = torch.from_numpy(q).permute(0, 2, 1, 3)  # [B,H,Nq,d]
    kt = torch.from_numpy(k).permute(0, 2, 1, 3)
    vt = torch.from_numpy(v).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(
        qt, kt, vt, is_causal=causal, scale=scale)
    s = scale * (qt @ kt.transpose(-1, -2))
    if causal:
        Nq, Nk = q.shape[1], k.shape[1]
        vis = torch.ones(Nq, Nk, dtype=torch.bool).tril()
        s = s.masked_fill(~vis, float("-inf"))
    lse = torch.logsumexp(s, dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


def pin_torch_sdpa() -> bool:
    rng = np.random.default_rng(123)
    cases = [(2, 3, 7, 7, 8, False), (1, 2, 9, 9, 16, True), (2, 2, 5, 11, 8, True),
             (1, 3, 12, 6, 4, True), (1, 2, 6, 13, 64, False)]
    for B, H, Nq, Nk, d, causal in cases:
        q = rng.standard_normal((B, Nq, H, d))
        k = rng.standard_normal((B, Nk, H, d))
        v = rng.standard_normal((B, Nk, H, d))
        scale = 0.37
        with np.errstate(all="ignore"):
            O, L = oracle.attention_fwd(q, k, v, causal, scale)
        O2, L2 = _torch_ref(q, k, v, causal, scale)
        if not np.all(np.isfinite(O)) or np.abs(O - O2).max() > 1e-12:
            return False
        if not np.all(np.isfinite(L)) or np.abs(L - L2).max() > 1e-12:
            return False
    return True


def pin_bruteforce() -> bool:
    rng = np.random.default_rng(7)
    for B, H, Nq, Nk, d, causal in [(2, 2, 5, 5, 4, False), (1, 2, 6, 6, 8, True),
                                    (2, 1, 4, 7, 4, True), (1, 1, 16, 16, 64, True)]:
        q = rng.standard_normal((B, Nq, H, d))
        k = rng.standard_normal((B, Nk, H, d))
        v = rng.standard_normal((B, Nk, H, d))
        with np.errstate(all="ignore"):
            O, L = oracle.attention_fwd(q, k, v, causal, 0.5)
        O2, L2 = oracle.attention_fwd_bruteforce(q, k, v, causal, 0.5)
        if not np.all(np.isfinite(O)) or np.abs(O - O2).max() > 1e-12:
            return False
        if np.abs(L - L2).max() > 1e-12:
            return False
    return True


def pin_uniform_scores() -> bool:
    """Q = 0: every score is 0, so O_i is the mean of V over the visible keys
    and LSE_i = ln(number of visible keys)."""
    rng = np.random.default_rng(3)
    B, H, Nq, Nk, d = 1, 2, 9, 9, 8
    q = np.zeros((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, H, d))
    v = rng.standard_normal((B, Nk, H, d))
    for causal in (False, True):
        with np.errstate(all="ignore"):
            O, L = oracle.attention_fwd(q, k, v, causal, 0.125)
        for i in range(Nq):
            n = i + 1 if causal else Nk
            want = v[:, :n].mean(axis=1)
            if not np.allclose(O[:, i], want, rtol=0, atol=1e-13):
                return False
            if not np.allclose(L[:, :, i], math.log(n), rtol=0, atol=1e-13):
                return False
    return True


def pin_causal_row0() -> bool:
    """Causal row 0 sees only key 0: O_0 = V_0 and LSE_0 = scale * q_0 . k_0."""
    rng = np.random.default_rng(4)
    B, H, N, d = 2, 2, 10, 16
    q = rng.standard_normal((B, N, H, d))
    k = rng.standard_normal((B, N, H, d))
    v = rng.standard_normal((B, N, H, d))
    with np.errstate(all="ignore"):
        O, L = oracle.attention_fwd(q, k, v, True, 0.25)
    if not np.array_equal(O[:, 0], v[:, 0]):
        return False
    want = 0.25 * np.einsum("bhc,bhc->bh", q[:, 0], k[:, 0])
    return bool(np.allclose(L[:, :, 0], want, rtol=0, atol=1e-13))


def pin_one_hot() -> bool:
    """One key has a dominant score c*scale for every query: O_i = V_j*
    (up to Nk*exp(-c*scale)) and LSE_i = c*scale + ln(1 + (Nk-1) e^{-c*scale})."""
    B, H, Nq, Nk, d = 1, 1, 6, 8, 8
    jstar, c, scale = 5, 320.0, 0.125
    q = np.zeros((B, Nq, H, d))
    q[..., 0] = c
    k = np.zeros((B, Nk, H, d))
    k[:, jstar, :, 0] = 1.0
    v = np.random.default_rng(5).standard_normal((B, Nk, H, d))
    with np.errstate(all="ignore"):
        O, L = oracle.attention_fwd(q, k, v, False, scale)
    t = c * scale
    if not np.allclose(O[:, :, 0], v[:, jstar, 0][:, None, :], rtol=0, atol=Nk * math.exp(-t) * 10):
        return False
    lse = t + math.log1p((Nk - 1) * math.exp(-t))
    if not np.allclose(L, lse, rtol=0, atol=1e-12):
        return False
    # causal rows before j* fall back to the uniform case (all their scores are 0)
    with np.errstate(all="ignore"):
        Oc, Lc = oracle.attention_fwd(q, k, v, True, scale)
    for i in range(Nq):
        if i < jstar:
            if not np.allclose(Oc[0, i, 0], v[0, : i + 1, 0].mean(0), atol=1e-13):
                return False
            if abs(Lc[0, 0, i] - math.log(i + 1)) > 1e-13:
                return False
    return True


def pin_probs_relations() -> bool:
    """Rows of P sum to 1, and P = exp(S - LSE) ("StreamKL" §2)."""
    rng = np.random.default_rng(8)
    B, H, Nq, Nk, d = 1, 2, 7, 9, 8
    q = rng.standard_normal((B, Nq, H, d))
    k = rng.standard_normal((B, Nk, H, d))
    for causal in (False, True):
        for h in range(H):
            with np.errstate(all="ignore"):
                P, lse = oracle.attention_probs(q, k, causal, 0.3, 0, h)
            if np.abs(P.sum(1) - 1).max() > 1e-12:
                return False
            S = 0.3 * q[0, :, h] @ k[0, :, h].T
            if causal:
                S = np.where(np.tril(np.ones((Nq, Nk), bool)), S, -np.inf)
            if np.abs(P - np.exp(S - lse[:, None])).max() > 1e-12:
                return False
    return True


PINS = {
    "worked_examples": pin_worked_examples,
    "torch_sdpa": pin_torch_sdpa,
    "bruteforce": pin_bruteforce,
    "uniform_scores": pin_uniform_scores,
    "causal_row0": pin_causal_row0,
    "one_hot": pin_one_hot,
    "probs_relations": pin_probs_relations,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    assert PINS[name](), f"oracle fails pin {name}"


# ------------------------------------------------------------ invariants
def test_affine_in_v():
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((1, 8, 2, 8)) for _ in range(3))
    for causal in (False, True):
        O, _ = oracle.attention_fwd(q, k, v, causal, 0.4)
        O2, _ = oracle.attention_fwd(q, k, 2 * v + 1, causal, 0.4)
        np.testing.assert_allclose(O2, 2 * O + 1, atol=1e-12)


def test_permutation_invariance():
    rng = np.random.default_rng(12)
    q, k, v = (rng.standard_normal((1, 10, 2, 8)) for _ in range(3))
    perm = rng.permutation(10)
    O, L = oracle.attention_fwd(q, k, v, False, 0.4)
    O2, L2 = oracle.attention_fwd(q, k[:, perm], v[:, perm], False, 0.4)
    np.testing.assert_allclose(O2, O, atol=1e-12)
    np.testing.assert_allclose(L2, L, atol=1e-12)
    O3, L3 = oracle.attention_fwd(q[:, perm], k, v, False, 0.4)
    np.testing.assert_allclose(O3, O[:, perm], atol=1e-12)
    np.testing.assert_allclose(L3, L[:, :, perm], atol=1e-12)


def test_causal_prefix():
    rng = np.random.default_rng(13)
    q, k, v = (rng.standard_normal((1, 12, 1, 8)) for _ in range(3))
    O, L = oracle.attention_fwd(q, k, v, True, 0.4)
    for i in (0, 3, 11):
        Oi, Li = oracle.attention_fwd(q[:, i:i + 1], k[:, : i + 1], v[:, : i + 1], False, 0.4)
        np.testing.assert_allclose(Oi[:, 0], O[:, i], atol=1e-12)
        np.testing.assert_allclose(Li[:, :, 0], L[:, :, i], atol=1e-12)


def test_head_isolation():
    rng = np.random.default_rng(14)
    q, k, v = (rng.standard_normal((2, 6, 3, 8)) for _ in range(3))
    O, L = oracle.attention_fwd(q, k, v, True, 0.4)
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    q2[:, :, 1] += 5
    k2[1] -= 3
    v2[:, :, 2] *= 7
    O2, L2 = oracle.attention_fwd(q2, k2, v2, True, 0.4)
    assert np.array_equal(O2[0, :, 0], O[0, :, 0])
    assert np.array_equal(L2[0, 0], L[0, 0])


def test_row_subset_equals_full():
    rng = np.random.default_rng(15)
    q, k, v = (rng.standard_normal((1, 20, 2, 8)) for _ in range(3))
    rows = np.array([0, 7, 19])
    for causal in (False, True):
        O, L = oracle.attention_fwd(q, k, v, causal, 0.4)
        Os, Ls = oracle.attention_fwd(q, k, v, causal, 0.4, rows=rows)
        assert np.array_equal(Os, O[:, rows])
        assert np.array_equal(Ls, L[:, :, rows])


# ---------------------------------------------------- planted mistakes
def _m_scores_noscale(q, k, scale):
    return np.asarray(q) @ np.asarray(k).T


def _m_scores_twice(q, k, scale):
    return scale * scale * (np.asarray(q) @ np.asarray(k).T)


def _m_scores_sqrt(q, k, scale):
    return math.sqrt(scale) * (np.asarray(q) @ np.asarray(k).T)


def _m_causal_reversed(rows, Nk):
    return np.arange(Nk)[None, :] >= np.asarray(rows)[:, None]


def _m_causal_strict(rows, Nk):
    return np.arange(Nk)[None, :] < np.asarray(rows)[:, None]


def _m_causal_off_by_one(rows, Nk):
    return np.arange(Nk)[None, :] <= np.asarray(rows)[:, None] + 1


def _m_softmax_cols(S):
    S = np.where(np.isfinite(S), S, -1e300)
    m = S.max(axis=0)
    E = np.exp(S - m[None, :])
    l = E.sum(axis=0)
    return E / l[None, :], S.max(axis=1), np.exp(S - S.max(axis=1)[:, None]).sum(1)


def _m_softmax_no_norm(S):
    m = S.max(axis=1)
    E = np.exp(S - m[:, None])
    return E, m, E.sum(axis=1)


def _m_softmax_sign(S):
    m = S.max(axis=1)
    E = np.exp(m[:, None] - S)
    l = E.sum(axis=1)
    return E / l[:, None], m, l


def _m_wv_transposed(P, v):
    return (P @ np.asarray(v)) if P.shape[0] != P.shape[1] else P.T @ np.asarray(v)


def _m_wv_reversed(P, v):
    return P @ np.asarray(v)[::-1]


def _m_lse_log2(m, l):
    return m + np.log2(l)


def _m_lse_no_max(m, l):
    return np.log(l)


def _m_lse_minus(m, l):
    return m - np.log(l)


MUTANTS = {
    "scale dropped": ("scores", _m_scores_noscale),
    "scale applied twice": ("scores", _m_scores_twice),
    "sqrt of scale": ("scores", _m_scores_sqrt),
    "causal mask reversed": ("causal_visible", _m_causal_reversed),
    "causal mask strict": ("causal_visible", _m_causal_strict),
    "causal mask off by one": ("causal_visible", _m_causal_off_by_one),
    "softmax over the wrong axis": ("softmax_rows", _m_softmax_cols),
    "softmax not normalised": ("softmax_rows", _m_softmax_no_norm),
    "softmax sign flipped": ("softmax_rows", _m_softmax_sign),
    "P transposed before P.V": ("weighted_values", _m_wv_transposed),
    "V rows reversed": ("weighted_values", _m_wv_reversed),
    "LSE in log2": ("log_sum_exp", _m_lse_log2),
    "LSE without the max": ("log_sum_exp", _m_lse_no_max),
    "LSE sign of log flipped": ("log_sum_exp", _m_lse_minus),
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    attr, fn = MUTANTS[mutant]
    monkeypatch.setattr(oa, attr, fn)
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake '{mutant}' passes every pin"
