"""Pins of the split-over-keys oracle (CPU only).

oracle/split.py computes the forward block by block over the keys and merges
the blocks by their LSE. It is pinned against the unsplit oracle (itself
pinned in test_oracle_pins.py) for several partitions, causal and not, with
Nq != Nk; a single block must reproduce the unsplit result; blocks that no
row can see must drop out; and planted mistakes in the merge fail a pin.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import oracle.split as osp


def _problem(seed, B=2, H=2, Nq=5, Nk=23, d=8):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Nq, H, d)), rng.standard_normal((B, Nk, H, d)),
            rng.standard_normal((B, Nk, H, d)))


PARTITIONS = [[0, 23], [0, 7, 23], [0, 1, 2, 3, 23], [0, 5, 10, 15, 20, 23], [0, 11, 11, 23],
              list(range(0, 24))]


def pin_matches_unsplit():
    ok = True
    for causal in (False, True):
        for Nq in (1, 5, 30):
            q, k, v = _problem(3 + Nq, Nq=Nq)
            O, L = oracle.attention_fwd(q, k, v, causal, 0.4)
            for bounds in PARTITIONS:
                Os, Ls = osp.attention_fwd_split(q, k, v, causal, 0.4, bounds)
                ok &= bool(np.allclose(Os, O, rtol=1e-12, atol=1e-13)
                           and np.allclose(Ls, L, rtol=1e-12, atol=1e-13))
    return ok


def pin_single_block_is_the_whole_softmax():
    q, k, v = _problem(7)
    O_p, L_p = osp.split_partials(q, k, v, False, 0.3, [0, 23])
    O, L = oracle.attention_fwd(q, k, v, False, 0.3)
    return bool(np.allclose(O_p[0], O, rtol=1e-13, atol=1e-14)
                and np.allclose(L_p[0], L, rtol=1e-13, atol=1e-14))


def pin_invisible_blocks_drop_out():
    """Causal, Nq = 4: keys 4.. are visible to no row; their blocks are -inf /
    zero and the merged result equals the result over keys 0..3 alone."""
    q, k, v = _problem(9, Nq=4, Nk=23)
    O_p, L_p = osp.split_partials(q, k, v, True, 0.5, [0, 4, 9, 23])
    ok = bool(np.all(L_p[1:] == -np.inf) and np.all(O_p[1:] == 0))
    O, L = osp.merge_splits(O_p, L_p)
    O4, L4 = oracle.attention_fwd(q, k[:, :4], v[:, :4], True, 0.5)
    return ok and bool(np.allclose(O, O4, rtol=1e-13, atol=1e-14)
                       and np.allclose(L, L4, rtol=1e-13, atol=1e-14))


def pin_two_block_closed_form():
    """One row, two single-key blocks with scores s1, s2: the merge weights
    are the two-way softmax, LSE = log(e^s1 + e^s2)."""
    q = np.array([[[[1.0]]]])
    k = np.array([[[[0.5]], [[-1.0]]]])
    v = np.array([[[[3.0]], [[7.0]]]])
    O, L = osp.attention_fwd_split(q, k, v, False, 1.0, [0, 1, 2])
    w1 = np.exp(0.5) / (np.exp(0.5) + np.exp(-1.0))
    return bool(np.isclose(O[0, 0, 0, 0], 3 * w1 + 7 * (1 - w1), rtol=1e-15)
                and np.isclose(L[0, 0, 0], np.log(np.exp(0.5) + np.exp(-1.0)), rtol=1e-15))


PINS = {
    "matches unsplit": pin_matches_unsplit,
    "single block": pin_single_block_is_the_whole_softmax,
    "invisible blocks": pin_invisible_blocks_drop_out,
    "two-block closed form": pin_two_block_closed_form,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    assert PINS[name](), name


def _m_plain_mean(O_parts, LSE_parts):
    n = np.isfinite(LSE_parts).sum(axis=0)
    M = np.where(np.isfinite(LSE_parts), LSE_parts, 0).max(axis=0)
    O = np.asarray(O_parts).sum(axis=0) / np.moveaxis(n, 2, 1)[..., None]
    return O, M + np.log(n)


def _m_weights_not_normalised(O_parts, LSE_parts):
    M = np.max(LSE_parts, axis=0)
    w = np.exp(np.asarray(LSE_parts) - M[None])
    return np.einsum("sbhn,sbnhc->bnhc", w, O_parts), M + np.log(w.sum(axis=0))


def _m_lse_max_only(O_parts, LSE_parts):
    M = np.max(LSE_parts, axis=0)
    w = np.exp(np.asarray(LSE_parts) - M[None])
    share = w / w.sum(axis=0)[None]
    return np.einsum("sbhn,sbnhc->bnhc", share, O_parts), M


MUTANTS = {
    "merge weights without the normaliser": _m_weights_not_normalised,
    "merge as a plain mean": _m_plain_mean,
    "LSE as the largest block LSE": _m_lse_max_only,
}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(osp, "merge_splits", MUTANTS[mutant])
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake '{mutant}' passes every pin"
