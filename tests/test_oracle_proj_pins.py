"""Pins of the output-projection oracle (CPU only): the matrix form against
element-by-element evaluation, the per-head sum form, the identity weight
(Y = the concatenated heads), a one-hot weight row (Y picks one channel of
one head), linearity in the bias, and planted mistakes (a transposed weight,
heads concatenated in the wrong order, a dropped bias)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle.proj as op


def _problem(seed, B=2, Nq=3, H=3, d=4, E=5):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, Nq, H, d)), rng.standard_normal((E, H * d)),
            rng.standard_normal(E))


def pin_bruteforce():
    o, w, b = _problem(1)
    return bool(np.allclose(op.out_proj(o, w, b), op.out_proj_bruteforce(o, w, b), rtol=1e-13,
                            atol=1e-13))


def pin_by_heads():
    o, w, b = _problem(2, H=4, d=8, E=6)
    return bool(np.allclose(op.out_proj(o, w, b), op.out_proj_by_heads(o, w, b), rtol=1e-12,
                            atol=1e-12))


def pin_identity_weight():
    o, _, _ = _problem(3)
    B, Nq, H, d = o.shape
    y = op.out_proj(o, np.eye(H * d))
    return bool(np.array_equal(y, o.reshape(B, Nq, H * d)))


def pin_one_hot_row():
    """W row e selects channel c of head h: Y[..., e] = O[..., h, c]."""
    o, _, _ = _problem(4)
    B, Nq, H, d = o.shape
    w = np.zeros((3, H * d))
    w[0, 1 * d + 2] = 1.0   # head 1, channel 2
    w[1, 2 * d + 0] = 1.0   # head 2, channel 0
    w[2, 0 * d + 3] = -2.0  # head 0, channel 3, scaled
    y = op.out_proj(o, w)
    return bool(np.array_equal(y[..., 0], o[:, :, 1, 2]) and np.array_equal(y[..., 1], o[:, :, 2, 0])
                and np.array_equal(y[..., 2], -2.0 * o[:, :, 0, 3]))


def pin_bias_is_added_once():
    o, w, b = _problem(5)
    return bool(np.allclose(op.out_proj(o, w, b) - op.out_proj(o, w), b[None, None, :],
                            rtol=1e-13, atol=1e-13))


PINS = {
    "brute force": pin_bruteforce,
    "by heads": pin_by_heads,
    "identity weight": pin_identity_weight,
    "one-hot rows": pin_one_hot_row,
    "bias once": pin_bias_is_added_once,
}


@pytest.mark.parametrize("name", list(PINS))
def test_pin(name):
    assert PINS[name](), name


_orig = op.out_proj


def _m_heads_reversed(o, w, bias=None):
    return _orig(np.asarray(o)[:, :, ::-1, :], w, bias)


def _m_weight_transposed_blocks(o, w, bias=None):
    o = np.asarray(o)
    H, d = o.shape[2], o.shape[3]
    w = np.asarray(w)
    # channel-major instead of head-major concatenation
    return _orig(np.ascontiguousarray(o.transpose(0, 1, 3, 2)).reshape(o.shape), w, bias)


def _m_bias_dropped(o, w, bias=None):
    return _orig(o, w, None)


MUTANTS = {"heads concatenated in reverse": _m_heads_reversed,
           "channel-major concatenation": _m_weight_transposed_blocks,
           "bias dropped": _m_bias_dropped}


@pytest.mark.parametrize("mutant", list(MUTANTS))
def test_planted_mistakes(mutant, monkeypatch):
    monkeypatch.setattr(op, "out_proj", MUTANTS[mutant])
    failed = []
    for name, pin in PINS.items():
        try:
            ok = pin()
        except Exception:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"planted mistake '{mutant}' passes every pin"
