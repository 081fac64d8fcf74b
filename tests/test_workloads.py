"""Seeded input generators: rounding, determinism, distributions, and the
output-rounding floor of each workload against the parity tolerance."""
import numpy as np
import pytest

import oracle
import workloads as wl


def test_bf16_round_to_nearest_even():
    # 1 + 2^-8 is exactly halfway between bf16 1.0 and 1 + 2^-7: ties to even -> 1.0
    # 1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6: ties to even -> 1 + 2^-6
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.5, 65504.0, 1e-40],
                 dtype=np.float32)
    bits = wl.f32_to_bf16_bits(x)
    back = wl.bits_to_f32(bits, "bf16")
    want = np.array([1.0, 1.0, 1 + 2**-6, 1 + 2**-7, -2.5, 65536.0, 0.0], dtype=np.float32)
    # 1e-40 is a subnormal fp32; bf16 keeps fp32's exponent range, so it rounds
    # to the nearest bf16 subnormal, which is close to but not exactly 1e-40
    np.testing.assert_array_equal(back[:6], want[:6])
    assert abs(back[6] - 1e-40) < 1e-41
    assert bits[0] == 0x3F80 and bits[4] == 0xC020


def test_bf16_nan_stays_nan():
    bits = wl.f32_to_bf16_bits(np.array([np.nan, np.inf, -np.inf], np.float32))
    back = wl.bits_to_f32(bits, "bf16")
    assert np.isnan(back[0]) and back[1] == np.inf and back[2] == -np.inf


def test_fp16_rounding_and_widening_exact():
    x = np.array([1 + 2**-11, 1 + 3 * 2**-11, 0.1], np.float32)
    back = wl.bits_to_f64(wl.f32_to_f16_bits(x), "fp16")
    np.testing.assert_array_equal(back, [1.0, 1 + 2**-9, float(np.float16(0.1))])


def test_generator_deterministic_and_shaped():
    for name in ("tiny", "cross"):
        w = wl.WORKLOADS[name]
        a = wl.make_inputs(w)
        b = wl.make_inputs(w)
        for x, y in zip(a, b):
            assert x.dtype == np.uint16
            assert np.array_equal(x, y)
        assert a[0].shape == (w.B, w.Nq, w.H, w.d)
        assert a[1].shape == (w.B, w.Nk, w.H, w.d)


def test_distribution_and_cross_doubling():
    w = wl.WORKLOADS["cross"]
    q, k, v = (wl.bits_to_f64(x, w.dtype) for x in wl.make_inputs(w))
    for x, sd in ((q, 1.0), (v, 1.0), (k, 2.0)):
        assert abs(x.mean()) < 0.01
        assert abs(x.std() - sd) < 0.01 * sd
    # K is doubled after rounding: every K value is twice an fp16 value
    k_half = (k / 2).astype(np.float16).astype(np.float64)
    assert np.array_equal(k_half * 2, k)


def test_workload_table():
    w = wl.WORKLOADS["long_causal"]
    assert (w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.causal, w.seed) == (1, 8, 16384, 16384, 128, "bf16", True, 3)
    assert w.flops == pytest.approx(4 * 8 * 16384 * 16384 * 128 / 2)
    assert w.scale == float(np.float32(1 / np.sqrt(128)))


def _floor_rows(w, rng):
    head = np.arange(min(w.Nq, 64))
    rest = rng.choice(w.Nq, size=min(w.Nq, 64), replace=False)
    return np.unique(np.concatenate([head, rest]))


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_output_rounding_floor(name):
    """The parity bound on O is max-abs <= 1e-2 against the unrounded fp64 O.
    Rounding the exact O to the output dtype already costs half an ulp; check
    on the rows where |O| is largest (the first causal rows) plus a random
    sample that this unavoidable floor stays well inside the bound."""
    w = wl.WORKLOADS[name]
    q, k, v = (wl.bits_to_f64(x, w.dtype) for x in wl.make_inputs(w))
    rows = _floor_rows(w, np.random.default_rng(0))
    heads = range(w.H) if w.H * w.B <= 16 else range(0, w.H, max(1, w.H // 4))
    worst = 0.0
    for b in range(min(w.B, 2)):
        for h in heads:
            O, _ = oracle.attention_fwd(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                        v[b:b + 1, :, h:h + 1], w.causal, w.scale, rows=rows)
            Or = wl.bits_to_f64(wl.round_bits(O.astype(np.float32), w.dtype), w.dtype)
            worst = max(worst, float(np.abs(Or - O).max()))
    print(f"{name}: output rounding floor on sampled rows = {worst:.3e}")
    assert worst < 8e-3
