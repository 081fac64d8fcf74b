"""The GPU-vs-oracle comparison rule itself (host only)."""
import numpy as np
import pytest

import workloads as wl
from parity import O_MAX_ABS, assert_parity, compare, half_ulp, passes, report, rounding_floor


def test_half_ulp_values():
    x = np.array([1.0, 1.5, 2.0, 3.9, 4.045, -5.0, 0.25])
    np.testing.assert_array_equal(half_ulp(x, "bf16"),
                                  [2**-8, 2**-8, 2**-7, 2**-7, 2**-6, 2**-6, 2**-10])
    np.testing.assert_array_equal(half_ulp(x, "fp16"),
                                  [2**-11, 2**-11, 2**-10, 2**-10, 2**-9, 2**-9, 2**-13])


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_rounding_floor_is_the_distance_to_the_nearest_value(dtype):
    # brute force: every finite value of the format, nearest by search
    allv = wl.bits_to_f64(np.arange(1 << 16, dtype=np.uint16), dtype)
    allv = np.unique(allv[np.isfinite(allv)])
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.normal(0, 3, 3000), rng.normal(0, 1e-3, 500),
                        [-4.045060491944182, 4.0, 3.9999, 1e-9, -6e-5]])
    pos = np.clip(np.searchsorted(allv, x), 1, len(allv) - 1)
    want = np.minimum(np.abs(x - allv[pos - 1]), np.abs(x - allv[pos]))
    np.testing.assert_array_equal(rounding_floor(x, dtype), want)
    assert np.all(rounding_floor(x, dtype) <= half_ulp(x, dtype))


def _case(values):
    O_ref = np.array(values, np.float64).reshape(1, -1, 1, 1)
    L_ref = np.zeros((1, 1, O_ref.shape[1]))
    return O_ref, L_ref


def test_correctly_rounded_output_passes_and_is_reported():
    # the exact answer rounded to the output format passes, including the
    # element (|O| >= 4, bf16) that no bf16 value brings within 1e-2
    rest = np.random.default_rng(0).normal(0, 0.1, 2000).tolist()
    O_ref, L_ref = _case([-4.045060491944182, 0.3, 1.7, 2.9] + rest)
    bits = wl.round_bits(O_ref.astype(np.float32), "bf16")
    st = compare(bits, L_ref, O_ref, L_ref, "bf16")
    assert st["o_max"] > O_MAX_ABS and st["o_n_over"] == 1 and st["o_over_at_floor"]
    assert st["o_max_at"] == (0, 0, 0, 0) and st["floor_at"] == (0, 0, 0, 0)
    assert st["o_max"] == st["floor"] == pytest.approx(0.013810, abs=1e-6)
    assert passes(st)
    assert_parity(st)
    line = report(st, "case")
    assert "vs 1e-2" in line and "floor 1.381e-02 at (0, 0, 0, 0)" in line
    assert "1 element(s) over 1e-2, all at the format's rounding floor" in line


def test_other_neighbour_at_the_floor_element_fails():
    # at the element whose floor exceeds 1e-2, the farther bf16 neighbour is
    # not allowed: the allowance is the floor itself, not a widened bar
    O_ref, L_ref = _case([-4.045060491944182, 0.5])
    near = wl.round_bits(O_ref.astype(np.float32), "bf16")
    x = wl.bits_to_f32(near, "bf16").astype(np.float64)
    far = x.copy()
    far[0, 0, 0, 0] += 2**-5 if x[0, 0, 0, 0] < O_ref[0, 0, 0, 0] else -2**-5
    st = compare(wl.round_bits(far.astype(np.float32), "bf16"), L_ref, O_ref, L_ref, "bf16")
    assert st["o_n_over"] == 1 and not st["o_over_at_floor"] and not passes(st)
    with pytest.raises(AssertionError):
        assert_parity(st)


def test_an_error_over_the_bar_elsewhere_is_not_excused_by_the_floor():
    # one element sits at its large floor (0.0138); another element, one the
    # format could bring within 1e-2, is off by more than 1e-2: it fails,
    # both above that floor (0.03) and between 1e-2 and it (0.0117)
    O_ref, L_ref = _case([-4.045060491944182, 3.0, 0.25])
    for where, bad in ((1, 3.0 + 0.03), (2, 0.25 + 0.01171875)):
        got = wl.bits_to_f32(wl.round_bits(O_ref.astype(np.float32), "bf16"), "bf16").astype(np.float64)
        got[0, where, 0, 0] = bad
        st = compare(wl.round_bits(got.astype(np.float32), "bf16"), L_ref, O_ref, L_ref, "bf16")
        assert st["o_n_over"] == 2 and not passes(st), (bad, st)


def test_errors_beyond_the_bar_fail():
    O_ref, L_ref = _case([0.5, 1.0, 3.0])
    for bad, which in (([0.5, 1.0, 3.0 + 0.03], "O max"), ([0.5, 1.0, 3.0], "LSE")):
        bits = wl.round_bits(np.array(bad, np.float32).reshape(O_ref.shape), "bf16")
        lse = L_ref + (2e-3 if which == "LSE" else 0.0)
        st = compare(bits, lse, O_ref, L_ref, "bf16")
        with pytest.raises(AssertionError):
            assert_parity(st)


def test_mean_abs_bar():
    O_ref, L_ref = _case(np.linspace(-1, 1, 1000))
    got = O_ref + 2e-3  # under the max-abs bar, over the mean-abs bar
    st = compare(wl.round_bits(got.astype(np.float32), "fp16"), L_ref, O_ref, L_ref, "fp16")
    assert st["o_max"] <= O_MAX_ABS and st["o_mean"] > 1e-3 and not passes(st)


def test_non_finite_fails():
    O_ref, L_ref = _case([0.5, 1.0])
    bits = wl.round_bits(np.array([0.5, np.nan], np.float32).reshape(O_ref.shape), "fp16")
    st = compare(bits, L_ref, O_ref, L_ref, "fp16")
    assert not st["finite"] and not passes(st)


def test_reported_positions_follow_the_row_subset():
    O_ref = np.zeros((2, 3, 2, 4))
    O_ref[1, 2, 1, 3] = 0.7
    L_ref = np.zeros((2, 2, 3))
    got = O_ref.copy()
    got[1, 2, 1, 3] += 0.005
    lse = L_ref.copy()
    lse[0, 1, 1] = 5e-4
    st = compare(wl.round_bits(got.astype(np.float32), "fp16"), lse, O_ref, L_ref, "fp16",
                 rows=np.array([10, 20, 30]))
    assert st["o_max_at"] == (1, 30, 1, 3)
    assert st["lse_max_at"] == (0, 1, 20)
