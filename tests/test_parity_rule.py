"""The GPU-vs-oracle comparison rule itself (host only)."""
import numpy as np

import workloads as wl
from parity import O_MAX_ABS, assert_parity, compare, half_ulp


def test_half_ulp_values():
    x = np.array([1.0, 1.5, 2.0, 3.9, 4.045, -5.0, 0.25])
    np.testing.assert_array_equal(half_ulp(x, "bf16"),
                                  [2**-8, 2**-8, 2**-7, 2**-7, 2**-6, 2**-6, 2**-10])
    np.testing.assert_array_equal(half_ulp(x, "fp16"),
                                  [2**-11, 2**-11, 2**-10, 2**-10, 2**-9, 2**-9, 2**-13])


def _case(values, dtype):
    O_ref = np.array(values, np.float64).reshape(1, -1, 1, 1)
    L_ref = np.zeros((1, 1, O_ref.shape[1]))
    return O_ref, L_ref


def test_correctly_rounded_output_passes():
    # the exact answer rounded to the output format passes, including the
    # element (|O| >= 4, bf16) that no bf16 value can bring within 1e-2
    rest = np.random.default_rng(0).normal(0, 0.1, 2000).tolist()
    O_ref, L_ref = _case([-4.045060491944182, 0.3, 1.7, 2.9] + rest, "bf16")
    bits = wl.round_bits(O_ref.astype(np.float32), "bf16")
    st = compare(bits, L_ref, O_ref, L_ref, "bf16")
    assert st["o_max"] > O_MAX_ABS and st["o_n_over_1e2"] == 1
    assert_parity(st)


def test_errors_beyond_the_bar_fail():
    O_ref, L_ref = _case([0.5, 1.0, 3.0], "bf16")
    for bad, which in (([0.5, 1.0, 3.0 + 0.03], "O max"), ([0.5, 1.0, 3.0], "LSE")):
        bits = wl.round_bits(np.array(bad, np.float32).reshape(O_ref.shape), "bf16")
        lse = L_ref + (2e-3 if which == "LSE" else 0.0)
        st = compare(bits, lse, O_ref, L_ref, "bf16")
        try:
            assert_parity(st)
        except AssertionError:
            continue
        raise AssertionError(f"{which} error not caught: {st}")


def test_non_finite_fails():
    O_ref, L_ref = _case([0.5, 1.0], "fp16")
    bits = wl.round_bits(np.array([0.5, np.nan], np.float32).reshape(O_ref.shape), "fp16")
    st = compare(bits, L_ref, O_ref, L_ref, "fp16")
    assert not st["finite"]
