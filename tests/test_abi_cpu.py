"""The C-ABI library loads, exports every declared symbol, and rejects bad
arguments on the host before touching any device (runs without a GPU)."""
import ctypes
import os
import re

import pytest

import head_attention_mha_amd as mha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mha.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mha_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mha.LIB_PATH):
        pytest.fail("libmha.so is not built; run `python -m head_attention_mha_amd.build`")
    return mha.load_library()


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert declared == sorted(mha.EXPORTED_SYMBOLS)
    raw = ctypes.CDLL(mha.LIB_PATH)
    for name in declared:
        assert hasattr(raw, name), f"{name} declared in include/mha.h but not exported"


def test_abi_version_matches_header(lib):
    m = re.search(r"#define\s+MHA_ABI_VERSION\s+(\d+)", open(HEADER).read())
    assert mha.mha_abi_version() == int(m.group(1))


def test_status_strings(lib):
    for s in range(5):
        assert mha.mha_status_string(s)
    assert mha.mha_status_string(99) == "unknown status"
    assert mha.mha_status_string(mha.MHA_OK) == "ok"


# Fake, well-separated, 256-byte aligned "device" addresses: validation only
# compares them, it never dereferences them.
Q, K, V, O, L = (0x10000000 * (i + 1) for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Nq=128, Nk=128, d=64, causal=0,
            scale=0.125, stream=None, dtype=mha.MHA_DTYPE_FP16)


def call(**kw):
    a = dict(GOOD)
    a.update(kw)
    return mha.mha_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"], a["Nk"],
                       a["d"], a["causal"], a["scale"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), mha.MHA_ERR_INVALID_ARG),
    (dict(k=0), mha.MHA_ERR_INVALID_ARG),
    (dict(v=0), mha.MHA_ERR_INVALID_ARG),
    (dict(o=0), mha.MHA_ERR_INVALID_ARG),
    (dict(lse=0), mha.MHA_ERR_INVALID_ARG),
    (dict(q=Q + 8), mha.MHA_ERR_INVALID_ARG),
    (dict(o=O + 2), mha.MHA_ERR_INVALID_ARG),
    (dict(lse=L + 2), mha.MHA_ERR_INVALID_ARG),
    (dict(B=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(H=-3), mha.MHA_ERR_INVALID_ARG),
    (dict(Nq=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(Nk=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(Nk=0), mha.MHA_ERR_INVALID_ARG),
    (dict(d=0), mha.MHA_ERR_INVALID_ARG),
    (dict(d=96), mha.MHA_ERR_UNSUPPORTED),
    (dict(d=256), mha.MHA_ERR_UNSUPPORTED),
    (dict(causal=2), mha.MHA_ERR_INVALID_ARG),
    (dict(causal=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(dtype=7), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=0.0), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=-0.125), mha.MHA_ERR_INVALID_ARG),
    (dict(o=Q), mha.MHA_ERR_INVALID_ARG),             # output aliases an input
    (dict(o=K + 64), mha.MHA_ERR_INVALID_ARG),        # output overlaps an input
    (dict(lse=O + 1024), mha.MHA_ERR_INVALID_ARG),    # lse inside o
    (dict(lse=V), mha.MHA_ERR_INVALID_ARG),
], ids=lambda x: str(x))
def test_validation_rejects(lib, kw, want):
    assert call(**kw) == want


@pytest.mark.parametrize("kw", [dict(Nq=0), dict(B=0), dict(H=0),
                                dict(Nq=0, Nk=0, q=0, o=0, lse=0)])
def test_empty_problem_is_a_noop(lib, kw):
    assert call(**kw) == mha.MHA_OK


def test_no_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call() == mha.MHA_ERR_DEVICE


def test_binding_has_no_fallback(tmp_path):
    # loading a missing library raises instead of computing anything else
    from head_attention_mha_amd import _binding
    saved = _binding._lib
    try:
        _binding._lib = None
        with pytest.raises(ImportError):
            _binding.load_library(str(tmp_path / "missing.so"))
    finally:
        _binding._lib = saved
