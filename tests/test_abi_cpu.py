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


# ------------------------------------------------------------------ mha_bwd
BQ, BK, BV, BO, BG, BL, DQ, DK, DV, DL = (0x10000000 * (i + 1) for i in range(10))
GOOD_BWD = dict(q=BQ, k=BK, v=BV, o=BO, dout=BG, lse=BL, dq=DQ, dk=DK, dv=DV, delta=DL,
                B=1, H=2, Nq=128, Nk=128, d=64, causal=0, scale=0.125, stream=None,
                dtype=mha.MHA_DTYPE_BF16)


def call_bwd(**kw):
    a = dict(GOOD_BWD)
    a.update(kw)
    return mha.mha_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                       a["dv"], a["delta"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["causal"],
                       a["scale"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,want", [
    *[(dict([(n, 0)]), mha.MHA_ERR_INVALID_ARG)
      for n in ("q", "k", "v", "o", "dout", "lse", "dq", "dk", "dv", "delta")],
    *[(dict([(n, GOOD_BWD[n] + 8)]), mha.MHA_ERR_INVALID_ARG)
      for n in ("q", "k", "v", "o", "dout", "dq", "dk", "dv")],
    (dict(lse=BL + 2), mha.MHA_ERR_INVALID_ARG),
    (dict(delta=DL + 1), mha.MHA_ERR_INVALID_ARG),
    (dict(B=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(Nq=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(Nk=0), mha.MHA_ERR_INVALID_ARG),
    (dict(d=96), mha.MHA_ERR_UNSUPPORTED),
    (dict(causal=3), mha.MHA_ERR_INVALID_ARG),
    (dict(dtype=5), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=0.0), mha.MHA_ERR_INVALID_ARG),
    (dict(dq=BQ), mha.MHA_ERR_INVALID_ARG),           # dq aliases q
    (dict(dk=BG + 256), mha.MHA_ERR_INVALID_ARG),     # dk inside dout
    (dict(dv=DK), mha.MHA_ERR_INVALID_ARG),           # two outputs alias
    (dict(delta=DQ + 4096), mha.MHA_ERR_INVALID_ARG), # delta inside dq
    (dict(delta=BL), mha.MHA_ERR_INVALID_ARG),        # delta aliases lse
], ids=lambda x: str(x))
def test_bwd_validation_rejects(lib, kw, want):
    assert call_bwd(**kw) == want


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(Nq=0, Nk=0),
                                dict(B=0, q=0, k=0, v=0, o=0, dout=0, lse=0, dq=0, dk=0, dv=0,
                                     delta=0)])
def test_bwd_empty_problem_is_a_noop(lib, kw):
    assert call_bwd(**kw) == mha.MHA_OK


def test_bwd_no_queries_still_needs_key_buffers(lib):
    # Nq == 0 with keys: dK = dV = 0 must be written, so their pointers are
    # required while the query-side ones may be null
    q_side = dict(q=0, o=0, dout=0, lse=0, dq=0, delta=0)
    assert call_bwd(Nq=0, dk=0, **q_side) == mha.MHA_ERR_INVALID_ARG
    assert call_bwd(Nq=0, v=0, **q_side) == mha.MHA_ERR_INVALID_ARG


def test_bwd_no_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_bwd() == mha.MHA_ERR_DEVICE
    assert call_bwd(Nq=0, q=0, o=0, dout=0, lse=0, dq=0, delta=0) == mha.MHA_ERR_DEVICE


# ---------------------------------------------------------- mha_fwd_splitkv
OP, LP = 0x10000000 * 20, 0x10000000 * 21
GOOD_SPLIT = dict(GOOD, Nq=4, n_splits=8, o_part=OP, lse_part=LP)


def call_split(**kw):
    a = dict(GOOD_SPLIT)
    a.update(kw)
    return mha.mha_fwd_splitkv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Nq"],
                               a["Nk"], a["d"], a["causal"], a["scale"], a["n_splits"],
                               a["o_part"], a["lse_part"], a["stream"], a["dtype"])


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), mha.MHA_ERR_INVALID_ARG),
    (dict(o_part=0), mha.MHA_ERR_INVALID_ARG),
    (dict(lse_part=0), mha.MHA_ERR_INVALID_ARG),
    (dict(o_part=OP + 4), mha.MHA_ERR_INVALID_ARG),     # o_part needs 16-byte alignment
    (dict(lse_part=LP + 2), mha.MHA_ERR_INVALID_ARG),
    (dict(n_splits=0), mha.MHA_ERR_INVALID_ARG),
    (dict(n_splits=257), mha.MHA_ERR_INVALID_ARG),
    (dict(Nq=9), mha.MHA_ERR_UNSUPPORTED),
    (dict(d=96), mha.MHA_ERR_UNSUPPORTED),
    (dict(Nk=0), mha.MHA_ERR_INVALID_ARG),
    (dict(o_part=K + 64), mha.MHA_ERR_INVALID_ARG),     # workspace overlaps an input
    (dict(lse_part=O), mha.MHA_ERR_INVALID_ARG),        # workspace overlaps the output
    (dict(lse_part=OP + 64), mha.MHA_ERR_INVALID_ARG),  # the two workspaces overlap
    (dict(scale=float("nan")), mha.MHA_ERR_INVALID_ARG),
], ids=lambda x: str(x))
def test_splitkv_validation_rejects(lib, kw, want):
    assert call_split(**kw) == want


def test_splitkv_empty_is_a_noop(lib):
    assert call_split(Nq=0, o_part=0, lse_part=0) == mha.MHA_OK
    assert call_split(B=0) == mha.MHA_OK


def test_splitkv_default_splits(lib):
    f = mha.mha_fwd_splitkv_splits
    assert f(4, 32, 1, 32768) == 16          # 2048 workgroups over 128 heads
    assert f(1, 1, 1, 100) == 1              # one 256-key block
    assert f(1, 1, 1, 10 ** 6) == 256        # capped
    assert f(64, 64, 1, 4096) == 1
    assert f(0, 1, 1, 1) == 1 and f(1, 1, 1, 0) == 1


def test_splitkv_no_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_split() == mha.MHA_ERR_DEVICE


# --------------------------------------------------------------- mha_kl_fwd
A1, A2, A3, A4, OK_, OL1, OL2 = (0x10000000 * (i + 30) for i in range(7))
GOOD_KL = dict(q1=A1, k1=A2, q2=A3, k2=A4, kl=OK_, lse1=OL1, lse2=OL2, B=1, H=2, Nq=128,
               Nk=128, d=128, causal=1, scale=0.088, stream=None, dtype=mha.MHA_DTYPE_BF16)


def call_kl(**kw):
    a = dict(GOOD_KL)
    a.update(kw)
    return mha.mha_kl_fwd(*(a[n] for n in ("q1", "k1", "q2", "k2", "kl", "lse1", "lse2", "B", "H",
                                         "Nq", "Nk", "d", "causal", "scale", "stream", "dtype")))


@pytest.mark.parametrize("kw,want", [
    *[(dict([(n, 0)]), mha.MHA_ERR_INVALID_ARG)
      for n in ("q1", "k1", "q2", "k2", "kl", "lse1", "lse2")],
    *[(dict([(n, GOOD_KL[n] + 8)]), mha.MHA_ERR_INVALID_ARG) for n in ("q1", "k1", "q2", "k2")],
    (dict(kl=OK_ + 2), mha.MHA_ERR_INVALID_ARG),
    (dict(Nk=0), mha.MHA_ERR_INVALID_ARG),
    (dict(d=32), mha.MHA_ERR_UNSUPPORTED),
    (dict(causal=5), mha.MHA_ERR_INVALID_ARG),
    (dict(dtype=3), mha.MHA_ERR_INVALID_ARG),
    (dict(scale=-1.0), mha.MHA_ERR_INVALID_ARG),
    (dict(kl=A2 + 64), mha.MHA_ERR_INVALID_ARG),   # output inside an input
    (dict(lse2=OL1), mha.MHA_ERR_INVALID_ARG),     # two outputs alias
], ids=lambda x: str(x))
def test_kl_validation_rejects(lib, kw, want):
    assert call_kl(**kw) == want


def test_kl_empty_is_a_noop(lib):
    assert call_kl(Nq=0, q1=0, q2=0, kl=0, lse1=0, lse2=0) == mha.MHA_OK
    assert call_kl(H=0) == mha.MHA_OK


def test_kl_no_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_kl() == mha.MHA_ERR_DEVICE


# ------------------------------------------------------------- mha_out_proj
PO, PW, PB, PY = (0x10000000 * (i + 40) for i in range(4))
GOOD_PROJ = dict(o=PO, w=PW, bias=PB, y=PY, B=1, Nq=100, H=8, d=128, E=1024, stream=None,
                 dtype=mha.MHA_DTYPE_BF16)


def call_proj(**kw):
    a = dict(GOOD_PROJ)
    a.update(kw)
    return mha.mha_out_proj(*(a[n] for n in ("o", "w", "bias", "y", "B", "Nq", "H", "d", "E",
                                           "stream", "dtype")))


@pytest.mark.parametrize("kw,want", [
    (dict(o=0), mha.MHA_ERR_INVALID_ARG),
    (dict(w=0), mha.MHA_ERR_INVALID_ARG),
    (dict(y=0), mha.MHA_ERR_INVALID_ARG),
    (dict(o=PO + 8), mha.MHA_ERR_INVALID_ARG),
    (dict(y=PY + 8), mha.MHA_ERR_INVALID_ARG),
    (dict(bias=PB + 4), mha.MHA_ERR_INVALID_ARG),
    (dict(H=3, d=48), mha.MHA_ERR_UNSUPPORTED),     # H*d = 144, not a multiple of 64
    (dict(E=1022), mha.MHA_ERR_UNSUPPORTED),        # E not a multiple of 4
    (dict(H=0), mha.MHA_ERR_INVALID_ARG),           # nothing to project from
    (dict(dtype=9), mha.MHA_ERR_INVALID_ARG),
    (dict(B=-1), mha.MHA_ERR_INVALID_ARG),
    (dict(y=PO + 1024), mha.MHA_ERR_INVALID_ARG),   # output overlaps O
    (dict(bias=PY + 64), mha.MHA_ERR_INVALID_ARG),  # bias inside the output
], ids=lambda x: str(x))
def test_proj_validation_rejects(lib, kw, want):
    assert call_proj(**kw) == want


def test_proj_empty_and_no_bias(lib):
    assert call_proj(Nq=0, o=0, y=0) == mha.MHA_OK
    assert call_proj(E=0) == mha.MHA_OK
    import torch
    if not torch.cuda.is_available():
        assert call_proj(bias=None) == mha.MHA_ERR_DEVICE  # a null bias is valid


# -------------------------------------- 32-bit offsets within a tile of rows
# A workgroup addresses up to 256 token rows of H*d elements (or 256 rows of
# K = H*d for the projection) through 32-bit byte offsets, so a row may hold
# at most 2^23 elements; every entry point rejects more before any HIP call.
@pytest.mark.parametrize("entry", ["fwd", "bwd", "kl", "split", "proj"])
def test_rows_past_2p23_elements_are_rejected(lib, entry):
    big = dict(H=65537, d=128, Nq=1, Nk=1)
    if entry == "fwd":
        st = call(**big)
    elif entry == "bwd":
        st = call_bwd(**big)
    elif entry == "kl":
        st = call_kl(**big)
    elif entry == "split":
        st = call_split(**big, n_splits=1)
    else:
        st = call_proj(H=65537, d=128, Nq=1, B=1)
    assert st == mha.MHA_ERR_INVALID_ARG


@pytest.mark.parametrize("entry", ["fwd", "bwd", "kl", "proj"])
def test_rows_of_2p23_elements_pass_validation(lib, entry):
    # passing every host check, the call reaches the device query; only run
    # where there is no device (the buffers here are not real)
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    at = dict(H=65536, d=128, Nq=1, Nk=1)
    st = {"fwd": lambda: call(**at), "bwd": lambda: call_bwd(**at),
          "kl": lambda: call_kl(**at),
          "proj": lambda: call_proj(H=65536, d=128, Nq=1, B=1, E=4)}[entry]()
    assert st == mha.MHA_ERR_DEVICE


def test_huge_sizes_are_rejected_without_overflow(lib):
    imax = 2**31 - 1
    assert call(B=imax, H=1, Nq=imax, Nk=imax) == mha.MHA_ERR_INVALID_ARG
    assert call(B=imax, H=65536, Nq=imax, Nk=imax, d=128) == mha.MHA_ERR_INVALID_ARG
    assert call_bwd(B=imax, H=2, Nq=imax, Nk=imax) == mha.MHA_ERR_INVALID_ARG
    assert call_kl(B=imax, H=4, Nq=imax, Nk=1) == mha.MHA_ERR_INVALID_ARG
    assert call_proj(B=imax, Nq=imax, H=imax, d=imax, E=imax) == mha.MHA_ERR_INVALID_ARG


# -------------------------------------------------- mha_fwd_splitkv_noalloc
def call_noalloc(**kw):
    a = dict(GOOD_SPLIT)
    a.update(kw)
    return mha.mha_fwd_splitkv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"],
                                       a["Nq"], a["Nk"], a["d"], a["causal"], a["scale"],
                                       a["n_splits"], a["stream"], a["dtype"])


def test_noalloc_refuses_a_workspace_over_the_scratch(lib):
    # 64 splits x 1*64*8 rows x (128 + 1) floats > 16 MiB (checked before any HIP call)
    assert mha.MHA_NOALLOC_SCRATCH_BYTES == 16 << 20
    st = call_noalloc(B=1, H=64, Nq=8, Nk=256, d=128, n_splits=64)
    assert st == mha.MHA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in mha.mha_status_string(st)


@pytest.mark.parametrize("kw,want", [
    (dict(q=0), mha.MHA_ERR_INVALID_ARG),
    (dict(n_splits=0), mha.MHA_ERR_INVALID_ARG),
    (dict(n_splits=257), mha.MHA_ERR_INVALID_ARG),
    (dict(Nq=9), mha.MHA_ERR_UNSUPPORTED),
    (dict(H=65537, d=128, Nq=1, Nk=1, n_splits=1), mha.MHA_ERR_INVALID_ARG),
], ids=lambda x: str(x))
def test_noalloc_validation_rejects(lib, kw, want):
    assert call_noalloc(**kw) == want


def test_noalloc_no_device_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert call_noalloc() == mha.MHA_ERR_DEVICE
    assert call_noalloc(B=0) == mha.MHA_OK
