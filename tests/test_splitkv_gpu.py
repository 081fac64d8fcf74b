"""Parity of the split-over-keys forward (mha_fwd_splitkv, through the C ABI)
with the fp64 oracle, on the GPU, under the forward's bar (tests/parity.py).

Shapes cover 1..8 query rows, key counts around the 256-key split block and
the per-workgroup step (1, 7, 255, 256, 257, 1000, 5000), both head sizes and
types, the causal mask (top-left: row i sees keys 0..i), one split, the
default split count and more splits than key blocks (empty splits), the
decoding workloads at full size, a workspace reused across calls, and the
error path for Nq > 8.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_parity, compare, report

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _announce(request):
    sys.__stderr__.write(f"\n[gpu-case] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield


@pytest.fixture(scope="module")
def torch_mod():
    import torch
    assert torch.cuda.is_available()
    return torch


@pytest.fixture(scope="module")
def mha(torch_mod):
    import head_attention_mha_amd as m
    m.load_library()
    return m


def to_dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def to_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_split(torch, mha, qb, kb, vb, dtype, causal, scale, n_splits, ws=None):
    """Raw mha_fwd_splitkv with NaN-prefilled outputs (and workspace)."""
    q, k, v = (to_dev(torch, x, dtype) for x in (qb, kb, vb))
    B, Nq, H, d = q.shape
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    if ws is None:
        o_part = torch.full((n_splits, B, H, Nq, d), float("nan"), dtype=torch.float32,
                            device=q.device)
        lse_part = torch.full((n_splits, B, H, Nq), float("nan"), dtype=torch.float32,
                              device=q.device)
    else:
        o_part, lse_part = ws
    dt = mha.MHA_DTYPE_BF16 if dtype == "bf16" else mha.MHA_DTYPE_FP16
    st = mha.mha_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                             lse.data_ptr(), B, H, Nq, k.shape[1], d, int(causal), scale,
                             n_splits, o_part.data_ptr(), lse_part.data_ptr(),
                             torch.cuda.current_stream().cuda_stream, dt)
    assert st == mha.MHA_OK, mha.mha_status_string(st)
    torch.cuda.synchronize()
    return to_bits(o), lse.cpu().numpy()


def check(torch, mha, qb, kb, vb, dtype, causal, scale, n_splits, label, ws=None):
    o_bits, lse = run_split(torch, mha, qb, kb, vb, dtype, causal, scale, n_splits, ws)
    assert np.all(np.isfinite(wl.bits_to_f32(o_bits, dtype))), f"{label}: unwritten/non-finite O"
    assert np.all(np.isfinite(lse)), f"{label}: unwritten/non-finite LSE"
    O_ref, L_ref = oracle.attention_fwd(*(wl.bits_to_f64(x, dtype) for x in (qb, kb, vb)),
                                        causal, scale)
    st = compare(o_bits, lse, O_ref, L_ref, dtype)
    sys.__stderr__.write(f"[splitkv-parity] {report(st, label)}\n")
    assert_parity(st, label)
    return st


SHAPES = [
    # B, H, Nq, Nk, d, dtype, causal, n_splits (None: default)
    (1, 1, 1, 1, 64, "fp16", False, None),
    (1, 1, 1, 1, 128, "bf16", True, 1),
    (2, 3, 1, 7, 128, "bf16", False, 4),      # more splits than keys: empty splits
    (2, 3, 2, 255, 64, "fp16", False, None),
    (1, 4, 3, 256, 128, "bf16", True, 2),
    (1, 4, 4, 257, 64, "bf16", False, 3),
    (3, 2, 5, 1000, 128, "fp16", True, None),
    (2, 2, 8, 1000, 64, "fp16", False, 1),
    (1, 2, 8, 5000, 128, "bf16", False, 7),
    (2, 8, 1, 5000, 64, "bf16", True, 16),    # causal decode row 0: key 0 only
    (1, 8, 6, 4097, 128, "fp16", False, 256),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}H{}q{}k{}d{}{}{}s{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "c" if c[6] else "", c[7]))
def test_splitkv_shapes(torch_mod, mha, case):
    B, H, Nq, Nk, d, dtype, causal, n_splits = case
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed=500 + Nq + Nk)
    scale = float(np.float32(1 / math.sqrt(d)))
    if n_splits is None:
        n_splits = mha.mha_fwd_splitkv_splits(B, H, Nq, Nk)
    check(torch_mod, mha, qb, kb, vb, dtype, causal, scale, n_splits, str(case))


def _random_split_cases(n=10, seed=5096):
    """Seeded decode shapes: Nq in 1..8, Nk on or next to a power-of-two
    tile edge or anywhere below 6000, the split count drawn (empty splits
    included) or left to the library."""
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        if rng.random() < 0.5:
            nk = int(rng.choice([64, 256, 1024, 4096])) + int(rng.integers(-1, 2))
        else:
            nk = int(rng.integers(1, 6000))
        splits = None if rng.random() < 0.4 else int(rng.integers(1, 65))
        cases.append((int(rng.integers(1, 3)), int(rng.integers(1, 5)), int(rng.integers(1, 9)), nk,
                      int(rng.choice([64, 128])), str(rng.choice(["fp16", "bf16"])),
                      bool(rng.random() < 0.5), splits))
    return cases


@pytest.mark.parametrize("case", _random_split_cases(), ids=lambda c: "B{}H{}q{}k{}d{}{}{}s{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "c" if c[6] else "", c[7]))
def test_splitkv_random_shapes(torch_mod, mha, case):
    B, H, Nq, Nk, d, dtype, causal, n_splits = case
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed=11000 + 3 * Nq + Nk)
    scale = float(np.float32(1 / math.sqrt(d)))
    if n_splits is None:
        n_splits = mha.mha_fwd_splitkv_splits(B, H, Nq, Nk)
    check(torch_mod, mha, qb, kb, vb, dtype, causal, scale, n_splits, str(case))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_splitkv_peaky_scores(torch_mod, mha, dtype):
    """Std-3 queries and keys at scale 0.25 make rows near one-hot, and the
    largest score sits in a different split for each row."""
    qb, kb, _ = wl.random_inputs(2, 2, 4, 3000, 64, dtype, seed=51, std=3.0)
    _, _, vb = wl.random_inputs(2, 2, 4, 3000, 64, dtype, seed=52)
    check(torch_mod, mha, qb, kb, vb, dtype, False, 0.25, 12, f"peaky-{dtype}")


@pytest.mark.parametrize("name", list(wl.DECODE_WORKLOADS))
def test_splitkv_decode_workloads(torch_mod, mha, name):
    w = wl.DECODE_WORKLOADS[name]
    qb, kb, vb = wl.make_inputs(w)
    n = mha.mha_fwd_splitkv_splits(w.B, w.H, w.Nq, w.Nk)
    check(torch_mod, mha, qb, kb, vb, w.dtype, w.causal, w.scale, n, name)


def test_splitkv_matches_whole_forward_closely(torch_mod, mha):
    """The two forwards agree with each other to within the output rounding
    (both are within the bar of the oracle; here they are compared directly)."""
    torch = torch_mod
    B, H, Nq, Nk, d, dtype = 2, 4, 3, 3000, 128, "bf16"
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed=53)
    o_s, l_s = run_split(torch, mha, qb, kb, vb, dtype, False, 0.088, 10)
    q, k, v = (to_dev(torch, x, dtype) for x in (qb, kb, vb))
    o_w, l_w = mha.attention(q, k, v, causal=False, scale=0.088)
    torch.cuda.synchronize()
    Os, Ow = wl.bits_to_f64(o_s, dtype), wl.bits_to_f64(to_bits(o_w), dtype)
    assert np.abs(Os - Ow).max() <= 2 * 2 ** -8 * max(1.0, np.abs(Ow).max())
    assert np.abs(l_s - l_w.cpu().numpy()).max() <= 1e-4


def test_splitkv_workspace_reused(torch_mod, mha):
    """One workspace serves a larger call and then a smaller one."""
    torch = torch_mod
    ws = (torch.full((16, 2, 4, 8, 128), float("nan"), dtype=torch.float32, device="cuda"),
          torch.full((16, 2, 4, 8), float("nan"), dtype=torch.float32, device="cuda"))
    qb, kb, vb = wl.random_inputs(2, 4, 8, 4000, 128, "bf16", seed=54)
    check(torch, mha, qb, kb, vb, "bf16", False, 0.088, 16, "ws-big", ws)
    qb, kb, vb = wl.random_inputs(1, 2, 3, 900, 64, "fp16", seed=55)
    check(torch, mha, qb, kb, vb, "fp16", True, 0.125, 5, "ws-small", ws)


def test_splitkv_binding_and_errors(torch_mod, mha):
    torch = torch_mod
    qb, kb, vb = wl.random_inputs(1, 2, 2, 600, 64, "fp16", seed=56)
    q, k, v = (to_dev(torch, x, "fp16") for x in (qb, kb, vb))
    o, lse = mha.attention_splitkv(q, k, v, causal=False, scale=0.125)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_fwd(*(wl.bits_to_f64(x, "fp16") for x in (qb, kb, vb)),
                                        False, 0.125)
    assert_parity(compare(to_bits(o), lse.cpu().numpy(), O_ref, L_ref, "fp16"), "binding")
    q9 = torch.zeros((1, 9, 2, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(mha.MhaError) as e:
        mha.attention_splitkv(q9, k, v)
    assert e.value.status == mha.MHA_ERR_UNSUPPORTED
