"""mha_fwd_splitkv_noalloc (the split-KV forward on the library's fixed
per-GPU scratch, no allocation) against mha_fwd_splitkv with a caller
workspace, through the C ABI: two calls in a row, the second smaller, both
equal bit for bit to the workspace entry point's results (same kernels, same
splits) and both within the forward's parity bars against the fp64 oracle;
a problem too large for the scratch is refused and writes nothing."""
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from parity import assert_parity, compare, report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    assert torch.cuda.is_available()
    import head_attention_mha_amd as mha
    mha.load_library()
    return torch, mha


def _dev(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _bits(torch, t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _run_both(torch, mha, B, H, Nq, Nk, d, dtype, causal, seed):
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed)
    q, k, v = (_dev(torch, x, dtype) for x in (qb, kb, vb))
    scale = float(np.float32(1 / np.sqrt(d)))
    n_splits = mha.mha_fwd_splitkv_splits(B, H, Nq, Nk)
    dt = mha.MHA_DTYPE_BF16 if dtype == "bf16" else mha.MHA_DTYPE_FP16
    stream = torch.cuda.current_stream().cuda_stream
    outs = []
    for noalloc in (True, False):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
        if noalloc:
            st = mha.mha_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             o.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                                             int(causal), scale, n_splits, stream, dt)
        else:
            o_part = torch.empty((n_splits, B, H, Nq, d), dtype=torch.float32, device=q.device)
            l_part = torch.empty((n_splits, B, H, Nq), dtype=torch.float32, device=q.device)
            st = mha.mha_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), B, H, Nq, Nk, d, int(causal), scale,
                                     n_splits, o_part.data_ptr(), l_part.data_ptr(), stream, dt)
        assert st == mha.MHA_OK, mha.mha_status_string(st)
        torch.cuda.synchronize()
        outs.append((_bits(torch, o), lse.cpu().numpy()))
    (o_na, l_na), (o_ws, l_ws) = outs
    assert np.array_equal(o_na, o_ws), "O differs from the workspace entry point"
    assert np.array_equal(l_na.view(np.uint32), l_ws.view(np.uint32)), "LSE differs"
    O_ref, L_ref = oracle.attention_fwd(*(wl.bits_to_f64(x, dtype) for x in (qb, kb, vb)),
                                        causal, scale)
    st = compare(o_na, l_na, O_ref, L_ref, dtype)
    label = f"noalloc B{B} H{H} Nq{Nq} Nk{Nk} d{d} {dtype}{' causal' if causal else ''}"
    sys.__stderr__.write(f"[noalloc] {report(st, label)}\n")
    assert_parity(st, label)


def test_two_calls_second_smaller(env):
    torch, mha = env
    # the decode workload's shape, then a smaller ragged one with a mask
    _run_both(torch, mha, 1, 32, 1, 32768, 128, "bf16", False, seed=5)
    _run_both(torch, mha, 2, 3, 3, 1000, 64, "fp16", True, seed=11)


def test_too_large_for_the_scratch_is_refused(env):
    torch, mha = env
    # 64 splits x 512 rows x (128 + 1) floats: just over 16 MiB
    B, H, Nq, Nk, d, n_splits = 1, 64, 8, 256, 128, 64
    need = n_splits * B * H * Nq * (d + 1) * 4
    assert need > mha.MHA_NOALLOC_SCRATCH_BYTES
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, "bf16", seed=13)
    q, k, v = (_dev(torch, x, "bf16") for x in (qb, kb, vb))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device="cuda")
    st = mha.mha_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), B, H, Nq, Nk, d, 0, 0.088, n_splits,
                                     torch.cuda.current_stream().cuda_stream, mha.MHA_DTYPE_BF16)
    assert st == mha.MHA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in mha.mha_status_string(st)
    torch.cuda.synchronize()
    assert torch.isnan(o.float()).all() and torch.isnan(lse).all()
    # one split fewer fits (63 x 512 x 129 x 4 bytes < 16 MiB) and runs
    st = mha.mha_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                     lse.data_ptr(), B, H, Nq, Nk, d, 0, 0.088, n_splits - 1,
                                     torch.cuda.current_stream().cuda_stream, mha.MHA_DTYPE_BF16)
    assert st == mha.MHA_OK
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()


def test_binding_writes_into_the_given_outputs(env):
    torch, mha = env
    qb, kb, vb = wl.random_inputs(1, 4, 2, 3000, 64, "fp16", seed=12)
    q, k, v = (_dev(torch, x, "fp16") for x in (qb, kb, vb))
    o = torch.empty_like(q)
    lse = torch.empty((1, 4, 2), dtype=torch.float32, device="cuda")
    r = mha.attention_splitkv_noalloc(q, k, v, o, lse)
    assert r[0] is o and r[1] is lse
    ref = mha.attention_splitkv(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o, ref[0]) and torch.equal(lse, ref[1])
