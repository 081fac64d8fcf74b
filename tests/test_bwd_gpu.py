"""Parity of the HIP backward (mha_bwd, through the C ABI) with the fp64
oracle, on the GPU.

The kernel is given Q, K, V, dO and the oracle's O and LSE (rounded to the
I/O type and to fp32), so that its inputs are exact and known; its dQ, dK, dV
and D are then held to the per-element bound and the RMS bar of
tests/parity_bwd.py. Shapes cover ragged tiles, single rows and keys,
Nq != Nk with the causal mask, both head sizes and both types, and head
counts that take the XCD-grouped block order (B*H a multiple of 8). The named
workloads run at full size in one call; the oracle checks sampled heads
(and, for the 16k-token one, sampled rows and keys) while every other head
gets the GPU forward's O and LSE.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import workloads as wl
from parity_bwd import assert_bwd_parity, compare_head, head_reference, merge_stats, unit_roundoff
from ragged import case_id, ragged_cases

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


def to_dev(torch, bits: np.ndarray, dtype: str):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def to_bits(t) -> np.ndarray:
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def oracle_fwd_head(q, k, v, causal, scale, b, h, chunk=2048):
    """Oracle O [Nq, d] and LSE [Nq] of one head, in blocks of query rows."""
    Nq = q.shape[1]
    qs, ks, vs = (x[b:b + 1, :, h:h + 1] for x in (q, k, v))
    O = np.empty((Nq, q.shape[3]))
    L = np.empty(Nq)
    for r0 in range(0, Nq, chunk):
        rows = np.arange(r0, min(Nq, r0 + chunk))
        nk = min(k.shape[1], int(rows[-1]) + 1) if causal else k.shape[1]
        o, l = oracle.attention_fwd(qs, ks[:, :nk], vs[:, :nk], causal, scale, rows=rows)
        O[rows] = o[0, :, 0]
        L[rows] = l[0, 0]
    return O, L


def run_bwd(torch, mha, q, k, v, o, lse, g, dtype, causal, scale):
    """Raw mha_bwd on device tensors with NaN-prefilled outputs."""
    B, Nq, H, d = q.shape
    dq = torch.full_like(q, float("nan"))
    dk = torch.full_like(k, float("nan"))
    dv = torch.full_like(v, float("nan"))
    delta = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=q.device)
    dt = mha.MHA_DTYPE_BF16 if dtype == "bf16" else mha.MHA_DTYPE_FP16
    st = mha.mha_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), g.data_ptr(),
                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                     B, H, Nq, k.shape[1], d, int(causal), scale,
                     torch.cuda.current_stream().cuda_stream, dt)
    assert st == mha.MHA_OK, mha.mha_status_string(st)
    torch.cuda.synchronize()
    return to_bits(dq), to_bits(dk), to_bits(dv), delta.cpu().numpy()


def check_problem(torch, mha, qb, kb, vb, gb, dtype, causal, scale, heads=None, rows=None,
                  cols=None, label=""):
    """Run mha_bwd at the problem's full size and check ``heads`` (default all)."""
    B, Nq, H, d = qb.shape
    q, k, v, do = (wl.bits_to_f64(x, dtype) for x in (qb, kb, vb, gb))
    heads = [(b, h) for b in range(B) for h in range(H)] if heads is None else heads
    dq_, dk_, dv_, gd = (to_dev(torch, x, dtype) for x in (qb, kb, vb, gb))
    if len(heads) < B * H:
        # the heads the oracle does not check get the GPU forward's O and LSE
        o_dev, l_dev = mha.attention(dq_, dk_, dv_, causal=causal, scale=scale)
        torch.cuda.synchronize()
        o_bits, lse = to_bits(o_dev), l_dev.cpu().numpy()
    else:
        o_bits = np.zeros_like(qb)
        lse = np.zeros((B, H, Nq), np.float32)
    refs_in = {}
    for b, h in heads:
        O, L = oracle_fwd_head(q, k, v, causal, scale, b, h)
        o_bits[b, :, h] = wl.round_bits(O.astype(np.float32), dtype)
        lse[b, h] = L.astype(np.float32)
        refs_in[(b, h)] = (wl.bits_to_f64(o_bits[b, :, h], dtype), lse[b, h].astype(np.float64))
    o_dev = to_dev(torch, o_bits, dtype)
    l_dev = torch.from_numpy(np.ascontiguousarray(lse)).cuda()
    sys.__stderr__.write(f"[bwd] {label}: launching mha_bwd\n")
    sys.__stderr__.flush()
    gq, gk, gv, gD = run_bwd(torch, mha, dq_, dk_, dv_, o_dev, l_dev, gd, dtype, causal, scale)
    stats = []
    r_sel = np.arange(Nq) if rows is None else np.asarray(rows)
    c_sel = np.arange(kb.shape[1]) if cols is None else np.asarray(cols)
    for b, h in heads:
        o_in, l_in = refs_in[(b, h)]
        ref = head_reference(q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h], o_in, l_in, causal,
                             scale, dtype, rows, cols)
        got = {
            "dq": wl.bits_to_f64(gq[b, r_sel, h], dtype),
            "dk": wl.bits_to_f64(gk[b, c_sel, h], dtype),
            "dv": wl.bits_to_f64(gv[b, c_sel, h], dtype),
            "D": gD[b, h, r_sel].astype(np.float64),
        }
        stats.append(compare_head(ref, got))
    st = merge_stats(stats)
    # every output element was written (NaN prefill), also on unchecked heads
    for name, x in (("dq", gq), ("dk", gk), ("dv", gv)):
        assert np.all(np.isfinite(wl.bits_to_f32(x, dtype))), f"{label}: unwritten/non-finite {name}"
    assert np.all(np.isfinite(gD)), f"{label}: unwritten/non-finite D"
    u, _ = unit_roundoff(dtype)
    short = {g: (round(st[g]["worst_ratio"], 3),
                 round(st[g]["rms_err"] / max(u * st[g]["rms_ref"], 1e-300), 3)) for g in st}
    sys.__stderr__.write(f"[bwd-parity] {label}: (worst bound ratio, rms/u*rms_ref) {short}\n")
    sys.__stderr__.flush()
    assert_bwd_parity(st, dtype, label)
    return st, (gq, gk, gv, gD)


# -------------------------------------------------------------- edge shapes
SHAPES = [
    # B, H, Nq, Nk, d, dtype, causal
    (1, 1, 1, 1, 64, "fp16", False),
    (1, 1, 1, 1, 128, "bf16", True),
    (2, 3, 77, 131, 64, "bf16", False),
    (2, 3, 77, 131, 128, "fp16", True),    # Nk > Nq, causal: keys >= 77 get zero gradients
    (1, 2, 131, 77, 64, "fp16", True),     # Nq > Nk, causal
    (1, 2, 131, 77, 128, "bf16", False),
    (1, 1, 129, 129, 128, "bf16", True),   # one row past a block
    (1, 2, 200, 1, 64, "fp16", False),     # a single key
    (1, 2, 1, 300, 128, "bf16", False),    # a single query
    (3, 1, 63, 65, 64, "bf16", True),
    (1, 4, 256, 256, 128, "fp16", True),
    (1, 1, 513, 1000, 64, "bf16", True),
    (1, 8, 300, 300, 128, "bf16", True),   # B*H = 8: XCD-grouped order
    (2, 8, 200, 333, 64, "fp16", False),
    (1, 16, 257, 257, 128, "bf16", True),
    # the dK/dV kernel's three query-tile buffers: 2, 3 and 5 tiles of 32
    # queries per key block (runs shorter than, equal to and past one turn)
    (2, 1, 64, 64, 128, "fp16", True),
    (1, 2, 96, 96, 128, "bf16", True),     # wave 3's keys all past Nk
    (1, 1, 160, 160, 128, "bf16", False),
]


@pytest.mark.parametrize("case", SHAPES, ids=lambda c: "B{}H{}q{}k{}d{}{}{}".format(
    c[0], c[1], c[2], c[3], c[4], c[5], "c" if c[6] else ""))
def test_bwd_shapes(torch_mod, mha, case):
    B, H, Nq, Nk, d, dtype, causal = case
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed=300 + Nq + Nk)
    gb = wl.random_grad(B, H, Nq, d, dtype, seed=1300 + Nq + Nk)
    scale = float(np.float32(1 / math.sqrt(d)))
    st, (gq, gk, gv, _) = check_problem(torch_mod, mha, qb, kb, vb, gb, dtype, causal, scale,
                                        label=str(case))
    if causal and Nk > Nq:
        # keys no query sees: exactly zero
        assert not np.any(wl.bits_to_f32(gk[:, Nq:], dtype)) and not np.any(
            wl.bits_to_f32(gv[:, Nq:], dtype))


# 32-row query tiles and 32-key blocks (pairs of them at d = 128), 256-row
# workgroups
@pytest.mark.parametrize("case", ragged_cases(10, 4048, [32, 64, 96, 128, 160, 256], 600), ids=case_id)
def test_bwd_random_ragged_shapes(torch_mod, mha, case):
    B, H, Nq, Nk, d, dtype, causal = case
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed=8000 + 3 * Nq + Nk)
    gb = wl.random_grad(B, H, Nq, d, dtype, seed=9000 + 3 * Nq + Nk)
    scale = float(np.float32(1 / math.sqrt(d)))
    check_problem(torch_mod, mha, qb, kb, vb, gb, dtype, causal, scale, label=str(case))


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_bwd_peaky_scores(torch_mod, mha, dtype):
    """Large score spread (std 3 inputs, scale 0.25): P near one-hot."""
    qb, kb, _ = wl.random_inputs(1, 2, 300, 700, 64, dtype, seed=31, std=3.0)
    _, _, vb = wl.random_inputs(1, 2, 300, 700, 64, dtype, seed=32)
    gb = wl.random_grad(1, 2, 300, 64, dtype, seed=33)
    check_problem(torch_mod, mha, qb, kb, vb, gb, dtype, True, 0.25, label=f"peaky-{dtype}")


def test_bwd_uniform_scores_closed_form(torch_mod, mha):
    """Q = 0: P_ij = 1/n_i, so dV_j = sum over the rows i that see j of dO_i / n_i."""
    B, H, N, d, dtype = 1, 2, 190, 64, "fp16"
    _, kb, vb = wl.random_inputs(B, H, N, N, d, dtype, seed=34)
    qb = np.zeros_like(kb)
    gb = wl.random_grad(B, H, N, d, dtype, seed=35)
    _, (_, _, gv, _) = check_problem(torch_mod, mha, qb, kb, vb, gb, dtype, True, 0.125,
                                     label="uniform")
    do = wl.bits_to_f64(gb, dtype)
    want = np.cumsum((do / np.arange(1, N + 1)[None, :, None, None])[:, ::-1], axis=1)[:, ::-1]
    assert np.abs(wl.bits_to_f64(gv, dtype) - want).max() <= 1e-2


# ---------------------------------------------------- full-size workloads
WORKLOAD_HEADS = {
    "tiny": None,
    "encoder_self": [(0, 0), (3, 7), (7, 15)],
    "decoder_causal": [(0, 0), (2, 17), (3, 31)],
    "cross": [(0, 0), (9, 4), (15, 15)],
    "long_causal": [(0, 0), (0, 5)],
}


def _sample(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    s = set(range(min(n, 40))) | set(range(max(0, n - 16), n))
    for t in (127, 128, 129, 255, 256, 1023, 1024, n // 2, n // 2 + 1):
        if 0 <= t < n:
            s.add(t)
    s |= set(rng.choice(n, size=min(n, 120), replace=False).tolist())
    return np.array(sorted(s))


@pytest.mark.parametrize("name", list(wl.WORKLOADS))
def test_bwd_workload(torch_mod, mha, name):
    w = wl.WORKLOADS[name]
    qb, kb, vb = wl.make_inputs(w)
    gb = wl.make_grad(w)
    rows = cols = None
    if w.Nq * w.Nk > 2 ** 26:
        rows, cols = _sample(w.Nq, 1), _sample(w.Nk, 2)
    check_problem(torch_mod, mha, qb, kb, vb, gb, w.dtype, w.causal, w.scale,
                  heads=WORKLOAD_HEADS[name], rows=rows, cols=cols, label=name)


# ------------------------------------------------------------ end to end
# plus seeded ragged shapes; the RMS bar needs nonzero reference gradients,
# so one query or one key (where dS is zero in exact arithmetic) is left out
@pytest.mark.parametrize("case", [(2, 4, 333, 333, 128, "bf16", True),
                                  (1, 8, 200, 450, 64, "fp16", False)] +
                         [c for c in ragged_cases(8, 4049, [32, 64, 96, 128, 160, 256], 600)
                          if c[2] > 1 and c[3] > 1], ids=case_id)
def test_bwd_after_gpu_forward(torch_mod, mha, case):
    """The GPU forward's O and LSE feed the GPU backward. The element bound
    needs the exact deviation of the kernel's inputs, which here come from the
    forward kernel, so only the RMS bar (which does not) is applied."""
    torch = torch_mod
    B, H, Nq, Nk, d, dtype, causal = case
    qb, kb, vb = wl.random_inputs(B, H, Nq, Nk, d, dtype, seed=400 + Nq)
    gb = wl.random_grad(B, H, Nq, d, dtype, seed=1400 + Nq)
    scale = float(np.float32(1 / math.sqrt(d)))
    q_, k_, v_, g_ = (to_dev(torch, x, dtype) for x in (qb, kb, vb, gb))
    o_, l_ = mha.attention(q_, k_, v_, causal=causal, scale=scale)
    gq, gk, gv, _ = run_bwd(torch, mha, q_, k_, v_, o_, l_, g_, dtype, causal, scale)
    dq, dk, dv, _ = oracle.attention_bwd(*(wl.bits_to_f64(x, dtype) for x in (qb, kb, vb, gb)),
                                         causal, scale)
    u, _ = unit_roundoff(dtype)
    for name, got, ref in (("dq", gq, dq), ("dk", gk, dk), ("dv", gv, dv)):
        g = wl.bits_to_f64(got, dtype)
        assert np.all(np.isfinite(g)), name
        rms_err = float(np.sqrt(((g - ref) ** 2).mean()))
        rms_ref = float(np.sqrt((ref ** 2).mean()))
        assert rms_err <= 4 * u * rms_ref, (name, rms_err, rms_ref)


# -------------------------------------------------------- structural checks
def test_bwd_deterministic(torch_mod, mha):
    """No atomics: two calls give identical bits."""
    torch = torch_mod
    B, H, N, d, dtype = 2, 8, 300, 128, "bf16"
    qb, kb, vb = wl.random_inputs(B, H, N, N, d, dtype, seed=41)
    gb = wl.random_grad(B, H, N, d, dtype, seed=42)
    q_, k_, v_, g_ = (to_dev(torch, x, dtype) for x in (qb, kb, vb, gb))
    o_, l_ = mha.attention(q_, k_, v_, causal=True, scale=0.09)
    a = run_bwd(torch, mha, q_, k_, v_, o_, l_, g_, dtype, True, 0.09)
    b = run_bwd(torch, mha, q_, k_, v_, o_, l_, g_, dtype, True, 0.09)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_runs_on_a_side_stream(torch_mod, mha):
    torch = torch_mod
    B, H, N, d, dtype = 1, 2, 150, 64, "fp16"
    qb, kb, vb = wl.random_inputs(B, H, N, N, d, dtype, seed=43)
    gb = wl.random_grad(B, H, N, d, dtype, seed=44)
    q_, k_, v_, g_ = (to_dev(torch, x, dtype) for x in (qb, kb, vb, gb))
    o_, l_ = mha.attention(q_, k_, v_, causal=False, scale=0.125)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        gq, gk, gv, D = mha.attention_backward(q_, k_, v_, o_, l_, g_, causal=False, scale=0.125)
    s.synchronize()
    ref = run_bwd(torch, mha, q_, k_, v_, o_, l_, g_, dtype, False, 0.125)
    for x, y in zip((to_bits(gq), to_bits(gk), to_bits(gv), D.cpu().numpy()), ref):
        assert np.array_equal(x, y)


def test_bwd_error_paths_raise(torch_mod, mha):
    torch = torch_mod
    q = torch.zeros((1, 8, 1, 96), dtype=torch.float16, device="cuda")
    lse = torch.zeros((1, 1, 8), dtype=torch.float32, device="cuda")
    with pytest.raises(mha.MhaError) as e:
        mha.attention_backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone())
    assert e.value.status == mha.MHA_ERR_UNSUPPORTED
    q = torch.zeros((1, 8, 1, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(mha.MhaError) as e:
        mha.attention_backward(q, q.clone(), q.clone(), q.clone(), lse, q.clone(), scale=-1.0)
    assert e.value.status == mha.MHA_ERR_INVALID_ARG
