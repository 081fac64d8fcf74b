"""Benchmark of the fused MHA forward (default) or backward on one MI355X.

A step is one mha_fwd call (``--pass fwd``) or one mha_bwd call (``--pass
bwd``: D, dQ and dK/dV, from the forward's O and LSE computed beforehand)
over the whole workload, inputs already resident in HBM. Default workload:
B=1, H=8, Nq=Nk=16384, d=128, bf16, causal (the long-sequence small-batch
regime of the FlashAttention long-sequence post). Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                  [--pass fwd|bwd] [--no-cpu-baseline] [--cpu-seconds S]
                  [--calib-copy-mib M]
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of MFMA bf16 peak (B=1,H=8,N=16k,d=128 causal)"
METRIC_BWD = ("attention bwd TFLOP/s (5-matmul count 10*B*H*Nq*Nk*d, halved causal) and % of "
              "MFMA bf16 peak")
PEAK_TFLOPS = 2500.0  # MI355X published dense bf16/fp16 MFMA peak
PEAK_GBS = 8000.0     # MI355X published HBM3E bandwidth
METRIC_KL = ("attention KL(P1||P2) forward TFLOP/s (two QK^T products, 4*B*H*Nq*Nk*d, halved "
             "causal) and % of MFMA bf16 peak")
METRIC_PROJ = ("output projection (head concat then O W^T + b) TFLOP/s, 2*B*Nq*H*d*E, and % of "
               "MFMA bf16 peak")
METRIC_SPLIT = ("attention decode forward (split over keys) HBM GB/s: Q, K, V read and O, LSE "
                "written once, per second")
_CSRC = os.path.join(ROOT, "head_attention_mha_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in
                  ("mha_common.hpp", "mha_fwd_kernel.hpp", "mha_fwd.hip")]
KERNEL_SOURCES_SPLIT = [os.path.join(_CSRC, f) for f in
                        ("mha_common.hpp", "mha_fwd_kernel.hpp", "mha_split_kernel.hpp",
                         "mha_splitkv.hip")]
KERNEL_SOURCES_BWD = [os.path.join(_CSRC, f) for f in
                      ("mha_common.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp",
                       "mha_bwd_kernel.hpp", "mha_bwd.hip")]
KERNEL_SOURCES_PROJ = [os.path.join(_CSRC, f) for f in
                       ("mha_common.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp",
                        "mha_proj_kernel.hpp", "mha_proj.hip")]
KERNEL_SOURCES_KL = [os.path.join(_CSRC, f) for f in
                     ("mha_common.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp", "mha_kl_kernel.hpp",
                      "mha_kl.hip")]


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources with comments and whitespace removed, so
    that editing a comment does not invalidate counters taken on the code."""
    h = hashlib.sha256()
    for p in sources or KERNEL_SOURCES:
        text = open(p, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def hbm_traffic(workload: str, which: str = "fwd"):
    """Per-launch HBM bytes (FETCH + WRITE) from the committed counter summary,
    or None when there is none or the kernel sources changed since."""
    name = f"hbm_traffic_{workload}.txt" if which == "fwd" else f"hbm_traffic_{which}_{workload}.txt"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    srcs = {"fwd": KERNEL_SOURCES, "bwd": KERNEL_SOURCES_BWD, "splitkv": KERNEL_SOURCES_SPLIT,
            "kl": KERNEL_SOURCES_KL, "proj": KERNEL_SOURCES_PROJ}[which]
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(srcs):
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def to_device(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def cpu_baseline(w: wl.Workload, qb, kb, vb, target_s: float) -> dict:
    """The fp64 oracle, as it stands, on evenly spaced query rows of every head."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = sum(int(i.get("num_threads", 1)) for i in threadpool_info()
                      if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v = (wl.bits_to_f64(x, w.dtype) for x in (qb, kb, vb))

    def timed(rows):
        t0 = time.perf_counter()
        oracle.attention_fwd(q, k, v, w.causal, w.scale, rows=rows)
        return time.perf_counter() - t0

    pilot = np.unique(np.linspace(0, w.Nq - 1, 16).astype(np.int64))
    t_p = max(timed(pilot), 1e-6)
    n = int(min(w.Nq, max(16, len(pilot) * target_s / t_p)))
    rows = np.unique(np.linspace(0, w.Nq - 1, n).astype(np.int64))
    t = timed(rows)
    vis = (rows + 1).clip(max=w.Nk) if w.causal else np.full(len(rows), w.Nk)
    flops = 4.0 * w.d * float(vis.sum()) * w.B * w.H
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(rows)} evenly spaced query rows of each of the {w.B * w.H} heads "
                   f"({len(rows) / w.Nq:.1%} of the rows, all their keys), fp64 NumPy, "
                   f"{t:.1f} s; FLOPs counted as 4*d*visible keys per row"),
        "seconds": t,
    }


def cpu_baseline_kl(w: wl.Workload, q1b, k1b, q2b, k2b, target_s: float) -> dict:
    """The fp64 KL oracle, as it stands, on evenly spaced query rows of every
    head (all keys), sized to about ``target_s``."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = sum(int(i.get("num_threads", 1)) for i in threadpool_info()
                      if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        threads = 1
    x = [wl.bits_to_f64(a, w.dtype) for a in (q1b, k1b, q2b, k2b)]

    def timed(rows):
        t0 = time.perf_counter()
        oracle.attention_kl(*x, w.causal, w.scale, rows=rows)
        return time.perf_counter() - t0

    pilot = np.unique(np.linspace(0, w.Nq - 1, 16).astype(np.int64))
    t_p = max(timed(pilot), 1e-6)
    n = int(min(w.Nq, max(16, len(pilot) * target_s / t_p)))
    rows = np.unique(np.linspace(0, w.Nq - 1, n).astype(np.int64))
    t = timed(rows)
    vis = (rows + 1).clip(max=w.Nk) if w.causal else np.full(len(rows), w.Nk)
    flops = 4.0 * w.d * float(vis.sum()) * w.B * w.H
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{len(rows)} evenly spaced query rows of each of the {w.B * w.H} heads "
                   f"({len(rows) / w.Nq:.1%} of the rows, all their keys), fp64 NumPy, "
                   f"{t:.1f} s; FLOPs counted as 4*d*visible keys per row"),
        "seconds": t,
    }


def cpu_baseline_split(w: wl.Workload, qb, kb, vb, target_s: float) -> dict:
    """The fp64 split-over-keys oracle, as it stands, on whole batch entries
    of the workload (all their heads), doubling their number until the run
    takes about a quarter of ``target_s`` or covers the workload."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = sum(int(i.get("num_threads", 1)) for i in threadpool_info()
                      if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        threads = 1
    n_splits = max(1, min(256, -(-w.Nk // 2048)))
    bounds = np.linspace(0, w.Nk, n_splits + 1).astype(np.int64)

    def timed(nb):
        q, k, v = (wl.bits_to_f64(x[:nb], w.dtype) for x in (qb, kb, vb))
        t0 = time.perf_counter()
        oracle.attention_fwd_split(q, k, v, w.causal, w.scale, bounds)
        return time.perf_counter() - t0

    nb = 1
    t = timed(nb)
    while nb < w.B and t < target_s / 4:
        nb = min(w.B, 2 * nb)
        t = timed(nb)
    bytes_ = nb * w.H * ((2 * w.Nq + 2 * w.Nk) * w.d * 2 + 4 * w.Nq)
    return {
        "value": bytes_ / t / 1e9,
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"batch entries 0..{nb - 1} ({nb} of {w.B}, all {w.H} heads), {n_splits} key "
                   f"splits, fp64 NumPy, {t:.2f} s; bytes counted as for the GPU line"),
        "seconds": t,
    }


def cpu_baseline_bwd(w: wl.Workload, qb, kb, vb, gb, target_s: float) -> dict:
    """The fp64 backward oracle, as it stands, on a bounded sample.

    The sample is the first n tokens (queries and keys) of the first m heads
    of batch entry 0: a prefix of a sequence is a complete problem of the
    same kind (causal stays causal). n grows until one head takes about a
    quarter of ``target_s`` or covers the whole sequence; then whole heads
    are added while the time stays within ``target_s``."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = sum(int(i.get("num_threads", 1)) for i in threadpool_info()
                      if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        threads = 1
    q, k, v, do = (wl.bits_to_f64(x[:1], w.dtype) for x in (qb, kb, vb, gb))

    def timed(n, m):
        nk = n if w.Nq == w.Nk else w.Nk
        t0 = time.perf_counter()
        oracle.attention_bwd(q[:, :n, :m], k[:, :nk, :m], v[:, :nk, :m], do[:, :n, :m],
                             w.causal, w.scale)
        return time.perf_counter() - t0, nk

    n, m = min(w.Nq, 256), 1
    t, nk = timed(n, m)
    while n < w.Nq and t < target_s / 4:
        n = min(w.Nq, int(n * 1.6))
        t, nk = timed(n, m)
    if n == w.Nq and w.H > 1:
        m = int(max(1, min(w.H, target_s / max(t, 1e-6))))
        if m > 1:
            t, nk = timed(n, m)
    flops = 10.0 * n * nk * w.d * m / (2.0 if w.causal else 1.0)
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"the first {n} queries and {nk} keys of heads 0..{m - 1} of batch entry 0, "
                   f"fp64 NumPy, {t:.1f} s; FLOPs counted as for the GPU line"),
        "seconds": t,
    }


def calib_copy(torch, mib: int, device) -> None:
    """Three plain device-to-device copies of ``mib`` MiB: a hardware counter
    of bytes read or written, taken over the same run, is scaled by what it
    reads for these copies of known size."""
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device=device)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"calibration copy: {n * 2} bytes read, {n * 2} bytes written per launch",
          file=sys.stderr, flush=True)


def bench_proj(args, torch, mha, w) -> int:
    """The output-projection pass (its own workload type: O, W, bias)."""
    ob, wb, bb = wl.make_proj_inputs(w)
    o, wt, b = (to_device(torch, x, w.dtype) for x in (ob, wb, bb))
    y = torch.empty((w.B, w.Nq, w.E), dtype=o.dtype, device=o.device)
    stream = torch.cuda.current_stream()
    dt = mha.MHA_DTYPE_BF16 if w.dtype == "bf16" else mha.MHA_DTYPE_FP16
    argv = (o.data_ptr(), wt.data_ptr(), b.data_ptr(), y.data_ptr(), w.B, w.Nq, w.H, w.d, w.E,
            stream.cuda_stream, dt)

    def step():
        st = mha.mha_out_proj(*argv)
        if st != mha.MHA_OK:
            raise mha.MhaError(st, "mha_out_proj")

    if args.calib_copy_mib:
        calib_copy(torch, args.calib_copy_mib, o.device)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])
    ms = ev[0].elapsed_time(ev[K]) / K
    tflops = w.flops / (ms * 1e-3) / 1e12
    achieved = w.flops / (per.mean() * 1e-3) / 1e12
    line = {
        "metric": METRIC_PROJ, "value": round(tflops, 2), "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS, 2), "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "pass": "proj", "B": w.B, "Nq": w.Nq, "H": w.H, "d": w.d,
                   "E": w.E, "io_dtype": w.dtype, "accumulate": "fp32", "flops_per_step": w.flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": hbm_traffic(w.name, "proj"), "kernel": "mha_proj_kernel",
                     "launch_ms": {"mean": round(float(per.mean()), 5),
                                   "median": round(float(np.median(per)), 5),
                                   "min": round(float(per.min()), 5)}},
        "timed_wall_s": round(wall, 3),
        "kernel_source_sha256_16": kernel_source_hash(KERNEL_SOURCES_PROJ),
        "device": torch.cuda.get_device_name(0),
    }
    if not args.no_cpu_baseline:
        print("bench.py: timing the fp64 oracle on the host (cpu_baseline) ...", file=sys.stderr,
              flush=True)
        line["cpu_baseline"] = cpu_baseline_proj(w, ob, wb, bb, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_proj(w, ob, wb, bb, target_s: float) -> dict:
    """The fp64 projection oracle, as it stands, on leading token rows."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = sum(int(i.get("num_threads", 1)) for i in threadpool_info()
                      if i.get("user_api") == "blas") or 1
    except Exception:  # pragma: no cover
        threads = 1
    wt, b = wl.bits_to_f64(wb, w.dtype), wl.bits_to_f64(bb, w.dtype)
    x = ob.reshape(w.B * w.Nq, w.H, w.d)

    def timed(n):
        o = wl.bits_to_f64(x[:n], w.dtype)[None]
        t0 = time.perf_counter()
        oracle.out_proj(o, wt, b)
        return time.perf_counter() - t0

    n = min(w.B * w.Nq, 256)
    t = timed(n)
    while n < w.B * w.Nq and t < target_s / 4:
        n = min(w.B * w.Nq, 2 * n)
        t = timed(n)
    flops = 2.0 * n * w.H * w.d * w.E
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": (f"the first {n} of {w.B * w.Nq} token rows, fp64 NumPy matmul, {t:.2f} s"),
            "seconds": t}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None,
                    choices=(list(wl.WORKLOADS) + list(wl.DECODE_WORKLOADS) + list(wl.KL_WORKLOADS)
                             + list(wl.PROJ_WORKLOADS)),
                    help="default: long_causal (fwd, bwd), decode (splitkv), kl_long (kl), "
                         "proj_long (proj)")
    ap.add_argument("--pass", dest="which", default="fwd",
                    choices=["fwd", "bwd", "splitkv", "kl", "proj"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this size (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards over heads with no communication; see DESIGN.md)",
              file=sys.stderr)
        return 2

    import torch

    import head_attention_mha_amd as mha

    if not torch.cuda.is_available():
        print("bench.py: no GPU available", file=sys.stderr)
        return 1
    mha.load_library()
    name = args.workload or {"splitkv": "decode", "kl": "kl_long",
                             "proj": "proj_long"}.get(args.which, "long_causal")
    if args.which == "proj":
        return bench_proj(args, torch, mha, wl.PROJ_WORKLOADS[name])
    w = wl.WORKLOADS.get(name) or wl.DECODE_WORKLOADS.get(name) or wl.KL_WORKLOADS[name]
    if args.which == "kl":
        qb, kb, q2b, k2b = wl.make_kl_inputs(w)
        vb = kb  # unused by the KL step
    else:
        qb, kb, vb = wl.make_inputs(w)
    q, k, v = (to_device(torch, x, w.dtype) for x in (qb, kb, vb))
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=q.device)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    dt = mha.MHA_DTYPE_BF16 if w.dtype == "bf16" else mha.MHA_DTYPE_FP16
    argv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
            w.B, w.H, w.Nq, w.Nk, w.d, int(w.causal), w.scale, sp, dt)

    def fwd_step():
        st = mha.mha_fwd(*argv)
        if st != mha.MHA_OK:
            raise mha.MhaError(st)

    step = fwd_step
    if args.which == "bwd":
        gb = wl.make_grad(w)
        g = to_device(torch, gb, w.dtype)
        fwd_step()  # O and LSE the backward starts from (not timed)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        delta = torch.empty_like(lse)
        bargv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), g.data_ptr(),
                 lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                 w.B, w.H, w.Nq, w.Nk, w.d, int(w.causal), w.scale, sp, dt)

        def bwd_step():
            st = mha.mha_bwd(*bargv)
            if st != mha.MHA_OK:
                raise mha.MhaError(st, "mha_bwd")

        step = bwd_step
    elif args.which == "splitkv":
        n_splits = mha.mha_fwd_splitkv_splits(w.B, w.H, w.Nq, w.Nk)
        o_part = torch.empty((n_splits, w.B, w.H, w.Nq, w.d), dtype=torch.float32, device=q.device)
        lse_part = torch.empty((n_splits, w.B, w.H, w.Nq), dtype=torch.float32, device=q.device)
        sargv = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                 w.B, w.H, w.Nq, w.Nk, w.d, int(w.causal), w.scale, n_splits,
                 o_part.data_ptr(), lse_part.data_ptr(), sp, dt)

        def split_step():
            st = mha.mha_fwd_splitkv(*sargv)
            if st != mha.MHA_OK:
                raise mha.MhaError(st, "mha_fwd_splitkv")

        step = split_step
    elif args.which == "kl":
        q2, k2 = to_device(torch, q2b, w.dtype), to_device(torch, k2b, w.dtype)
        kl_out = torch.empty_like(lse)
        lse2 = torch.empty_like(lse)
        kargv = (q.data_ptr(), k.data_ptr(), q2.data_ptr(), k2.data_ptr(), kl_out.data_ptr(),
                 lse.data_ptr(), lse2.data_ptr(), w.B, w.H, w.Nq, w.Nk, w.d, int(w.causal),
                 w.scale, sp, dt)

        def kl_step():
            st = mha.mha_kl_fwd(*kargv)
            if st != mha.MHA_OK:
                raise mha.MhaError(st, "mha_kl_fwd")

        step = kl_step

    if args.calib_copy_mib:
        calib_copy(torch, args.calib_copy_mib, q.device)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # timed region: events on the stream the kernel is launched on
    K = args.steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(K):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])  # ms
    total_ms = ev[0].elapsed_time(ev[K])
    ms_per_step = total_ms / K

    flops = 2.5 * w.flops if args.which == "bwd" else w.flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (per.mean() * 1e-3) / 1e12
    traffic = hbm_traffic(w.name, args.which)
    srcs = {"fwd": KERNEL_SOURCES, "bwd": KERNEL_SOURCES_BWD, "splitkv": KERNEL_SOURCES_SPLIT,
            "kl": KERNEL_SOURCES_KL}
    if args.which == "splitkv":
        # HBM-bound: the metric is the algorithmic bytes moved per second
        gbs = w.io_bytes / (ms_per_step * 1e-3) / 1e9
        gbs_launch = w.io_bytes / (per.mean() * 1e-3) / 1e9
        line = {
            "metric": METRIC_SPLIT,
            "value": round(gbs, 1),
            "unit": "GB/s",
            "pct_of_peak": round(100.0 * gbs / PEAK_GBS, 2),
            "tflops": round(tflops, 3),
        }
        roof = {"bound": "hbm", "achieved": round(gbs_launch, 1), "peak": PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs_launch / PEAK_GBS, 4), "traffic": traffic,
                "kernel": "mha_fwd_splitkv (partial and merge kernels, one call)",
                "bytes_per_step": w.io_bytes, "n_splits": n_splits}
    else:
        line = {
            "metric": {"fwd": METRIC, "bwd": METRIC_BWD, "kl": METRIC_KL}[args.which],
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS, 2),
        }
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": {"fwd": "mha_fwd_kernel", "kl": "mha_kl_kernel",
                           "bwd": "mha_bwd (delta, dq and dkdv kernels, one call)"}[args.which]}
    roof["launch_ms"] = {"mean": round(float(per.mean()), 5),
                         "median": round(float(np.median(per)), 5),
                         "min": round(float(per.min()), 5)}
    line.update({
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": args.which, "B": w.B, "H": w.H, "Nq": w.Nq,
                   "Nk": w.Nk, "d": w.d, "causal": w.causal, "io_dtype": w.dtype,
                   "accumulate": "fp32", "flops_per_step": flops},
        "roofline": roof,
        "timed_wall_s": round(wall, 3),
        "kernel_source_sha256_16": kernel_source_hash(srcs[args.which]),
        "device": torch.cuda.get_device_name(0),
    })
    if not args.no_cpu_baseline:
        print("bench.py: timing the fp64 oracle on the host (cpu_baseline) ...", file=sys.stderr,
              flush=True)
        if args.which == "fwd":
            line["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, args.cpu_seconds)
        elif args.which == "bwd":
            line["cpu_baseline"] = cpu_baseline_bwd(w, qb, kb, vb, gb, args.cpu_seconds)
        elif args.which == "kl":
            line["cpu_baseline"] = cpu_baseline_kl(w, qb, kb, q2b, k2b, args.cpu_seconds)
        else:
            line["cpu_baseline"] = cpu_baseline_split(w, qb, kb, vb, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
