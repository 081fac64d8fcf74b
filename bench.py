"""Benchmark of the fused MHA forward (default) or backward on one MI355X.

A step is one mha_fwd call (``--pass fwd``) or one mha_bwd call (``--pass
bwd``: dQ with D, then dK/dV, from the forward's O and LSE computed beforehand)
over the whole workload, inputs already resident in HBM. After the W
warm-up steps, untimed steps run for SETTLE_S seconds (the engine clock
ramps up under load); then K steps run back to back between two events on
the launch stream. Default workload:
B=1, H=8, Nq=Nk=16384, d=128, bf16, causal (the long-sequence small-batch
regime of the FlashAttention long-sequence post). Prints ONE JSON line.

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload NAME]
                  [--pass fwd|bwd|splitkv|kl|proj] [--no-cpu-baseline]
                  [--cpu-seconds S] [--calib-copy-mib M] [--counters]
                  [--no-gemm-ref]

For the MFMA-bound passes the roofline object also carries the rate of the
vendor library's bf16 GEMM (torch.matmul, 8192^3) timed the same way on the
same box after the kernel: the dense rate the engine clock sustains under a
pure GEMM load, beside the published peak (frac_of_vendor_gemm).

With --counters, rocprofv3 counter passes over this script run first (as
child processes, before this process touches the GPU) and their HBM bytes,
MFMA busy fraction and engine clock are reported live in the line;
otherwise those fields come from the committed profiles/ summaries while
the kernel sources match them.
"""
from __future__ import annotations

import argparse
import csv
import ctypes
import glob
import hashlib
import re
import json
import math
import os
import resource
import shutil
import subprocess
import sys
import tempfile
import time
from concurrent.futures import ThreadPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "attention fwd TFLOP/s and % of MFMA bf16 peak (B=1,H=8,N=16k,d=128 causal)"
METRIC_BWD = ("attention bwd TFLOP/s (5-matmul count 10*B*H*Nq*Nk*d, halved causal) and % of "
              "MFMA bf16 peak")
PEAK_TFLOPS = 2500.0  # MI355X published dense bf16/fp16 MFMA peak
PEAK_GBS = 8000.0     # MI355X published HBM3E bandwidth
MFMA_FLOP_PER_CLK_PER_CU = 4096  # dense bf16/fp16 MFMA work per CU per cycle (gfx950)
MALL_FLUSH_MIB = 1024  # larger than the 256 MB last-level (MALL) cache
METRIC_KL = ("attention KL(P1||P2) forward TFLOP/s (two QK^T products, 4*B*H*Nq*Nk*d, halved "
             "causal) and % of MFMA bf16 peak")
METRIC_PROJ = ("output projection (head concat then O W^T + b) TFLOP/s, 2*B*Nq*H*d*E, and % of "
               "MFMA bf16 peak")
METRIC_SPLIT = ("attention decode forward (split over keys) HBM GB/s: Q, K, V read and O, LSE "
                "written once, per second")
_CSRC = os.path.join(ROOT, "head_attention_mha_amd", "csrc")
KERNEL_SOURCES = [os.path.join(_CSRC, f) for f in
                  ("mha_common.hpp", "mha_tiles.hpp", "mha_fwd_kernel.hpp", "mha_fwd.hip")]
KERNEL_SOURCES_SPLIT = [os.path.join(_CSRC, f) for f in
                        ("mha_common.hpp", "mha_tiles.hpp", "mha_fwd_kernel.hpp", "mha_split_kernel.hpp",
                         "mha_splitkv.hip")]
KERNEL_SOURCES_BWD = [os.path.join(_CSRC, f) for f in
                      ("mha_common.hpp", "mha_tiles.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp",
                       "mha_bwd_kernel.hpp", "mha_bwd.hip")]
KERNEL_SOURCES_PROJ = [os.path.join(_CSRC, f) for f in
                       ("mha_common.hpp", "mha_tiles.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp",
                        "mha_proj_kernel.hpp", "mha_proj.hip")]
KERNEL_SOURCES_KL = [os.path.join(_CSRC, f) for f in
                     ("mha_common.hpp", "mha_tiles.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp", "mha_kl_kernel.hpp",
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


def profile_fields(kind: str, workload: str, which: str = "fwd"):
    """Fields of a committed counter summary (``profiles/<kind>_[<pass>_]<workload>.txt``,
    ``key: value`` lines), or None when there is none or the kernel sources
    changed since the counters were taken."""
    name = f"{kind}_{workload}.txt" if which == "fwd" else f"{kind}_{which}_{workload}.txt"
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    srcs = {"fwd": KERNEL_SOURCES, "bwd": KERNEL_SOURCES_BWD, "splitkv": KERNEL_SOURCES_SPLIT,
            "kl": KERNEL_SOURCES_KL, "proj": KERNEL_SOURCES_PROJ}[which]
    if fields.get("kernel_source_sha256_16") != kernel_source_hash(srcs):
        return None
    return fields


def _float(fields, key):
    try:
        return float(fields[key]) if fields else None
    except (KeyError, ValueError):
        return None


def hbm_traffic(workload: str, which: str = "fwd"):
    """Per-launch HBM bytes (FETCH + WRITE) from the committed counter summary,
    or None when there is none or the kernel sources changed since."""
    return _float(profile_fields("hbm_traffic", workload, which), "hbm_bytes_per_launch")


def sq_counters(workload: str, which: str = "fwd") -> dict:
    """MFMA busy fraction and the engine clock under load from the committed
    SQ/GRBM counter summary (None where it is missing or stale)."""
    f = profile_fields("sq_counters", workload, which)
    out = {"mfma_busy": _float(f, "mfma_busy_frac"),
           "sclk_mhz_under_load": _float(f, "grbm_sclk_mhz")}
    lb = _float(f, "mfma_busy_frac_lower_bound")
    if lb is not None:  # dispatch too short for the engine-cycle count
        out["mfma_busy_lower_bound"] = lb
    return out


def device_info(torch) -> dict:
    """CU count and peak engine clock of device 0 (hipDeviceGetAttribute) and
    the dense bf16/fp16 MFMA peak they give: CUs x clock x 4096 FLOP/clk."""
    props = torch.cuda.get_device_properties(0)
    cus, khz = int(props.multi_processor_count), None
    try:
        hip = ctypes.CDLL("libamdhip64.so.7")
        val = ctypes.c_int(0)
        if hip.hipDeviceGetAttribute(ctypes.byref(val), 5, 0) == 0:  # hipDeviceAttributeClockRate
            khz = val.value
    except OSError:  # pragma: no cover
        pass
    info = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "cus": cus,
            "max_sclk_mhz": khz / 1000.0 if khz else None}
    info["peak_tflops_from_device"] = (round(cus * khz * 1e3 * MFMA_FLOP_PER_CLK_PER_CU / 1e12, 1)
                                       if khz else None)
    return info


def cpu_workers() -> tuple[int, int]:
    """(workers, CPUs in this process's affinity set): one worker per CPU,
    capped by OMP_NUM_THREADS (the host's share of CPUs per GPU) when set."""
    aff = len(os.sched_getaffinity(0))
    cap = int(os.environ.get("OMP_NUM_THREADS") or aff)
    return max(1, min(aff, cap)), aff


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    return "unknown"


def to_device(torch, bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def run_pool(thunks):
    """Run the oracle calls ``thunks`` on a pool of threads, one per worker
    CPU, each with BLAS pinned to one thread (NumPy releases the GIL inside
    its matrix products and array loops). Returns (results, seconds,
    workers)."""
    from threadpoolctl import threadpool_limits
    workers, _ = cpu_workers()
    with threadpool_limits(limits=1, user_api="blas"):
        t0 = time.perf_counter()
        with ThreadPoolExecutor(max_workers=workers) as ex:
            out = list(ex.map(lambda f: f(), thunks))
        t = time.perf_counter() - t0
    return out, t, min(workers, max(1, len(thunks)))


def _host_fields(workers: int) -> dict:
    _, aff = cpu_workers()
    return {"cores": workers, "affinity_cpus": aff, "cpu_model": cpu_model(),
            "blas_threads_per_worker": 1,
            "peak_rss_gib": round(resource.getrusage(resource.RUSAGE_SELF).ru_maxrss / 2**20, 2)}


def _row_tasks(fn, B, H, rows, chunk=2048):
    """One oracle call per (b, h, chunk of rows); returns thunks and keys."""
    thunks, keys = [], []
    for b in range(B):
        for h in range(H):
            for r0 in range(0, len(rows), chunk):
                r = rows[r0:r0 + chunk]
                thunks.append(lambda b=b, h=h, r=r: fn(b, h, r))
                keys.append((b, h, r0, len(r)))
    return thunks, keys


def _sized_run(one, w, target_s: float):
    """Runs ``one`` over evenly spaced rows of every (b, h), growing the row
    count from 16 until a run takes at least a third of ``target_s`` or
    covers every row; returns that run (rows, thunks, keys, results,
    seconds, workers)."""
    n = 16
    while True:
        rows = np.unique(np.linspace(0, w.Nq - 1, min(n, w.Nq)).astype(np.int64))
        thunks, keys = _row_tasks(one, w.B, w.H, rows)
        res, t, workers = run_pool(thunks)
        if len(rows) >= w.Nq or t >= target_s / 3:
            return rows, thunks, keys, res, t, workers
        n = int(len(rows) * min(8.0, max(1.5, target_s / max(t, 1e-6))))


def cpu_baseline(w: wl.Workload, qb, kb, vb, target_s: float, gpu=None) -> dict:
    """The fp64 oracle, as it stands, on evenly spaced query rows of every
    (batch, head), one call per (b, h, chunk of rows) on a pool of worker
    threads. With ``gpu`` = (O bits, LSE) of the GPU run, the same oracle
    results also give the parity line for the rows timed."""
    import oracle
    q, k, v = (wl.bits_to_f64(x, w.dtype) for x in (qb, kb, vb))

    def one(b, h, r):
        return oracle.attention_fwd(q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1],
                                    v[b:b + 1, :, h:h + 1], w.causal, w.scale, rows=r)

    rows, thunks, keys, res, t, workers = _sized_run(one, w, target_s)
    vis = (rows + 1).clip(max=w.Nk) if w.causal else np.full(len(rows), w.Nk)
    flops = 4.0 * w.d * float(vis.sum()) * w.B * w.H
    own = 4.0 * w.d * w.Nk * len(rows) * w.B * w.H  # the oracle forms every score, then masks
    out = {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        **_host_fields(workers),
        "kind": "oracle",
        "sample": (f"{len(rows)} evenly spaced query rows of each of the {w.B * w.H} (batch, head) "
                   f"pairs ({len(rows) / w.Nq:.1%} of the rows, all their keys), fp64 NumPy, "
                   f"{len(thunks)} calls of <= 2048 rows on {workers} worker threads, {t:.1f} s; "
                   f"FLOPs counted as 4*d*visible keys per row"),
        "seconds": t,
        "oracle_own_tflops": own / t / 1e12,
    }
    if gpu is not None:
        from parity import compare, report  # tests/parity.py: the comparison rule
        O_ref = np.empty((w.B, len(rows), w.H, w.d))
        L_ref = np.empty((w.B, w.H, len(rows)))
        for (b, h, r0, n), (O, L) in zip(keys, res):
            O_ref[b, r0:r0 + n, h] = O[0, :, 0]
            L_ref[b, h, r0:r0 + n] = L[0, 0]
        o_bits, lse = gpu
        st = compare(o_bits[:, rows], lse[:, :, rows], O_ref, L_ref, w.dtype, rows=rows)
        out["parity"] = {"line": report(st, w.name), "o_max_abs": st["o_max"],
                         "o_max_at": st["o_max_at"], "o_mean_abs": st["o_mean"],
                         "floor": st["floor"], "floor_at": st["floor_at"],
                         "o_n_over_1e-2": st["o_n_over"], "lse_max_abs": st["lse_max"],
                         "rows_compared": int(len(rows)), "finite": st["finite"]}
    return out


def cpu_baseline_kl(w: wl.Workload, q1b, k1b, q2b, k2b, target_s: float) -> dict:
    """The fp64 KL oracle, as it stands, on evenly spaced query rows of every
    (batch, head) (all keys), one call per (b, h, chunk of rows) on the pool."""
    import oracle
    x = [wl.bits_to_f64(a, w.dtype) for a in (q1b, k1b, q2b, k2b)]

    def one(b, h, r):
        return oracle.attention_kl(*(a[b:b + 1, :, h:h + 1] for a in x), w.causal, w.scale, rows=r)

    rows, thunks, _, _, t, workers = _sized_run(one, w, target_s)
    vis = (rows + 1).clip(max=w.Nk) if w.causal else np.full(len(rows), w.Nk)
    flops = 4.0 * w.d * float(vis.sum()) * w.B * w.H
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        **_host_fields(workers),
        "kind": "oracle",
        "sample": (f"{len(rows)} evenly spaced query rows of each of the {w.B * w.H} (batch, head) "
                   f"pairs ({len(rows) / w.Nq:.1%} of the rows, all their keys), fp64 NumPy, "
                   f"{len(thunks)} calls on {workers} worker threads, {t:.1f} s; FLOPs counted as "
                   f"4*d*visible keys per row"),
        "seconds": t,
    }


def cpu_baseline_split(w: wl.Workload, qb, kb, vb, target_s: float) -> dict:
    """The fp64 split-over-keys oracle, as it stands, one call per (batch
    entry, head) on the pool, over whole batch entries, doubling their number
    until the run takes about a quarter of ``target_s`` or covers the
    workload."""
    import oracle
    n_splits = max(1, min(256, -(-w.Nk // 2048)))
    bounds = np.linspace(0, w.Nk, n_splits + 1).astype(np.int64)
    q, k, v = (wl.bits_to_f64(x, w.dtype) for x in (qb, kb, vb))

    def timed(nb):
        thunks = [lambda b=b, h=h: oracle.attention_fwd_split(
            q[b:b + 1, :, h:h + 1], k[b:b + 1, :, h:h + 1], v[b:b + 1, :, h:h + 1],
            w.causal, w.scale, bounds) for b in range(nb) for h in range(w.H)]
        _, t, workers = run_pool(thunks)
        return t, workers

    nb = 1
    t, workers = timed(nb)
    while nb < w.B and t < target_s / 4:
        nb = min(w.B, 2 * nb)
        t, workers = timed(nb)
    bytes_ = nb * w.H * ((2 * w.Nq + 2 * w.Nk) * w.d * 2 + 4 * w.Nq)
    return {
        "value": bytes_ / t / 1e9,
        "unit": "GB/s",
        **_host_fields(workers),
        "kind": "oracle",
        "sample": (f"batch entries 0..{nb - 1} ({nb} of {w.B}, all {w.H} heads), {n_splits} key "
                   f"splits, fp64 NumPy, one call per (b, h) on {workers} worker threads, "
                   f"{t:.2f} s; bytes counted as for the GPU line"),
        "seconds": t,
    }


def cpu_baseline_bwd(w: wl.Workload, qb, kb, vb, gb, target_s: float) -> dict:
    """The fp64 backward oracle, as it stands, on a bounded sample, one call
    per head on the pool.

    The sample is the first n tokens (queries and keys) of the first m heads
    of batch entry 0: a prefix of a sequence is a complete problem of the
    same kind (causal stays causal). n grows until the heads take about a
    quarter of ``target_s`` or cover the whole sequence; then more heads are
    added while the time stays within ``target_s``."""
    import oracle
    q, k, v, do = (wl.bits_to_f64(x[:1], w.dtype) for x in (qb, kb, vb, gb))
    workers, _ = cpu_workers()

    def timed(n, m):
        nk = n if w.Nq == w.Nk else w.Nk
        thunks = [lambda h=h: oracle.attention_bwd(
            q[:, :n, h:h + 1], k[:, :nk, h:h + 1], v[:, :nk, h:h + 1], do[:, :n, h:h + 1],
            w.causal, w.scale) for h in range(m)]
        _, t, used = run_pool(thunks)
        return t, nk, used

    m = min(w.H, workers)
    n = min(w.Nq, 256)
    t, nk, used = timed(n, m)
    while n < w.Nq and t < target_s / 4:
        n = min(w.Nq, int(n * 1.6))
        t, nk, used = timed(n, m)
    if n == w.Nq and w.H > m and t < target_s / 2:
        m = int(max(m, min(w.H, m * target_s / max(t, 1e-6))))
        t, nk, used = timed(n, m)
    flops = 10.0 * n * nk * w.d * m / (2.0 if w.causal else 1.0)
    return {
        "value": flops / t / 1e12,
        "unit": "TFLOP/s",
        **_host_fields(used),
        "kind": "oracle",
        "sample": (f"the first {n} queries and {nk} keys of heads 0..{m - 1} of batch entry 0, "
                   f"fp64 NumPy, one call per head on {used} worker threads, {t:.1f} s; FLOPs "
                   f"counted as for the GPU line"),
        "seconds": t,
    }


SETTLE_S = 0.25  # untimed load before the timed region (engine clock ramp)


def settle(torch, step, min_s: float = SETTLE_S) -> int:
    """Untimed launches, in batches of 10, until min_s seconds of load have
    passed: after the warm-up steps the engine clock is still ramping up (the
    first hundred launches after idle run a few percent slower than the
    ones after them). Returns the number of launches."""
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
        n += 10
    return n


VENDOR_GEMM_N = 8192


def vendor_gemm_ref(torch) -> dict:
    """The vendor library's bf16 GEMM (torch.matmul, N x N x N, N = 8192) on
    this box, warmed up, settled and timed back to back like the kernels: the
    dense MFMA rate the engine clock sustains under a pure GEMM load, beside
    the published peak. Runs after the kernel's timed region; not part of
    any step."""
    n = VENDOR_GEMM_N
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)

    def step():
        torch.matmul(a, b)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    settle(torch, step)
    ms, _ = time_steps(torch, torch.cuda.current_stream(), step, 20)
    del a, b
    return {"what": f"torch.matmul bf16 {n}x{n}x{n} (vendor GEMM library), same box",
            "ms": round(ms, 4), "tflops": round(2.0 * n ** 3 / (ms * 1e-3) / 1e12, 1)}


def apply_live(roof: dict, live, flops: float, ms_per_step: float, dev: dict) -> None:
    """Put live counter results (--counters) into the roofline object, in
    place of the committed summaries' figures."""
    if not live:
        return
    roof["counters_live"] = live
    if "error" in live:
        return
    roof["traffic"] = live["hbm_bytes_per_step"]
    roof["traffic_source"] = "live counters"
    roof["traffic_gbs"] = round(live["hbm_bytes_per_step"] / (ms_per_step * 1e-3) / 1e9, 1)
    for src, dst in (("mfma_busy", "mfma_busy"), ("sclk_mhz", "sclk_mhz_under_load"),
                     ("mfma_busy_lower_bound", "mfma_busy_lower_bound")):
        if src in live:
            roof[dst] = live[src]
    if roof.get("sclk_mhz_under_load") and dev.get("cus") and roof.get("unit") == "TFLOP/s":
        pk = dev["cus"] * roof["sclk_mhz_under_load"] * 1e6 * MFMA_FLOP_PER_CLK_PER_CU / 1e12
        roof["peak_at_sclk_under_load"] = round(pk, 1)
        roof["frac_at_sclk_under_load"] = round(flops / (ms_per_step * 1e-3) / 1e12 / pk, 4)


def time_steps(torch, stream, step, K: int):
    """The timed region: K steps back to back between two events recorded on
    the launch stream, bracketed by device synchronisation. Returns (ms per
    step, wall seconds)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(K):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / K, time.perf_counter() - t0


def per_launch_events(torch, stream, step, K: int) -> np.ndarray:
    """Outside the timed region: K launches, each between its own pair of
    events. An event's release between launches adds a gap of a few
    microseconds and starts the next launch with flushed caches, so these
    times are longer than the back-to-back average; reported, not used."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    torch.cuda.synchronize()
    ev[0].record(stream)
    for i in range(K):
        step()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(K)])


def launch_fields(ms_per_step: float, per: np.ndarray) -> dict:
    return {"mean": round(ms_per_step, 5),
            "per_launch_events": {"mean": round(float(per.mean()), 5),
                                  "median": round(float(np.median(per)), 5),
                                  "min": round(float(per.min()), 5)}}


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


def bench_proj(args, torch, mha, w, live=None) -> int:
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
    n_settle = settle(torch, step)
    ms, wall = time_steps(torch, stream, step, K)
    per = per_launch_events(torch, stream, step, K)
    tflops = w.flops / (ms * 1e-3) / 1e12
    achieved = tflops
    line = {
        "metric": f"{METRIC_PROJ} (B={w.B},Nq={w.Nq},H={w.H},d={w.d},E={w.E}, {w.dtype})",
        "value": round(tflops, 2), "unit": "TFLOP/s",
        "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS, 2), "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "pass": "proj", "B": w.B, "Nq": w.Nq, "H": w.H, "d": w.d,
                   "E": w.E, "io_dtype": w.dtype, "accumulate": "fp32", "flops_per_step": w.flops},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4),
                     "traffic": hbm_traffic(w.name, "proj"), "kernel": "mha_proj_kernel",
                     "launch_ms": launch_fields(ms, per)},
        "timed_wall_s": round(wall, 3),
        "settle_launches": n_settle,
        "kernel_source_sha256_16": kernel_source_hash(KERNEL_SOURCES_PROJ),
        "device": device_info(torch),
    }
    if not args.no_gemm_ref:
        ref = vendor_gemm_ref(torch)
        line["roofline"]["vendor_bf16_gemm"] = ref
        line["roofline"]["frac_of_vendor_gemm"] = round(achieved / ref["tflops"], 4)
    apply_live(line["roofline"], live, w.flops, ms, line["device"])
    if not args.no_cpu_baseline:
        print("bench.py: timing the fp64 oracle on the host (cpu_baseline) ...", file=sys.stderr,
              flush=True)
        line["cpu_baseline"] = cpu_baseline_proj(w, ob, wb, bb, args.cpu_seconds)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)
    return 0


def cpu_baseline_proj(w, ob, wb, bb, target_s: float) -> dict:
    """The fp64 projection oracle, as it stands, on leading token rows, one
    call per chunk of 256 rows on the pool."""
    import oracle
    wt, b = wl.bits_to_f64(wb, w.dtype), wl.bits_to_f64(bb, w.dtype)
    x = ob.reshape(w.B * w.Nq, w.H, w.d)

    def timed(n):
        xs = wl.bits_to_f64(x[:n], w.dtype)
        thunks = [lambda r=r: oracle.out_proj(xs[None, r:r + 256], wt, b) for r in range(0, n, 256)]
        _, t, used = run_pool(thunks)
        return t, used

    n = min(w.B * w.Nq, 1024)
    t, used = timed(n)
    while n < w.B * w.Nq and t < target_s / 4:
        n = min(w.B * w.Nq, 2 * n)
        t, used = timed(n)
    flops = 2.0 * n * w.H * w.d * w.E
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", **_host_fields(used), "kind": "oracle",
            "sample": (f"the first {n} of {w.B * w.Nq} token rows, fp64 NumPy matmul, chunks of "
                       f"256 rows on {used} worker threads, {t:.2f} s"),
            "seconds": t}


# ---- live counters (--counters) ----------------------------------------------
# rocprofv3 counter passes over this same script, each a child process of its
# own started before this process touches the GPU: FETCH_SIZE and WRITE_SIZE
# (HBM bytes, scaled by what they read for three plain 512 MiB device copies
# in the same run) and SQ/GRBM counters (MFMA busy cycles and the engine
# clock). The timed launches of a child are found from the settle count it
# prints; their mean per step is reported.
STEP_KERNELS = {"fwd": ["mha_fwd_kernel"],
                "bwd": ["mha_bwd_dq_kernel", "mha_bwd_dkdv_kernel", "mha_bwd_dkdv_pair_kernel"],
                "splitkv": ["mha_split_partial_kernel", "mha_split_merge_kernel"],
                "kl": ["mha_kl_kernel"], "proj": ["mha_proj_kernel"]}
LIVE_SQ = ["SQ_WAVES", "SQ_INSTS_MFMA", "SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE"]
N_XCD, N_SIMD = 8, 1024
CALIB_MIB = 512


def _kernel_key(name: str):
    m = re.search(r"(mha_\w+?_kernel|__amd_rocclr_copyBuffer)", name)
    return m.group(1) if m else None


def _pmc_run(rocprof, counters, which, workload, steps, calib, workdir, timeout_s=240):
    """One rocprofv3 --pmc pass over a child bench run; returns (child's JSON
    line, dispatches in order as dicts of kernel key and counter values)."""
    out = tempfile.mkdtemp(prefix="pmc_", dir=workdir)
    child = [sys.executable, os.path.abspath(__file__), "--pass", which, "--workload", workload,
             "--steps", str(steps), "--warmup", "1", "--no-cpu-baseline", "--no-gemm-ref"]
    if calib:
        child += ["--calib-copy-mib", str(CALIB_MIB)]
    cmd = [rocprof, "--pmc", *counters, "--output-format", "csv", "-d", out, "-o", "p", "--", *child]
    print("bench.py: " + " ".join(cmd), file=sys.stderr, flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout_s)
    line = None
    for ln in res.stdout.splitlines():
        if ln.startswith("{") and '"metric"' in ln:
            line = json.loads(ln)
    files = glob.glob(os.path.join(out, "**", "*counter_collection.csv"), recursive=True)
    if res.returncode != 0 or line is None or not files:
        raise RuntimeError(f"counter pass {counters} failed (rc {res.returncode}): "
                           + res.stderr[-500:])
    return line, read_counter_csv(files[0]), cmd


def read_counter_csv(path: str) -> list:
    """rocprofv3 counter_collection.csv -> one dict per dispatch, in dispatch
    order: kernel key, start and end timestamps (ns) and each counter summed
    over the rows of that dispatch."""
    disp = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            e = disp.setdefault(int(r["Dispatch_Id"]), {"key": _kernel_key(r["Kernel_Name"]),
                                                         "start": int(r["Start_Timestamp"]),
                                                         "end": int(r["End_Timestamp"])})
            e[r["Counter_Name"]] = e.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    return [disp[k] for k in sorted(disp)]


def _timed(dispatches, key, line, steps):
    """The child's timed launches of kernel `key` (one per step): after its
    one warm-up launch and its settling launches."""
    ds = [d for d in dispatches if d["key"] == key]
    first = 1 + int(line.get("settle_launches", 0))
    return ds[first:first + steps]


def live_counters(which: str, workload: str) -> dict:
    rocprof = shutil.which("rocprofv3") or "/opt/rocm/bin/rocprofv3"
    if not os.path.exists(rocprof):
        raise RuntimeError("rocprofv3 not found")
    steps = 3
    work = tempfile.mkdtemp(prefix="bench_counters_")
    try:
        out = {"source": "live rocprofv3 counter passes", "timed_launches": steps, "commands": []}
        per = {}
        for ctr in ("FETCH_SIZE", "WRITE_SIZE"):
            line, ds, cmd = _pmc_run(rocprof, [ctr], which, workload, steps, True, work)
            out["commands"].append(" ".join(cmd[cmd.index("--pmc"):]))
            copies = [d[ctr] for d in ds if d["key"] == "__amd_rocclr_copyBuffer"
                      and d[ctr] > 0.4 * CALIB_MIB * 1024]
            factor = CALIB_MIB * 1024 / (sum(copies) / len(copies))
            tot = 0.0
            for k in STEP_KERNELS[which]:
                t = _timed(ds, k, line, steps)
                if t:  # (one of the dK/dV kernels, by head size)
                    tot += sum(d[ctr] for d in t) / len(t) * 1024 * factor
            per[ctr] = tot
            out[f"{ctr.lower()}_calibration_factor"] = round(factor, 4)
        out["fetch_bytes_per_step"] = round(per["FETCH_SIZE"])
        out["write_bytes_per_step"] = round(per["WRITE_SIZE"])
        out["hbm_bytes_per_step"] = round(per["FETCH_SIZE"] + per["WRITE_SIZE"])
        if which != "splitkv":
            line, ds, cmd = _pmc_run(rocprof, LIVE_SQ, which, workload, steps, False, work)
            out["commands"].append(" ".join(cmd[cmd.index("--pmc"):]))
            kern = {}
            for k in STEP_KERNELS[which]:
                t = _timed(ds, k, line, steps)
                if not t:
                    continue
                dur = sum(d["end"] - d["start"] for d in t) / len(t)
                busy = sum(d["SQ_VALU_MFMA_BUSY_CYCLES"] for d in t) / len(t) / N_SIMD
                grbm = sum(d["GRBM_GUI_ACTIVE"] for d in t) / len(t) / N_XCD
                e = {"dispatch_us": round(dur / 1e3, 1), "mfma_busy_cycles_per_simd": round(busy)}
                if dur >= 1e5:  # GRBM also counts the dispatch's start and end
                    e["mfma_busy"] = round(busy / grbm, 4)
                    e["sclk_mhz"] = round(grbm / dur * 1e3)
                else:
                    e["mfma_busy_lower_bound"] = round(busy / grbm, 4)
                kern[k] = e
            out["kernels"] = kern
            dom = max(kern, key=lambda k: kern[k]["dispatch_us"])
            out["dominant_kernel"] = dom
            for f in ("mfma_busy", "sclk_mhz", "mfma_busy_lower_bound"):
                if f in kern[dom]:
                    out[f] = kern[dom][f]
        return out
    finally:
        shutil.rmtree(work, ignore_errors=True)


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
    ap.add_argument("--no-gemm-ref", action="store_true",
                    help="skip the vendor bf16 GEMM reference rate (MFMA-bound passes)")
    ap.add_argument("--counters", action="store_true",
                    help="also run rocprofv3 counter passes (HBM bytes, MFMA busy, engine "
                         "clock) over this script first and report them live")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the forward shards over heads with no communication; see DESIGN.md)",
              file=sys.stderr)
        return 2

    live = None
    if args.counters:
        # child processes, started before this process touches the GPU
        wname = args.workload or {"splitkv": "decode", "kl": "kl_long",
                                  "proj": "proj_long"}.get(args.which, "long_causal")
        try:
            live = live_counters(args.which, wname)
        except (RuntimeError, subprocess.TimeoutExpired, ZeroDivisionError, IndexError) as e:
            live = {"error": str(e)[-300:]}

    import torch

    import head_attention_mha_amd as mha

    if not torch.cuda.is_available():
        print("bench.py: no GPU available", file=sys.stderr)
        return 1
    mha.load_library()
    name = args.workload or {"splitkv": "decode", "kl": "kl_long",
                             "proj": "proj_long"}.get(args.which, "long_causal")
    if args.which == "proj":
        return bench_proj(args, torch, mha, wl.PROJ_WORKLOADS[name], live)
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

    # untimed settling load, then the timed region: K steps back to back, one
    # event pair on the launch stream
    K = args.steps
    n_settle = settle(torch, step)
    ms_per_step, wall = time_steps(torch, stream, step, K)
    # outside the timed region: each launch between its own events, and
    # launches each preceded by a write of MALL_FLUSH_MIB MiB (the inputs
    # then come from HBM, not from the last-level cache)
    per = per_launch_events(torch, stream, step, K)
    flushed_ms = None
    if args.which == "fwd":
        scratch = torch.empty(MALL_FLUSH_MIB << 18, dtype=torch.float32, device=q.device)
        fl = []
        for _ in range(min(K, 20)):
            scratch.fill_(1.0)
            a, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b_.record(stream)
            torch.cuda.synchronize()
            fl.append(a.elapsed_time(b_))
        flushed_ms = float(np.median(fl))
        del scratch

    dev = device_info(torch)
    flops = 2.5 * w.flops if args.which == "bwd" else w.flops
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    achieved = tflops  # per launch: the back-to-back average launch duration
    traffic = hbm_traffic(w.name, args.which)
    srcs = {"fwd": KERNEL_SOURCES, "bwd": KERNEL_SOURCES_BWD, "splitkv": KERNEL_SOURCES_SPLIT,
            "kl": KERNEL_SOURCES_KL}
    shape = (f"B={w.B},H={w.H},Nq={w.Nq},Nk={w.Nk},d={w.d}{' causal' if w.causal else ''}, "
             f"{w.dtype}")
    if args.which == "splitkv":
        # HBM-bound: the metric is the algorithmic bytes moved per second
        gbs = w.io_bytes / (ms_per_step * 1e-3) / 1e9
        gbs_launch = gbs
        line = {
            "metric": f"{METRIC_SPLIT} ({shape})",
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
        metric = {"fwd": METRIC, "bwd": METRIC_BWD, "kl": METRIC_KL}[args.which]
        if args.which == "fwd" and w.name != "long_causal":
            metric = f"attention fwd TFLOP/s and % of MFMA bf16 peak ({shape})"
        elif args.which != "fwd":
            metric = f"{metric} ({shape})"
        line = {
            "metric": metric,
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "pct_of_peak": round(100.0 * tflops / PEAK_TFLOPS, 2),
        }
        io_bytes = w.io_bytes if args.which == "fwd" else None
        roof = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS, 4), "traffic": traffic,
                "kernel": {"fwd": "mha_fwd_kernel", "kl": "mha_kl_kernel",
                           "bwd": "mha_bwd (dq with D, then dkdv, one call)"}[args.which]}
        if dev["peak_tflops_from_device"]:
            roof["peak_from_device"] = dev["peak_tflops_from_device"]
            roof["frac_of_device_peak"] = round(achieved / dev["peak_tflops_from_device"], 4)
        if io_bytes:
            # algorithmic bytes (Q, K, V read once, O and LSE written once) per second
            roof["algorithmic_bytes"] = io_bytes
            roof["achieved_gbs"] = round(io_bytes / (ms_per_step * 1e-3) / 1e9, 1)
            roof["achieved_gbs_frac"] = round(roof["achieved_gbs"] / PEAK_GBS, 4)
            if traffic:
                roof["traffic_gbs"] = round(traffic / (ms_per_step * 1e-3) / 1e9, 1)
        roof.update(sq_counters(w.name, args.which))
        if traffic:
            roof["traffic_source"] = "committed summary (kernel sources match)"
        if roof.get("sclk_mhz_under_load") and dev["cus"]:
            # the dense ceiling at the engine clock the counters saw under this load
            pk = dev["cus"] * roof["sclk_mhz_under_load"] * 1e6 * MFMA_FLOP_PER_CLK_PER_CU / 1e12
            roof["peak_at_sclk_under_load"] = round(pk, 1)
            roof["frac_at_sclk_under_load"] = round(achieved / pk, 4)
    roof["launch_ms"] = launch_fields(ms_per_step, per)
    if roof["bound"] == "mfma" and not args.no_gemm_ref:
        ref = vendor_gemm_ref(torch)
        roof["vendor_bf16_gemm"] = ref
        roof["frac_of_vendor_gemm"] = round(achieved / ref["tflops"], 4)
    if flushed_ms is not None:
        roof["mall_flushed"] = {"flush_mib": MALL_FLUSH_MIB, "launch_ms_median": round(flushed_ms, 5),
                                "tflops": round(flops / (flushed_ms * 1e-3) / 1e12, 2),
                                "achieved_gbs": round(w.io_bytes / (flushed_ms * 1e-3) / 1e9, 1)}
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
        "settle_launches": n_settle,
        "kernel_source_sha256_16": kernel_source_hash(srcs[args.which]),
        "device": dev,
    })
    apply_live(roof, live, flops, ms_per_step, dev)
    if not args.no_cpu_baseline:
        print("bench.py: timing the fp64 oracle on the host (cpu_baseline) ...", file=sys.stderr,
              flush=True)
        if args.which == "fwd":
            sys.path.insert(0, os.path.join(ROOT, "tests"))
            step()  # one more launch: the outputs the parity line compares
            torch.cuda.synchronize()
            got = (o.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy())
            line["cpu_baseline"] = cpu_baseline(w, qb, kb, vb, args.cpu_seconds, gpu=got)
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
