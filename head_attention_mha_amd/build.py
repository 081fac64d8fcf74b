"""Build the HIP library ``libmha.so`` in-tree for gfx950.

Run as ``python -m head_attention_mha_amd.build`` (or through
``__graft_entry__.build()``). It always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmha.so")
SOURCES = [os.path.join(CSRC, f) for f in
           ("mha_api.hip", "mha_fwd.hip", "mha_splitkv.hip", "mha_bwd.hip", "mha_kl.hip",
            "mha_proj.hip")]
DEPS = [os.path.join(CSRC, f) for f in
        ("mha_common.hpp", "mha_validate.hpp", "mha_tiles.hpp", "mha_sync.hpp", "mha_fwd_kernel.hpp", "mha_split_kernel.hpp",
         "mha_bwd_kernel.hpp", "mha_kl_kernel.hpp", "mha_proj_kernel.hpp")]
DEPS.append(os.path.join(ROOT, "include", "mha.h"))

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    # Packed fp32 VALU ops stay off: plain scalar fp32 code only.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: with accumulators in AGPRs the compiler moved
    # every score block to VGPRs before its softmax (v_accvgpr_read).
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    "-Wno-unused-result",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; install ROCm or set HIPCC")


def build(verbose: bool = False, extra_flags: list[str] | None = None) -> str:
    """Compile libmha.so; returns its path. Raises on failure."""
    tmp = LIB + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *(extra_flags or []), "-I", os.path.join(ROOT, "include"),
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
