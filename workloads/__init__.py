"""Seeded synthetic inputs for the fused MHA forward.

This module is shared by the tests, the bench and the smoke check. It only
draws random numbers and rounds them to the 16-bit storage formats; it holds
none of the attention arithmetic, so the oracle and the HIP path can both be
fed from it without sharing any of the method.

Workloads (shapes and distributions follow the attention kinds the pages
describe: encoder self-attention, masked decoder self-attention and decoder
cross-attention in "SparkAttention", Transformer data-flow passage around
Fig. 1; the long-sequence, small-batch training regime in the FlashAttention
long-sequence post, "Motivation: long sequences"):

=================  ==  ==  =====  =====  ===  =====  ======  ====  ===========
name               B   H   Nq     Nk     d    dtype  causal  seed  K multiplier
=================  ==  ==  =====  =====  ===  =====  ======  ====  ===========
tiny               1   2   128    128    64   fp16   no      0     1
encoder_self       8   16  512    512    64   fp16   no      1     1
decoder_causal     4   32  2048   2048   128  bf16   yes     2     1
long_causal        1   8   16384  16384  128  bf16   yes     3     1
cross              16  16  256    2048   64   fp16   no      4     2
=================  ==  ==  =====  =====  ===  =====  ======  ====  ===========

Recipe (the pages leave the generator open; this is the plainest reading):
``numpy.random.default_rng(seed).standard_normal(shape, dtype=float32)`` drawn
in the order Q, K, V, each of shape [B, N, H, d] in C order; rounded to fp16
with numpy's round-to-nearest-even, or to bf16 with round-to-nearest-even on
the fp32 bit pattern; for ``cross`` K is then multiplied by 2, which is exact
in fp16.  The softmax scale is the fp32 value of 1/sqrt(d).

Decoding workloads (few new query rows against a long key/value cache, the
small-NQ case "StreamKL" splits over keys, Methodology section 3; its
contexts run from 4K to 512K tokens), drawn the same way:

=============  ==  ==  ==  =====  ===  =====  ======  ====
name           B   H   Nq  Nk     d    dtype  causal  seed
=============  ==  ==  ==  =====  ===  =====  ======  ====
decode         1   32  1   32768  128  bf16   no      5
decode_multi   8   16  4   8192   64   fp16   no      6
=============  ==  ==  ==  =====  ===  =====  ======  ====

Attention-KL workloads (two distributions over the same keys: a fixed one
from Q1, K1 and one to be trained towards it from Q2, K2; "StreamKL" uses
4K-512K contexts, 32 heads, bf16):

=========  ==  ==  =====  =====  ===  =====  ======  ====
name       B   H   Nq     Nk     d    dtype  causal  seed
=========  ==  ==  =====  =====  ===  =====  ======  ====
kl_long    1   8   16384  16384  128  bf16   yes     7
kl_mid     2   16  4096   4096   64   fp16   no      8
=========  ==  ==  =====  =====  ===  =====  ======  ====

Recipe: from ``default_rng(seed)`` draw N1 (shape of Q), N2 (shape of K), N3
(shape of Q), N4 (shape of K) in that order (standard normal, float32); Q1 and
K1 are N1 and N2 rounded to the type; Q2 and K2 are Q1 + N3/2 and K1 + N4/2
computed in float32 from the rounded Q1, K1 and rounded to the type (a
perturbed copy, as a student near its teacher).

Output-projection workloads (the attention output of the long and decoder
shapes projected back to the model width H*d, "SparkAttention" Eq. 1):

============  ==  =====  ==  ===  ====  =====  ====
name          B   Nq     H   d    E     dtype  seed
============  ==  =====  ==  ===  ====  =====  ====
proj_long     1   16384  8   128  1024  bf16   9
proj_decoder  4   2048   32  128  4096  bf16   10
============  ==  =====  ==  ===  ====  =====  ====

Recipe: from ``default_rng(seed)`` draw O [B, Nq, H, d] standard normal, W
[E, H*d] standard normal times 1/sqrt(H*d), bias [E] standard normal times
0.1 (float32, in that order), each rounded to the type.

The backward's output gradient dO of a workload is drawn the same way from
``default_rng(seed + 1000)`` with the shape of Q ([B, Nq, H, d]) and rounded to
the workload's type.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "f32_to_bf16_bits",
    "f32_to_f16_bits",
    "bits_to_f64",
    "bits_to_f32",
    "round_bits",
    "make_inputs",
    "random_inputs",
    "random_grad",
    "make_grad",
    "DECODE_WORKLOADS",
    "KL_WORKLOADS",
    "make_kl_inputs",
    "ProjWorkload",
    "PROJ_WORKLOADS",
    "make_proj_inputs",
]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "fp16" or "bf16"
    causal: bool
    seed: int
    k_mult: float = 1.0

    @property
    def scale(self) -> float:
        """fp32 value of 1/sqrt(d), returned as a Python float."""
        return float(np.float32(1.0 / math.sqrt(self.d)))

    @property
    def flops(self) -> float:
        """Counted FLOPs: 4*B*H*Nq*Nk*d, halved when causal."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2.0 if self.causal else f

    @property
    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O and fp32 LSE written once."""
        e = 2  # bytes per fp16/bf16 element
        q = self.B * self.Nq * self.H * self.d * e
        kv = 2 * self.B * self.Nk * self.H * self.d * e
        o = q
        lse = self.B * self.H * self.Nq * 4
        return q + kv + o + lse


WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("tiny", 1, 2, 128, 128, 64, "fp16", False, 0),
        Workload("encoder_self", 8, 16, 512, 512, 64, "fp16", False, 1),
        Workload("decoder_causal", 4, 32, 2048, 2048, 128, "bf16", True, 2),
        Workload("long_causal", 1, 8, 16384, 16384, 128, "bf16", True, 3),
        Workload("cross", 16, 16, 256, 2048, 64, "fp16", False, 4, 2.0),
    ]
}


DECODE_WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("decode", 1, 32, 1, 32768, 128, "bf16", False, 5),
        Workload("decode_multi", 8, 16, 4, 8192, 64, "fp16", False, 6),
    ]
}


KL_WORKLOADS: dict[str, Workload] = {
    w.name: w
    for w in [
        Workload("kl_long", 1, 8, 16384, 16384, 128, "bf16", True, 7),
        Workload("kl_mid", 2, 16, 4096, 4096, 64, "fp16", False, 8),
    ]
}


@dataclass(frozen=True)
class ProjWorkload:
    name: str
    B: int
    Nq: int
    H: int
    d: int
    E: int
    dtype: str
    seed: int

    @property
    def flops(self) -> float:
        """2 * (B*Nq) * (H*d) * E multiply-adds counted as two FLOPs."""
        return 2.0 * self.B * self.Nq * self.H * self.d * self.E


PROJ_WORKLOADS: dict[str, ProjWorkload] = {
    w.name: w
    for w in [
        ProjWorkload("proj_long", 1, 16384, 8, 128, 1024, "bf16", 9),
        ProjWorkload("proj_decoder", 4, 2048, 32, 128, 4096, "bf16", 10),
    ]
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bits.

    NaN inputs stay NaN (quiet bit forced)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb cannot wrap for non-NaN patterns (the largest, -inf,
    # is 0xFF800000), so uint32 arithmetic is exact there
    r = (u >> 16) & np.uint32(1)
    r += u
    r += np.uint32(0x7FFF)
    r >>= 16
    rounded = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)
    return rounded


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to fp16 (numpy: nearest, ties to even); uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def round_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp16":
        return f32_to_f16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen fp16/bf16 bit patterns (uint16) to fp32 exactly."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Widen fp16/bf16 bit patterns (uint16) to fp64 exactly."""
    return bits_to_f32(bits, dtype).astype(np.float64)


def _double_bits(bits: np.ndarray, dtype: str, mult: float) -> np.ndarray:
    """Multiply stored 16-bit values by a power of two (exact for N(0,1) data)."""
    x = bits_to_f32(bits, dtype) * np.float32(mult)
    out = round_bits(x, dtype)
    return out


def make_inputs(w: Workload | str) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Q, K, V of a named workload as uint16 bit arrays of shape [B, N, H, d]."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return random_inputs(w.B, w.H, w.Nq, w.Nk, w.d, w.dtype, w.seed, w.k_mult)


def random_inputs(B: int, H: int, Nq: int, Nk: int, d: int, dtype: str, seed: int,
                  k_mult: float = 1.0, std: float = 1.0
                  ) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """iid N(0, std^2) Q [B,Nq,H,d], K and V [B,Nk,H,d], rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    out = []
    for n in (Nq, Nk, Nk):
        x = rng.standard_normal((B, n, H, d), dtype=np.float32)
        if std != 1.0:
            x *= np.float32(std)
        out.append(round_bits(x, dtype))
    q, k, v = out
    if k_mult != 1.0:
        k = _double_bits(k, dtype, k_mult)
    return q, k, v


def random_grad(B: int, H: int, Nq: int, d: int, dtype: str, seed: int) -> np.ndarray:
    """iid N(0, 1) output gradient dO [B, Nq, H, d], rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    return round_bits(rng.standard_normal((B, Nq, H, d), dtype=np.float32), dtype)


def make_grad(w: Workload | str) -> np.ndarray:
    """dO of a named workload as uint16 bits of Q's shape (seed + 1000)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    return random_grad(w.B, w.H, w.Nq, w.d, w.dtype, w.seed + 1000)


def make_kl_inputs(w: Workload | str, noise: float = 0.5):
    """Q1, K1, Q2, K2 of an attention-KL workload as uint16 bits."""
    if isinstance(w, str):
        w = KL_WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    qs, ks = (w.B, w.Nq, w.H, w.d), (w.B, w.Nk, w.H, w.d)
    q1 = round_bits(rng.standard_normal(qs, dtype=np.float32), w.dtype)
    k1 = round_bits(rng.standard_normal(ks, dtype=np.float32), w.dtype)
    n3 = rng.standard_normal(qs, dtype=np.float32)
    n4 = rng.standard_normal(ks, dtype=np.float32)
    q2 = round_bits(bits_to_f32(q1, w.dtype) + np.float32(noise) * n3, w.dtype)
    k2 = round_bits(bits_to_f32(k1, w.dtype) + np.float32(noise) * n4, w.dtype)
    return q1, k1, q2, k2


def make_proj_inputs(w: ProjWorkload | str):
    """O [B, Nq, H, d], W [E, H*d], bias [E] of a projection workload (uint16 bits)."""
    if isinstance(w, str):
        w = PROJ_WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    o = rng.standard_normal((w.B, w.Nq, w.H, w.d), dtype=np.float32)
    wt = rng.standard_normal((w.E, w.H * w.d), dtype=np.float32) * np.float32(1 / math.sqrt(w.H * w.d))
    b = rng.standard_normal(w.E, dtype=np.float32) * np.float32(0.1)
    return round_bits(o, w.dtype), round_bits(wt, w.dtype), round_bits(b, w.dtype)
