"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no arithmetic of the attention method: it only draws the
inputs (Gaussian rows, unit-normalised q and k, Gaussian v), rounds them to the
workload's dtype and names the workload shapes.  The HIP path and the CPU
oracle both consume exactly the arrays produced here.

Recipe (the same for every workload):
  * ``numpy.random.Generator(PCG64(s))`` with s = 1000 * (workload seed) + {q: 1, k: 2, v: 3};
    draws are taken in C order over ``[B, H, n, d]``.
  * q and k rows are i.i.d. N(0, 1) in float64, scaled to unit L2 norm;
    v is i.i.d. N(0, 1).
  * The float64 values are cast to float32 (round to nearest even) and, for
    bf16 workloads, further rounded to bfloat16 with round to nearest even.
    The oracle reads the rounded values, widened back to float64.
"""
from __future__ import annotations

import dataclasses
import numpy as np

F32 = "f32"
BF16 = "bf16"


@dataclasses.dataclass(frozen=True)
class Workload:
    """One named workload: shapes, order count P, logit scale c and input dtype."""
    name: str
    seed: int         # seed family (1..6): seeds derive from 1000 * seed
    B: int
    H: int
    n: int
    d_k: int
    d_v: int
    P: int
    c: float
    dtype: str


# The five workloads of the causal SATA study (single head n=256 d=8 P=3 fp32,
# 4x8 heads n=4096 d=16 P=4 fp32, 1x4 heads n=16384 d=64 P=4 bf16, the decode
# workload with 256 resident d=64 states, and 16 heads of d=32 at n=2^20), and
# an order-5 variant of the decode workload.
WORKLOADS = {
    "tiny_d8_n256": Workload("tiny_d8_n256", 1, 1, 1, 256, 8, 8, 3, 1.0, F32),
    "d16_n4096": Workload("d16_n4096", 2, 4, 8, 4096, 16, 16, 4, 1.0, F32),
    "d64_n16384": Workload("d64_n16384", 3, 1, 4, 16384, 64, 64, 4, 1.0, BF16),
    # decode: 8 x 32 = 256 states, 4096-token prefill then 1024 single-token steps
    "decode_256x4096_d64": Workload("decode_256x4096_d64", 4, 8, 32, 4096, 64, 64, 4, 1.0, BF16),
    "long_d32_n1m": Workload("long_d32_n1m", 5, 1, 16, 1 << 20, 32, 32, 4, 1.0, BF16),
    # orders 0..4 at d = 64 (state 814385 x 65 floats, 211.7 MB a head): 32
    # states, 4096-token prefill then single-token steps
    "order5_32x4096_d64": Workload("order5_32x4096_d64", 6, 1, 32, 4096, 64, 64, 5, 1.0, BF16),
}
DECODE_STEPS = 1024


def round_f32(x: np.ndarray) -> np.ndarray:
    """float64 -> float32 with round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round to bfloat16 (nearest even) and return the value as float32.

    The result holds only values representable in bfloat16, so reading its
    upper 16 bits gives the bfloat16 encoding exactly.
    """
    f = round_f32(x)
    bits = f.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    bits = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return bits.view(np.float32)


def bf16_bits(x_bf16_valued_f32: np.ndarray) -> np.ndarray:
    """The bfloat16 encodings (uint16) of float32 values that are bf16-exact."""
    b = np.ascontiguousarray(x_bf16_valued_f32, dtype=np.float32).view(np.uint32)
    if np.any(b & 0xFFFF):
        raise ValueError("values are not exactly representable in bfloat16")
    return (b >> 16).astype(np.uint16)


def _unit_rows(g: np.random.Generator, shape) -> np.ndarray:
    x = g.standard_normal(shape)
    nrm = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
    return x / nrm


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    return round_bf16(x) if dtype == BF16 else round_f32(x)


def make_qkv(B: int, H: int, n: int, d_k: int, d_v: int, dtype: str, seed_base: int):
    """Seeded q, k, v of shape [B, H, n, d] (float32 arrays holding dtype-exact values)."""
    gq = np.random.Generator(np.random.PCG64(seed_base + 1))
    gk = np.random.Generator(np.random.PCG64(seed_base + 2))
    gv = np.random.Generator(np.random.PCG64(seed_base + 3))
    q = _cast(_unit_rows(gq, (B, H, n, d_k)), dtype)
    k = _cast(_unit_rows(gk, (B, H, n, d_k)), dtype)
    v = _cast(gv.standard_normal((B, H, n, d_v)), dtype)
    return q, k, v


def workload_inputs(w: Workload, n: int | None = None):
    """Inputs of a workload (optionally a shorter prefix length n, same seeds)."""
    nn = w.n if n is None else n
    return make_qkv(w.B, w.H, nn, w.d_k, w.d_v, w.dtype, 1000 * w.seed)


def head_inputs(w: Workload, h: int, n: int | None = None):
    """Per-head inputs for the long-context workload (seed + 10*h), shape [n, d]."""
    nn = w.n if n is None else n
    q, k, v = make_qkv(1, 1, nn, w.d_k, w.d_v, w.dtype, 1000 * w.seed + 10 * h)
    return q[0, 0], k[0, 0], v[0, 0]


def decode_inputs(w: Workload, steps: int = DECODE_STEPS):
    """Per-step decode inputs [steps, S, d] with S = B*H states (seed + 100)."""
    S = w.B * w.H
    q, k, v = make_qkv(1, steps, S, w.d_k, w.d_v, w.dtype, 1000 * w.seed + 100)
    return q[0], k[0], v[0]


def sampled_rows(n: int, count: int = 64, seed: int = 5999) -> np.ndarray:
    """Row indices checked on very long sequences: rows 0 and n-1 plus
    count-2 distinct rows drawn from [1, n-2], sorted."""
    g = np.random.Generator(np.random.PCG64(seed))
    inner = g.choice(np.arange(1, n - 1), size=count - 2, replace=False)
    return np.sort(np.concatenate([[0, n - 1], inner])).astype(np.int64)
