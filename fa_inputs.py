"""Seeded synthetic inputs for the attention-forward workloads.

This module is shared by the oracle's tests and by the HIP path's tests and
benchmark. It holds no attention arithmetic: it only draws random numbers,
rounds them to the storage dtype and decodes stored bits back to exact values.

Recipe (the pages draw their inputs with ``torch.randn``; see "FlashAttention 2
from PyTorch to Triton", Step 3, and "Building a Verifiable FlashAttention
Forward from PyTorch to Triton", Part 4): a numpy ``default_rng(seed)``
generator draws float32 values in C order, first Q, then K, then V, each of
shape [B, H, N, D]; a per-workload transform is applied in float32 (a power-of-
two multiplier on Q commutes with rounding); the result is rounded to the
storage dtype with round-to-nearest-even. The same bits go to the GPU and the
oracle, which widens them to float64 exactly.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")
ESIZE = {"fp32": 4, "fp16": 2, "bf16": 2}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str
    seed: int
    masks: tuple            # which of (False, True) = (non-causal, causal) it runs
    q_mult: float = 1.0     # Q is drawn N(0,1) and multiplied by this
    v_dist: str = "normal"  # "normal": N(0,1); "uniform": U(-1, 1)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.D)


# The workloads are named by what they are. Shapes, dtypes, distributions and
# masks follow the five configurations of the attention-forward study plus the
# headline shape (N=4096, D=128, bf16).
WORKLOADS = {
    w.name: w
    for w in (
        Workload("b1h1_n128_d64_fp32", 1, 1, 128, 64, "fp32", 1, (False,)),
        Workload("b8h1_n1024_d64_bf16", 8, 1, 1024, 64, "bf16", 2, (False, True)),
        Workload("b4h16_n4096_d64_bf16", 4, 16, 4096, 64, "bf16", 3, (False, True)),
        Workload("b2h16_n4000_d128_fp16", 2, 16, 4000, 128, "fp16", 4, (False, True)),
        Workload("b1h32_n16384_d128_bf16_q8", 1, 32, 16384, 128, "bf16", 5, (True,),
                 q_mult=8.0, v_dist="uniform"),
        Workload("b4h16_n4096_d128_bf16", 4, 16, 4096, 128, "bf16", 6, (False, True)),
    )
}

HEADLINE = "b4h16_n4096_d128_bf16"


def round_to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round float32 values to the storage dtype (RNE); returns the storage bits.

    bf16 and fp16 come back as uint16 arrays of raw bits, fp32 as float32.
    """
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        b = x32.view(np.uint32).astype(np.uint64)
        lsb = (b >> 16) & 1
        return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 values of stored bits (every bf16/fp16 value is a float32)."""
    if dtype == "fp32":
        return np.ascontiguousarray(bits, dtype=np.float32)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float32)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw_qkv(B, H, N, D, dtype, seed, q_mult=1.0, v_dist="normal"):
    """Draw Q, K, V of shape [B, H, N, D]; returns storage bits (q, k, v)."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    shape = (B, H, N, D)
    q = rng.standard_normal(shape, dtype=np.float32)
    if q_mult != 1.0:
        q *= np.float32(q_mult)
    k = rng.standard_normal(shape, dtype=np.float32)
    if v_dist == "normal":
        v = rng.standard_normal(shape, dtype=np.float32)
    elif v_dist == "uniform":
        v = rng.random(shape, dtype=np.float32) * np.float32(2.0) - np.float32(1.0)
    else:
        raise ValueError(f"unknown v_dist {v_dist!r}")
    return tuple(round_to_dtype(t, dtype) for t in (q, k, v))


def draw_qkv_cross(B, H, Nq, Nk, D, dtype, seed):
    """Q of shape [B, H, Nq, D] and K, V of shape [B, H, Nk, D] (query and key
    lengths differ), drawn N(0,1) in the same order and rounding as draw_qkv."""
    if dtype not in DTYPES:
        raise ValueError(f"unknown dtype {dtype!r}")
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, D), dtype=np.float32)
    k = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    v = rng.standard_normal((B, H, Nk, D), dtype=np.float32)
    return tuple(round_to_dtype(t, dtype) for t in (q, k, v))


def workload_inputs(w: Workload, N: int | None = None, B: int | None = None,
                    H: int | None = None):
    """Inputs of a workload (optionally at a different B/H/N, same recipe)."""
    return draw_qkv(B or w.B, H or w.H, N or w.N, w.D, w.dtype, w.seed,
                    w.q_mult, w.v_dist)
