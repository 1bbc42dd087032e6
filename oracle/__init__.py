"""Oracle for the attention forward pass (fp64, CPU).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP path
never imports it and shares no code with it.

Functions:

* :func:`attention_rows` / :func:`attention` -- the explicit definition of
  softmax attention in fp64 (C, ``attention_ref.c``): S = scale*QK^T,
  P = softmax(S), O = PV and LSE = log sum exp(S) per row ("A09 - Advanced
  Triton & FlashAttention", section 2; "Building a Verifiable FlashAttention
  Forward from PyTorch to Triton", Part 1).
* :func:`oracle.tiled.tiled_attention` -- the online-softmax tile recurrence
  in fp64 (numpy), used to check that the recurrence reaches the explicit
  result.
* :func:`attention_bwd` -- the explicit fp64 gradients dQ, dK, dV of the
  forward for an upstream gradient dO (C, ``attention_bwd_ref.c``), in the
  order the pages give for the FlashAttention-2 backward ("FlashAttention 2
  from PyTorch to Triton", What is wrong with this kernel, item 5).
* :func:`attention_bwd_sampled` -- the same gradients for one head on
  selected query rows (dQ) and key rows (dK, dV) only, evaluated element by
  element so that single outputs of a long sequence can be checked.

Pins that tie these to the pages and to mathematics (not to themselves) live
in ``tests/test_oracle.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "attention_ref.c")
LIBRARY = os.path.join(_HERE, "liboracle_attention.so")
BWD_SOURCE = os.path.join(_HERE, "attention_bwd_ref.c")
BWD_LIBRARY = os.path.join(_HERE, "liboracle_attention_bwd.so")

# -ffp-contract=off: every product and sum is rounded on its own, as written.
GCC_FLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off", "-std=c11"]


def build(source: str = SOURCE, output: str = LIBRARY) -> str:
    """Compile the C oracle with gcc (no GPU involved)."""
    cmd = ["gcc", *GCC_FLAGS, "-o", output, source, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def build_all() -> None:
    """Compile the forward and backward oracles."""
    build(SOURCE, LIBRARY)
    build(BWD_SOURCE, BWD_LIBRARY)


_lib_cache: dict = {}


def load(path: str = LIBRARY):
    """Load (building if absent or stale) the oracle library at ``path``."""
    if path in _lib_cache:
        return _lib_cache[path]
    if path == LIBRARY and (not os.path.exists(path)
                            or os.path.getmtime(path) < os.path.getmtime(SOURCE)):
        build()
    lib = ctypes.CDLL(path)
    fn = lib.oracle_attention_rows
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 3 + [ctypes.c_int64] * 5 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_void_p]
    _lib_cache[path] = lib
    return lib


def _as_bhnd(x):
    x = np.ascontiguousarray(x, dtype=np.float32)
    if x.ndim == 3:
        return x
    if x.ndim == 4:
        return x.reshape(x.shape[0] * x.shape[1], x.shape[2], x.shape[3])
    raise ValueError("expected [BH, N, D] or [B, H, N, D]")


ALIGNMENTS = ("top-left", "bottom-right")


def causal_offset(nq, nk, causal_align):
    """The diagonal shift coff of the causal mask (query i sees keys j <= i + coff):
    0 for the top-left alignment, Nk - Nq for the bottom-right one."""
    if causal_align not in ALIGNMENTS:
        raise ValueError(f"causal_align must be one of {ALIGNMENTS}")
    return 0 if causal_align == "top-left" else nk - nq


def attention_rows(q, k, v, scale, causal, rows, n_kv=None, causal_align="top-left",
                   lib_path=LIBRARY):
    """O and LSE for the listed rows.

    q: float32 array [B, H, Nq, D] or [BH, Nq, D]; k, v: [.., Nk, D], holding
    exact input values. rows: int array of shape [R, 2] with (flattened head
    bh, query i). n_kv: keys >= n_kv are masked (default Nk). causal_align:
    "top-left" or "bottom-right" (only used when causal). Returns
    (o [R, D], lse [R]) in fp64.
    """
    q3, k3, v3 = _as_bhnd(q), _as_bhnd(k), _as_bhnd(v)
    BH, Nq, D = q3.shape
    Nk = k3.shape[1]
    if k3.shape != (BH, Nk, D) or v3.shape != k3.shape:
        raise ValueError("k and v must be [BH, Nk, D] with the heads and D of q")
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int64).reshape(-1, 2))
    R = rows.shape[0]
    o = np.empty((R, D), dtype=np.float64)
    lse = np.empty((R,), dtype=np.float64)
    if n_kv is None:
        n_kv = Nk
    coff = causal_offset(Nq, Nk, causal_align)
    rc = load(lib_path).oracle_attention_rows(
        q3.ctypes.data, k3.ctypes.data, v3.ctypes.data, BH, Nq, Nk, int(n_kv), D,
        float(scale), int(bool(causal)), int(coff), rows.ctypes.data, R,
        o.ctypes.data, lse.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attention_rows failed with code {rc}")
    return o, lse


def attention(q, k, v, scale, causal, n_kv=None, causal_align="top-left", lib_path=LIBRARY):
    """O [..., Nq, D] and LSE [..., Nq] for every row (small inputs only)."""
    q = np.asarray(q)
    k = np.asarray(k)
    lead = q.shape[:-2]
    Nq, D = q.shape[-2:]
    Nk = k.shape[-2]
    BH = int(np.prod(lead)) if lead else 1
    bh, i = np.meshgrid(np.arange(BH), np.arange(Nq), indexing="ij")
    rows = np.stack([bh.ravel(), i.ravel()], axis=1)
    o, lse = attention_rows(q.reshape(BH, Nq, D), k.reshape(BH, Nk, D),
                            np.asarray(v).reshape(BH, Nk, D), scale, causal, rows,
                            n_kv, causal_align, lib_path)
    return o.reshape(*lead, Nq, D), lse.reshape(*lead, Nq)


def load_bwd(path: str = BWD_LIBRARY):
    """Load (building if absent or stale) the backward oracle library."""
    key = ("bwd", path)
    if key in _lib_cache:
        return _lib_cache[key]
    if path == BWD_LIBRARY and (not os.path.exists(path)
                                or os.path.getmtime(path) < os.path.getmtime(BWD_SOURCE)):
        build(BWD_SOURCE, BWD_LIBRARY)
    lib = ctypes.CDLL(path)
    fn = lib.oracle_attention_bwd
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 4 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_int64] + [ctypes.c_void_p] * 3
    fs = lib.oracle_attention_bwd_sampled
    fs.restype = ctypes.c_int
    fs.argtypes = [ctypes.c_void_p] * 4 + [ctypes.c_int64] * 3 + [
        ctypes.c_double, ctypes.c_int, ctypes.c_int64,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64] + [ctypes.c_void_p] * 3
    _lib_cache[key] = lib
    return lib


def attention_bwd(q, k, v, dout, scale, causal, causal_align="top-left", lib_path=BWD_LIBRARY):
    """dQ, dK, dV (fp64) of O = softmax(scale Q K^T) V for upstream gradient dout.

    q, dout: float32 [..., Nq, D]; k, v: [..., Nk, D] (exact input values).
    Returns arrays shaped like q, k and v respectively.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    lead = q.shape[:-2]
    Nq, D = q.shape[-2:]
    Nk = k.shape[-2]
    BH = int(np.prod(lead)) if lead else 1
    q3 = np.ascontiguousarray(q, dtype=np.float32).reshape(BH, Nq, D)
    k3 = np.ascontiguousarray(k, dtype=np.float32).reshape(BH, Nk, D)
    v3 = np.ascontiguousarray(v, dtype=np.float32).reshape(BH, Nk, D)
    d3 = np.ascontiguousarray(dout, dtype=np.float32).reshape(BH, Nq, D)
    dq = np.empty((BH, Nq, D), np.float64)
    dk = np.empty((BH, Nk, D), np.float64)
    dv = np.empty((BH, Nk, D), np.float64)
    coff = causal_offset(Nq, Nk, causal_align)
    rc = load_bwd(lib_path).oracle_attention_bwd(
        q3.ctypes.data, k3.ctypes.data, v3.ctypes.data, d3.ctypes.data, BH, Nq, Nk, D,
        float(scale), int(bool(causal)), int(coff), dq.ctypes.data, dk.ctypes.data,
        dv.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attention_bwd failed with code {rc}")
    return dq.reshape(*lead, Nq, D), dk.reshape(*lead, Nk, D), dv.reshape(*lead, Nk, D)


def attention_bwd_sampled(q, k, v, dout, scale, causal, rows, cols, causal_align="top-left",
                          lib_path=BWD_LIBRARY):
    """Selected outputs of the fp64 gradients for ONE head: dQ at query rows
    ``rows`` and dK, dV at key rows ``cols`` (the definition evaluated element
    by element, ``oracle_attention_bwd_sampled``).

    q, dout: float32 [Nq, D]; k, v: [Nk, D]. Returns (dq [len(rows), D],
    dk [len(cols), D], dv [len(cols), D]) in float64.
    """
    q2 = np.ascontiguousarray(q, dtype=np.float32)
    k2 = np.ascontiguousarray(k, dtype=np.float32)
    v2 = np.ascontiguousarray(v, dtype=np.float32)
    d2 = np.ascontiguousarray(dout, dtype=np.float32)
    if q2.ndim != 2 or k2.shape != v2.shape or d2.shape != q2.shape or k2.shape[1] != q2.shape[1]:
        raise ValueError("attention_bwd_sampled takes one head: q, dout [Nq, D] and k, v [Nk, D]")
    Nq, D = q2.shape
    Nk = k2.shape[0]
    r = np.ascontiguousarray(rows, dtype=np.int64).reshape(-1)
    c = np.ascontiguousarray(cols, dtype=np.int64).reshape(-1)
    dq = np.empty((len(r), D), np.float64)
    dk = np.empty((len(c), D), np.float64)
    dv = np.empty((len(c), D), np.float64)
    rc = load_bwd(lib_path).oracle_attention_bwd_sampled(
        q2.ctypes.data, k2.ctypes.data, v2.ctypes.data, d2.ctypes.data, Nq, Nk, D,
        float(scale), int(bool(causal)), int(causal_offset(Nq, Nk, causal_align)),
        r.ctypes.data, len(r), c.ctypes.data, len(c), dq.ctypes.data, dk.ctypes.data,
        dv.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attention_bwd_sampled failed with code {rc}")
    return dq, dk, dv
