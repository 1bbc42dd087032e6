"""Helpers for GPU-vs-oracle parity tests.

Tolerances (written here, used by every parity test):
* O in bf16/fp16: max over all checked elements of |O_gpu - O_ref| <= 1e-2.
* O in fp32: normwise, max|O_gpu - O_ref| / max|O_ref| <= 1e-5 (elementwise
  relative error is unbounded near zero outputs).
* LSE (fp32, natural log): max |LSE_gpu - LSE_ref| <= 1e-3.
O_ref and LSE_ref are the fp64 oracle on the same rounded inputs.

Backward (dQ, dK, dV in bf16/fp16): normwise per tensor,
max|G_gpu - G_ref| / max|G_ref| <= 1e-2 for bf16 and 3e-3 for fp16, against
the fp64 backward oracle on the same rounded inputs. The kernels round P and
dS to the input type before their products and the gradients once at the end
(relative 2^-9 each for bf16, 2^-11 for fp16); sums of many terms with
independent rounding errors keep a relative error of that order, so the bound
leaves a margin of about 2.5x over three such roundings. D = rowsum(dO * O)
(fp32) is checked against the same sum in fp64 over the kernel's own O,
relative to max|D|, within 1e-5.
"""
from __future__ import annotations

import math

import numpy as np

import fa_inputs
import oracle

TOL_O_16 = 1e-2
TOL_O_32_NORMWISE = 1e-5
TOL_LSE = 1e-3
TOL_GRAD = {"bf16": 1e-2, "fp16": 3e-3}
TOL_DELTA = 1e-5


def torch_dtype(dtype):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def to_device(bits, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits))
    if dtype == "bf16":
        t = t.view(torch.int16).view(torch.bfloat16)
    elif dtype == "fp16":
        t = t.view(torch.int16).view(torch.float16)
    return t.cuda()


def from_device(t):
    import torch
    return t.float().cpu().numpy() if t.dtype != torch.float32 else t.cpu().numpy()


def sample_rows(B, H, N, count, seed, bm=128):
    """Rows to check at full size: first/last rows, rows around every
    multiple of the query tile near both ends, and random rows, spread over
    heads. Returns an int array [R, 2] of (bh, i)."""
    rng = np.random.default_rng(seed)
    BH = B * H
    special = {0, 1, N - 1, N - 2}
    for t in (1, 2, 3, N // bm - 1, N // bm, N // bm + 1):
        for d in (-1, 0, 1):
            i = t * bm + d
            if 0 <= i < N:
                special.add(i)
    rows = [(int(bh), int(i)) for bh in {0, BH - 1, BH // 2} for i in special]
    rest = max(0, count - len(rows))
    rows += [(int(a), int(b)) for a, b in zip(rng.integers(0, BH, rest), rng.integers(0, N, rest))]
    return np.unique(np.array(rows, dtype=np.int64), axis=0)


def check(o_gpu, lse_gpu, o_ref, lse_ref, dtype, what=""):
    """Assert parity; returns (o_err, lse_err) with o_err in the metric of the
    dtype (absolute for 16-bit, normwise for fp32)."""
    o_gpu = np.asarray(o_gpu, dtype=np.float64)
    o_ref = np.asarray(o_ref, dtype=np.float64)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    diff = np.abs(o_gpu - o_ref).max() if o_ref.size else 0.0
    if dtype == "fp32":
        ref_max = np.abs(o_ref).max() if o_ref.size else 0.0
        o_err = diff / ref_max if ref_max > 0 else diff
        assert o_err <= TOL_O_32_NORMWISE, f"{what}: fp32 O normwise error {o_err:.3e}"
    else:
        o_err = diff
        assert o_err <= TOL_O_16, f"{what}: O max abs error {o_err:.3e}"
    lse_err = 0.0
    if lse_gpu is not None:
        lse_gpu = np.asarray(lse_gpu, dtype=np.float64)
        lse_ref = np.asarray(lse_ref, dtype=np.float64)
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lse_gpu)), f"{what}: LSE finiteness differs"
        assert (lse_gpu[~fin] == lse_ref[~fin]).all(), f"{what}: LSE infinities differ"
        if fin.any():
            lse_err = np.abs(lse_gpu[fin] - lse_ref[fin]).max()
        assert lse_err <= TOL_LSE, f"{what}: LSE max abs error {lse_err:.3e}"
    return o_err, lse_err


def check_every_row(o_gpu, lse_gpu, q_bits, k_bits, v_bits, dtype, scale, causal, what="",
                    chunk=16384):
    """Compare every output element and every LSE of a [B, H, N, D] result
    with the fp64 oracle, which is evaluated in chunks of query rows so that
    memory stays bounded at any size. The tolerances are those of check().
    Returns (o_err, lse_err, worst): o_err in the metric of the dtype, and
    worst = (head, row, d, |O_ref| there) for the largest O difference."""
    B, H, N, D = q_bits.shape
    BH = B * H
    q, k, v = (fa_inputs.to_f32(x, dtype).reshape(BH, N, D) for x in (q_bits, k_bits, v_bits))
    o_gpu = np.asarray(o_gpu).reshape(BH * N, D)
    lse_gpu = np.asarray(lse_gpu, dtype=np.float64).reshape(BH * N)
    assert np.isfinite(o_gpu).all(), f"{what}: non-finite O"
    diff_max, ref_max, lse_err, worst = 0.0, 0.0, 0.0, None
    for start in range(0, BH * N, chunk):
        idx = np.arange(start, min(start + chunk, BH * N), dtype=np.int64)
        rows = np.stack([idx // N, idx % N], axis=1)
        o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, causal, rows)
        d = np.abs(o_gpu[idx].astype(np.float64) - o_ref)
        at = np.unravel_index(np.argmax(d), d.shape)
        if d[at] > diff_max:
            diff_max = float(d[at])
            r = int(idx[at[0]])
            worst = (r // N, r % N, int(at[1]), float(abs(o_ref[at])))
        ref_max = max(ref_max, float(np.abs(o_ref).max()))
        lg = lse_gpu[idx]
        fin = np.isfinite(lse_ref)
        assert np.array_equal(fin, np.isfinite(lg)), f"{what}: LSE finiteness differs"
        assert (lg[~fin] == lse_ref[~fin]).all(), f"{what}: LSE infinities differ"
        if fin.any():
            lse_err = max(lse_err, float(np.abs(lg[fin] - lse_ref[fin]).max()))
    if dtype == "fp32":
        o_err = diff_max / ref_max if ref_max > 0 else diff_max
        assert o_err <= TOL_O_32_NORMWISE, f"{what}: fp32 O normwise error {o_err:.3e}"
    else:
        o_err = diff_max
        assert o_err <= TOL_O_16, f"{what}: O max abs error {o_err:.3e} at {worst}"
    assert lse_err <= TOL_LSE, f"{what}: LSE max abs error {lse_err:.3e}"
    return o_err, lse_err, worst


def reference_full(q_bits, k_bits, v_bits, dtype, scale, causal, n_kv=None):
    q, k, v = (fa_inputs.to_f32(x, dtype) for x in (q_bits, k_bits, v_bits))
    return oracle.attention(q, k, v, scale, causal, n_kv=n_kv)


def reference_full_ex(q_bits, k_bits, v_bits, dtype, scale, causal, causal_align):
    """Oracle for separate query and key lengths (q [B,H,Nq,D], k/v [B,H,Nk,D])."""
    q, k, v = (fa_inputs.to_f32(x, dtype) for x in (q_bits, k_bits, v_bits))
    return oracle.attention(q, k, v, scale, causal, causal_align=causal_align)


def reference_rows(q_bits, k_bits, v_bits, dtype, scale, causal, rows, n_kv=None):
    q, k, v = (fa_inputs.to_f32(x, dtype) for x in (q_bits, k_bits, v_bits))
    return oracle.attention_rows(q, k, v, scale, causal, rows, n_kv=n_kv)


def default_scale(D):
    return 1.0 / math.sqrt(D)


def check_grad(g_gpu, g_ref, dtype, what=""):
    """Normwise parity of one gradient tensor; returns the error."""
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    assert np.isfinite(g_gpu).all(), f"{what}: non-finite gradient"
    ref_max = np.abs(g_ref).max() if g_ref.size else 0.0
    diff = np.abs(g_gpu - g_ref).max() if g_ref.size else 0.0
    err = diff / ref_max if ref_max > 0 else diff
    assert err <= TOL_GRAD[dtype], f"{what}: normwise gradient error {err:.3e}"
    return err
