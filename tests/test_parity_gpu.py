"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle.

Small shapes and the full-size workloads are compared on every output
element; the full-size workloads run in the launch configuration the
benchmark times (fa_fwd, variant 0). Other full-size cases (long keys,
paired causal grids) are compared on sampled rows that the oracle computes
one by one.
"""
import math
import sys

import numpy as np
import pytest

import exact_attention_10_amd as fa
import fa_inputs
import oracle
from tests import parity

pytestmark = pytest.mark.gpu

DTYPES = ["fp32", "fp16", "bf16"]


def _banner(msg):
    print(f"\n[case] {msg}", flush=True)
    sys.stdout.flush()


def _run(qb, kb, vb, dtype, causal, scale, n_kv=None, variant=None):
    import torch
    q, k, v = (parity.to_device(x, dtype) for x in (qb, kb, vb))
    if variant is not None:
        o, lse = fa.fa_fwd_variant(q, k, v, causal=causal, scale=scale, variant=variant,
                                   n_kv=n_kv)
    elif n_kv is not None:
        o, lse = fa.fa_fwd_nk(q, k, v, n_kv=n_kv, causal=causal, scale=scale)
    else:
        o, lse = fa.fa_fwd(q, k, v, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return parity.from_device(o), lse.cpu().numpy()


# ---------------------------------------------------------------------------
# Small shapes, every element: several query/key tiles and ragged tails


@pytest.mark.parametrize("N", [1, 37, 64, 127, 128, 129, 200, 383])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", DTYPES)
def test_small_full_parity(dtype, D, causal, N):
    _banner(f"small dtype={dtype} D={D} causal={causal} N={N}")
    B, H = 2, 3
    seed = 1000 + N + D + (7 if causal else 0) + DTYPES.index(dtype)
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, seed)
    scale = parity.default_scale(D)
    o, lse = _run(qb, kb, vb, dtype, causal, scale)
    o_ref, lse_ref = parity.reference_full(qb, kb, vb, dtype, scale, causal)
    parity.check(o, lse, o_ref, lse_ref, dtype, f"{dtype} D={D} causal={causal} N={N}")


@pytest.mark.parametrize("n_kv", [0, 1, 63, 64, 65, 150, 257])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_key_length_mask(dtype, causal, n_kv):
    """Keys >= n_kv are invisible; n_kv = 0 leaves every row without a key:
    O = 0 and LSE = -inf exactly (the guard for fully masked rows)."""
    _banner(f"n_kv dtype={dtype} causal={causal} n_kv={n_kv}")
    B, H, N, D = 1, 2, 257, 64
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 77 + n_kv)
    scale = parity.default_scale(D)
    o, lse = _run(qb, kb, vb, dtype, causal, scale, n_kv=n_kv)
    o_ref, lse_ref = parity.reference_full(qb, kb, vb, dtype, scale, causal, n_kv=n_kv)
    parity.check(o, lse, o_ref, lse_ref, dtype, f"n_kv={n_kv}")
    if n_kv == 0:
        assert (o == 0).all() and np.isneginf(lse).all()


VARIANTS = ["default", "simple_bm128_xcd", "simple_bm128_linear", "simple_bm256_xcd",
            "simple_bm256_linear", "twogroup_bm256_xcd", "twogroup16_bm256_xcd",
            "simple16_bm128_xcd", "simple16_bm256_xcd"]


def test_variant_list():
    assert [fa.fa_variant_name(i) for i in range(fa.fa_num_variants())] == VARIANTS


@pytest.mark.parametrize("name", VARIANTS)
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 128), ("fp16", 64), ("fp32", 64)])
def test_variants(name, causal, dtype, D):
    """Every kernel variant (tile shape / schedule / workgroup order) computes
    the same attention; variants that only reorder workgroups agree bitwise.
    The 8-wave schedules exist for 16-bit inputs only: fp32 is rejected; the
    two-group schedule on 32x32x16 MFMAs has no causal mask either."""
    variant = VARIANTS.index(name)
    _banner(f"variant {variant} ({name}) dtype={dtype} D={D} causal={causal}")
    B, H, N = 2, 4, 520
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 500 + variant)
    scale = parity.default_scale(D)
    unsupported = (dtype == "fp32" and name != "default" and not name.startswith("simple_bm128")) \
        or (name == "twogroup_bm256_xcd" and causal)
    if unsupported:
        with pytest.raises(fa.FAError):
            _run(qb, kb, vb, dtype, causal, scale, variant=variant)
        return
    o, lse = _run(qb, kb, vb, dtype, causal, scale, variant=variant)
    o_ref, lse_ref = parity.reference_full(qb, kb, vb, dtype, scale, causal)
    parity.check(o, lse, o_ref, lse_ref, dtype, f"variant {name}")
    if name.endswith("_xcd"):
        linear = [i for i in range(fa.fa_num_variants())
                  if fa.fa_variant_name(i) == name[:-4] + "_linear"]
        if linear:
            o2, l2 = _run(qb, kb, vb, dtype, causal, scale, variant=linear[0])
            assert np.array_equal(o, o2) and np.array_equal(lse, l2), "workgroup order changed bits"


@pytest.mark.parametrize("n_kv", [0, 1, 63, 64, 65, 128, 191, 192, 193, 255, 256, 257, 320,
                                  449, 520])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("vname", ["twogroup_bm256_xcd", "twogroup16_bm256_xcd"])
def test_twogroup_key_tails(vname, dtype, D, n_kv):
    """The two-group schedule streams 64-key tiles through four LDS stages
    per matrix, loads K three tiles and V two tiles ahead, and unrolls its
    loop by four periods: key counts from none to a ragged last tile, after
    every remainder of tiles modulo 4, with a ragged query tail (520 = 2 * 256
    + 8 rows), every element against the oracle."""
    _banner(f"{vname} dtype={dtype} D={D} n_kv={n_kv}")
    B, H, N = 1, 2, 520
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 900 + n_kv + D)
    scale = parity.default_scale(D)
    o, lse = _run(qb, kb, vb, dtype, False, scale, n_kv=n_kv, variant=VARIANTS.index(vname))
    o_ref, lse_ref = parity.reference_full(qb, kb, vb, dtype, scale, False, n_kv=n_kv)
    parity.check(o, lse, o_ref, lse_ref, dtype, f"{vname} n_kv={n_kv}")
    if n_kv == 0:
        assert (o == 0).all() and np.isneginf(lse).all()


@pytest.mark.parametrize("n_kv", [0, 1, 31, 63, 65, 128, 160, 192, 257, 383, 449, 520])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 64)])
@pytest.mark.parametrize("vname", ["simple16_bm128_xcd", "simple16_bm256_xcd", "twogroup16_bm256_xcd"])
def test_causal_16x16x32_key_tails(vname, dtype, D, n_kv):
    """The causal kernels on 16x16x32 MFMAs. The simple schedule splits its
    key loop at each wave's last visible tile: full steps up to it, then steps
    that only keep the workgroup's barriers and transfers going, starting on
    either LDS buffer. The two-group schedule has every wave compute every
    tile of its workgroup, masked past the wave's rows, through its four-stage
    rings. Key counts that end before, on and past the diagonal of each query
    tile, with a ragged query tail (520 rows), every element against the
    oracle."""
    _banner(f"{vname} causal dtype={dtype} D={D} n_kv={n_kv}")
    B, H, N = 1, 2, 520
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 1900 + n_kv + D)
    scale = parity.default_scale(D)
    o, lse = _run(qb, kb, vb, dtype, True, scale, n_kv=n_kv, variant=VARIANTS.index(vname))
    o_ref, lse_ref = parity.reference_full(qb, kb, vb, dtype, scale, True, n_kv=n_kv)
    parity.check(o, lse, o_ref, lse_ref, dtype, f"{vname} causal n_kv={n_kv}")
    if n_kv == 0:
        assert (o == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------------------
# Separate query and key lengths (fa_fwd_ex), both causal alignments


def _run_ex(qb, kb, vb, dtype, causal, align, scale):
    import torch
    q, k, v = (parity.to_device(x, dtype) for x in (qb, kb, vb))
    o, lse = fa.fa_fwd_ex(q, k, v, causal=causal, causal_align=align, scale=scale)
    torch.cuda.synchronize()
    return parity.from_device(o), lse.cpu().numpy()


CROSS_SHAPES = [(1, 2), (37, 200), (200, 37), (128, 300), (300, 129), (1, 513), (64, 64)]
MASKS = [(False, "top-left"), (True, "top-left"), (True, "bottom-right")]


@pytest.mark.parametrize("causal,align", MASKS)
@pytest.mark.parametrize("nq,nk", CROSS_SHAPES)
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 64), ("bf16", 64), ("fp32", 64)])
def test_cross_attention_full_parity(dtype, D, nq, nk, causal, align):
    _banner(f"cross dtype={dtype} D={D} Nq={nq} Nk={nk} causal={causal} {align}")
    B, H = 2, 3
    seed = 3000 + nq * 7 + nk + D + DTYPES.index(dtype) + (11 if causal else 0) + (5 if align == "bottom-right" else 0)
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, dtype, seed)
    scale = parity.default_scale(D)
    o, lse = _run_ex(qb, kb, vb, dtype, causal, align, scale)
    o_ref, lse_ref = parity.reference_full_ex(qb, kb, vb, dtype, scale, causal, align)
    parity.check(o, lse, o_ref, lse_ref, dtype, f"cross {dtype} D={D} {nq}x{nk} {causal} {align}")


# The test matrix of "FlashAttention 2 from PyTorch to Triton" (Step 3): shapes
# (batch, query rows, key rows, head dim) without a head axis (H = 1), fp32 and
# bf16, causal only where the matrix is square. Its (1, 37, 53, 32) entry has a
# head dimension outside {64, 128}, which the library rejects as unsupported.
PAGE_MATRIX = [(4, 128, 128, 64), (2, 1024, 1024, 64), (2, 100, 100, 64), (1, 200, 96, 128)]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("B,nq,nk,D", PAGE_MATRIX)
def test_pages_test_matrix(B, nq, nk, D, dtype):
    _banner(f"pages' matrix B={B} Nq={nq} Nk={nk} D={D} {dtype}")
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, 1, nq, nk, D, dtype, 9000 + nq + nk + D)
    scale = parity.default_scale(D)
    for causal in ((False, True) if nq == nk else (False,)):
        o, lse = _run_ex(qb, kb, vb, dtype, causal, "top-left", scale)
        o_ref, lse_ref = parity.reference_full_ex(qb, kb, vb, dtype, scale, causal, "top-left")
        parity.check(o, lse, o_ref, lse_ref, dtype, f"pages' matrix {B}x{nq}x{nk}x{D} causal={causal}")


def test_pages_test_matrix_head_dim_32_is_rejected():
    import torch
    qb, kb, vb = fa_inputs.draw_qkv_cross(1, 1, 37, 53, 32, "bf16", 9001)
    q, k, v = (parity.to_device(x, "bf16") for x in (qb, kb, vb))
    with pytest.raises(fa.FAError):
        fa.fa_fwd_ex(q, k, v, causal=False)


def test_cross_attention_one_query_two_keys():
    """One query, two keys, equal scores, value rows 5 and 10: O = 7.5 and
    LSE = ln 2 exactly representable; top-left causal sees key 0 only (O = 5)."""
    import torch
    _banner("cross one query two keys")
    D = 64
    q = torch.zeros(1, 1, 1, D, dtype=torch.bfloat16, device="cuda")
    k = torch.randn(1, 1, 2, D, device="cuda").to(torch.bfloat16)
    v = torch.tensor([5.0, 10.0], device="cuda").view(1, 1, 2, 1).expand(1, 1, 2, D)
    v = v.to(torch.bfloat16).contiguous()
    for causal, align, want, lse_want in ((False, "top-left", 7.5, math.log(2.0)),
                                          (True, "bottom-right", 7.5, math.log(2.0)),
                                          (True, "top-left", 5.0, 0.0)):
        o, lse = fa.fa_fwd_ex(q, k, v, causal=causal, causal_align=align)
        torch.cuda.synchronize()
        assert (o.float() == want).all(), (causal, align, o.float().unique())
        assert abs(float(lse) - lse_want) <= 1e-6, (causal, align, float(lse))


def test_cross_attention_equal_lengths_match_fa_fwd():
    """fa_fwd_ex with Nq = Nk (either alignment) is bit-identical to fa_fwd."""
    import torch
    _banner("cross equal lengths == fa_fwd")
    qb, kb, vb = fa_inputs.draw_qkv(2, 4, 333, 128, "bf16", 77)
    q, k, v = (parity.to_device(x, "bf16") for x in (qb, kb, vb))
    for causal in (False, True):
        o1, l1 = fa.fa_fwd(q, k, v, causal=causal)
        for align in ("top-left", "bottom-right"):
            o2, l2 = fa.fa_fwd_ex(q, k, v, causal=causal, causal_align=align)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_cross_attention_long_keys_sampled():
    """A longer cross-attention case (Nq = 1000, Nk = 5000, D = 128, bf16,
    causal bottom-right) checked on sampled rows, including the first rows,
    whose visible range starts at Nk - Nq keys."""
    _banner("cross long keys sampled rows")
    B, H, nq, nk, D = 1, 4, 1000, 5000, 128
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, "bf16", 4242)
    scale = parity.default_scale(D)
    o, lse = _run_ex(qb, kb, vb, "bf16", True, "bottom-right", scale)
    rows = parity.sample_rows(B, H, nq, 200, 99)
    q, k, v = (fa_inputs.to_f32(x, "bf16") for x in (qb, kb, vb))
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, True, rows, causal_align="bottom-right")
    o_s = o.reshape(B * H, nq, D)[rows[:, 0], rows[:, 1]]
    l_s = lse.reshape(B * H, nq)[rows[:, 0], rows[:, 1]]
    parity.check(o_s, l_s, o_ref, lse_ref, "bf16", "cross long keys")


@pytest.mark.parametrize("causal,align", [(False, "top-left"), (True, "bottom-right")])
def test_longest_key_sequence(causal, align):
    """The largest key length one head may have at D = 128 bf16: the K and V
    heads are 2^31 - 256 bytes, the limit of the kernels' 32-bit byte offsets
    (one key more is rejected on the host). Three query rows over 8388607 keys
    (the last tile ragged), single pass and split-KV, against the oracle; the
    O check is also held to |O| of order 1 (a near-uniform average of 8M
    values would be ~0 and pass any absolute tolerance)."""
    D = 128
    nk = (2 ** 31 - 1) // (D * 2)
    nq = 3
    _banner(f"longest key sequence Nk={nk} causal={causal} {align}")
    qb, kb, vb = fa_inputs.draw_qkv_cross(1, 1, nq, nk, D, "bf16", 4343)
    # Q x 8 (exact): the softmax concentrates on a few of the 8M keys, so O is
    # of order 1 and its check is not trivially met
    qb = fa_inputs.round_to_dtype(fa_inputs.to_f32(qb, "bf16") * 8.0, "bf16")
    scale = parity.default_scale(D)
    o1, l1 = _run_ex(qb, kb, vb, "bf16", causal, align, scale)
    o2, l2 = _run_split(qb, kb, vb, "bf16", causal, align, scale, 0)
    rows = np.array([[0, i] for i in range(nq)])
    q, k, v = (fa_inputs.to_f32(x, "bf16") for x in (qb, kb, vb))
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, causal, rows, causal_align=align)
    for what, o, l in (("single pass", o1, l1), ("split-KV", o2, l2)):
        oe, le = parity.check(o.reshape(nq, D), l.reshape(nq), o_ref, lse_ref, "bf16",
                              f"longest keys {what}")
        print(f"[parity] longest keys {what} causal={causal}: O err {oe:.2e} LSE err {le:.2e}",
              flush=True)
    assert np.abs(o_ref).max() > 0.5


@pytest.mark.parametrize("dtype,D", [("fp32", 64), ("fp16", 64), ("fp16", 128)])
def test_paired_causal_dtypes_sampled(dtype, D):
    """Causal grids of 32 heads at N = 4096 pair query tiles for every dtype
    (the fp32 and fp16 instances share the pairing with bf16); sampled rows,
    including both ends of every paired tile, against the oracle."""
    B, H, N = 4, 8, 4096
    _banner(f"paired causal dtype={dtype} D={D}")
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 5300 + D + (1 if dtype == "fp16" else 0))
    scale = parity.default_scale(D)
    o, lse = _run(qb, kb, vb, dtype, True, scale)
    o = o.reshape(B * H, N, D)
    lse = lse.reshape(B * H, N)
    bm = 128 if (dtype == "fp32" or D == 64) else 256
    rows = parity.sample_rows(B, H, N, 200, seed=D + 3, bm=bm)
    o_ref, lse_ref = parity.reference_rows(qb, kb, vb, dtype, scale, True, rows)
    parity.check(o[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], o_ref, lse_ref, dtype,
                 f"paired causal {dtype} D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_paired_causal_odd_tiles_sampled(D):
    """129 heads of 600 rows: an odd number of query tiles (and of the
    backward's key tiles), so one workgroup per head runs the middle tile
    alone, on a paired grid whose size is not a multiple of 8 (no XCD
    reordering). Forward on sampled rows, dQ, dK, dV of three heads."""
    B, H, N = 1, 129, 600
    _banner(f"paired causal odd tiles D={D}")
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, "bf16", 5400 + D)
    dob = fa_inputs.draw_qkv(B, H, N, D, "bf16", 5401 + D)[0]
    scale = parity.default_scale(D)
    dq, dk, dv, _, o = _run_fwd_bwd(qb, kb, vb, dob, "bf16", True, "top-left", scale)
    o = o.reshape(B * H, N, D)
    bm = 128 if D == 64 else 256
    rows = parity.sample_rows(B, H, N, 160, seed=D + 11, bm=bm)
    q, k, v, do = (fa_inputs.to_f32(x, "bf16") for x in (qb, kb, vb, dob))
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, True, rows)
    parity.check(o[rows[:, 0], rows[:, 1]], None, o_ref, lse_ref, "bf16", f"odd tiles fwd D={D}")
    rng = np.random.default_rng(D)
    edge = np.array([0, 127, 128, 255, 256, 383, 384, 511, 512, N - 1])
    for h in (0, H // 2, H - 1):
        r = np.unique(np.concatenate([edge, rng.integers(0, N, 12)]))
        dq_r, dk_r, dv_r = oracle.attention_bwd_sampled(q[0, h], k[0, h], v[0, h], do[0, h],
                                                        scale, True, r, r)
        for n, g, ref in (("dQ", dq[0, h, r], dq_r), ("dK", dk[0, h, r], dk_r),
                          ("dV", dv[0, h, r], dv_r)):
            parity.check_grad(g, ref, "bf16", f"odd tiles bwd D={D} head {h} {n}")


@pytest.mark.parametrize("n_kv", [0, 1, 300, 599])
def test_paired_causal_key_length_mask_sampled(n_kv):
    """The key-length mask on a paired causal grid (129 heads x 3 tiles of
    256 rows): sampled rows against the oracle with the same n_kv."""
    B, H, N, D = 1, 129, 600, 128
    _banner(f"paired causal n_kv={n_kv}")
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, "bf16", 5500 + n_kv)
    scale = parity.default_scale(D)
    o, lse = _run(qb, kb, vb, "bf16", True, scale, n_kv=n_kv)
    o = o.reshape(B * H, N, D)
    lse = lse.reshape(B * H, N)
    rows = parity.sample_rows(B, H, N, 160, seed=n_kv, bm=256)
    o_ref, lse_ref = parity.reference_rows(qb, kb, vb, "bf16", scale, True, rows, n_kv=n_kv)
    parity.check(o[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], o_ref, lse_ref, "bf16",
                 f"paired causal n_kv={n_kv}")


@pytest.mark.parametrize("align", ["top-left", "bottom-right"])
@pytest.mark.parametrize("D", [64, 128])
def test_paired_causal_cross_sampled(D, align):
    """Causal grids large enough for paired query / key tiles (128 heads),
    with Nq != Nk and both alignments: the forward on sampled rows and the
    backward (dQ rows, dK/dV key rows) of two heads against the oracle."""
    B, H, nq, nk = 8, 16, 1000, 2500
    _banner(f"paired causal cross D={D} {align}")
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, "bf16", 5150 + D)
    dob = fa_inputs.draw_qkv_cross(B, H, nq, 1, D, "bf16", 5151 + D)[0]
    scale = parity.default_scale(D)
    dq, dk, dv, _, o = _run_fwd_bwd(qb, kb, vb, dob, "bf16", True, align, scale)
    o = o.reshape(B * H, nq, D)
    rows = parity.sample_rows(B, H, nq, 160, seed=D)
    q, k, v, do = (fa_inputs.to_f32(x, "bf16") for x in (qb, kb, vb, dob))
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, True, rows, causal_align=align)
    parity.check(o[rows[:, 0], rows[:, 1]], None, o_ref, lse_ref, "bf16", f"paired fwd {align}")
    rng = np.random.default_rng(D)
    edge = np.array([0, 1, 127, 128, nq - 1])
    for b, h in ((0, 0), (B - 1, H - 1)):
        r = np.unique(np.concatenate([edge, rng.integers(0, nq, 16)]))
        c = np.unique(np.concatenate([[0, 127, 128, nk - nq - 1, nk - nq, nk - 1],
                                      rng.integers(0, nk, 16)]))
        dq_r, dk_r, dv_r = oracle.attention_bwd_sampled(q[b, h], k[b, h], v[b, h], do[b, h],
                                                        scale, True, r, c, causal_align=align)
        for n, g, ref in (("dQ", dq[b, h, r], dq_r), ("dK", dk[b, h, c], dk_r),
                          ("dV", dv[b, h, c], dv_r)):
            parity.check_grad(g, ref, "bf16", f"paired bwd {align} head ({b},{h}) {n}")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 128), ("bf16", 64)])
def test_paired_causal_more_queries_than_keys(dtype, D):
    """Bottom-right causal with Nq > Nk on a grid large enough to pair query
    tiles: the diagonal offset Nk - Nq is negative, so the first Nq - Nk rows
    see no key (O = 0, LSE = -inf) and whole query tiles, and whole waves of
    the tiles that straddle that boundary, have nothing to compute. Every row
    of two heads and sampled rows of the rest, O and LSE against the oracle."""
    B, H, nq, nk = 8, 16, 2500, 1000
    _banner(f"paired causal Nq > Nk dtype={dtype} D={D}")
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, dtype, 6160 + D)
    scale = parity.default_scale(D)
    o, lse = _run_ex(qb, kb, vb, dtype, True, "bottom-right", scale)
    o = o.reshape(B * H, nq, D)
    lse = lse.reshape(B * H, nq)
    full = np.array([(bh, i) for bh in (0, B * H - 1) for i in range(nq)], dtype=np.int64)
    rows = np.unique(np.concatenate([full, parity.sample_rows(B, H, nq, 300, seed=D)]), axis=0)
    q, k, v = (fa_inputs.to_f32(x, dtype) for x in (qb, kb, vb))
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, True, rows, causal_align="bottom-right")
    parity.check(o[rows[:, 0], rows[:, 1]], lse[rows[:, 0], rows[:, 1]], o_ref, lse_ref, dtype,
                 f"paired causal Nq > Nk {dtype} D={D}")
    assert (o[:, : nq - nk] == 0).all() and np.isneginf(lse[:, : nq - nk]).all()


# ---------------------------------------------------------------------------
# Split-KV (fa_fwd_splitkv): the same attention, keys split over workgroups


def _run_split(qb, kb, vb, dtype, causal, align, scale, num_splits, poison=True):
    import torch
    q, k, v = (parity.to_device(x, dtype) for x in (qb, kb, vb))
    B, H, nq, D = q.shape
    nk = k.shape[2]
    need = fa.fa_fwd_splitkv_workspace_size(B, H, nq, nk, D, num_splits)
    ws = None
    if need:
        # the workspace's contents on entry must not matter: fill it with NaNs
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        if poison:
            ws.view(torch.float32)[: need // 4].fill_(float("nan"))
    o, lse = fa.fa_fwd_splitkv(q, k, v, causal=causal, causal_align=align, scale=scale,
                               num_splits=num_splits, workspace=ws)
    torch.cuda.synchronize()
    return parity.from_device(o), lse.cpu().numpy()


@pytest.mark.parametrize("num_splits", [2, 5, 32])
@pytest.mark.parametrize("causal,align", MASKS)
@pytest.mark.parametrize("nq,nk", [(37, 200), (128, 300), (300, 129), (1, 513), (200, 37)])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("fp16", 64), ("fp32", 64)])
def test_splitkv_full_parity(dtype, D, nq, nk, causal, align, num_splits):
    _banner(f"splitkv dtype={dtype} D={D} Nq={nq} Nk={nk} causal={causal} {align} splits={num_splits}")
    B, H = 2, 2
    seed = 5000 + nq + 3 * nk + D + num_splits + DTYPES.index(dtype) + (7 if causal else 0)
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, dtype, seed)
    scale = parity.default_scale(D)
    o, lse = _run_split(qb, kb, vb, dtype, causal, align, scale, num_splits)
    o_ref, lse_ref = parity.reference_full_ex(qb, kb, vb, dtype, scale, causal, align)
    parity.check(o, lse, o_ref, lse_ref, dtype,
                 f"splitkv {dtype} D={D} {nq}x{nk} {causal} {align} s={num_splits}")


@pytest.mark.parametrize("num_splits", [0, 4])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_small_grid_workload(causal, num_splits):
    """The [B=8, N=1024, D=64] bf16 workload (64 workgroups of 128 query rows),
    with the library's split choice and with 4 splits, every output element
    against the oracle."""
    name = "b8h1_n1024_d64_bf16"
    _banner(f"splitkv {name} causal={causal} splits={num_splits}")
    w = fa_inputs.WORKLOADS[name]
    qb, kb, vb = fa_inputs.workload_inputs(w)
    o, lse = _run_split(qb, kb, vb, w.dtype, causal, "top-left", w.scale, num_splits)
    o_ref, lse_ref = parity.reference_full(qb, kb, vb, w.dtype, w.scale, causal)
    parity.check(o, lse, o_ref, lse_ref, w.dtype, f"splitkv {name} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_long_keys_sampled(causal):
    """One query tile over 16384 keys (D = 128, bf16): the library picks 32
    splits; sampled rows against the oracle."""
    _banner(f"splitkv long keys causal={causal}")
    B, H, nq, nk, D = 1, 2, 200, 16384, 128
    assert fa.fa_splitkv_auto_splits(B, H, nq, nk, D) > 8
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, "bf16", 8080 + causal)
    scale = parity.default_scale(D)
    o, lse = _run_split(qb, kb, vb, "bf16", causal, "bottom-right", scale, 0)
    rows = parity.sample_rows(B, H, nq, 80, 5)
    q, k, v = (fa_inputs.to_f32(x, "bf16") for x in (qb, kb, vb))
    o_ref, lse_ref = oracle.attention_rows(q, k, v, scale, causal, rows, causal_align="bottom-right")
    o_s = o.reshape(B * H, nq, D)[rows[:, 0], rows[:, 1]]
    l_s = lse.reshape(B * H, nq)[rows[:, 0], rows[:, 1]]
    parity.check(o_s, l_s, o_ref, lse_ref, "bf16", "splitkv long keys")


def test_splitkv_one_split_is_single_pass():
    """num_splits = 1 runs the single-pass kernel: bit-identical to fa_fwd_ex."""
    import torch
    _banner("splitkv one split")
    qb, kb, vb = fa_inputs.draw_qkv_cross(1, 3, 150, 400, 128, "bf16", 61)
    q, k, v = (parity.to_device(x, "bf16") for x in (qb, kb, vb))
    o1, l1 = fa.fa_fwd_ex(q, k, v, causal=True, causal_align="bottom-right")
    o2, l2 = fa.fa_fwd_splitkv(q, k, v, causal=True, causal_align="bottom-right", num_splits=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_splitkv_workspace_reuse():
    """Two calls in a row on one workspace, the second smaller: both correct."""
    import torch
    _banner("splitkv workspace reuse")
    big = fa_inputs.draw_qkv_cross(2, 2, 256, 1000, 64, "bf16", 71)
    small = fa_inputs.draw_qkv_cross(1, 1, 64, 300, 64, "bf16", 72)
    need = fa.fa_fwd_splitkv_workspace_size(2, 2, 256, 1000, 64, 6)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for qb, kb, vb in (big, small):
        q, k, v = (parity.to_device(x, "bf16") for x in (qb, kb, vb))
        o, lse = fa.fa_fwd_splitkv(q, k, v, causal=True, num_splits=6, workspace=ws)
        torch.cuda.synchronize()
        o_ref, lse_ref = parity.reference_full_ex(qb, kb, vb, "bf16", 0.125, True, "top-left")
        parity.check(parity.from_device(o), lse.cpu().numpy(), o_ref, lse_ref, "bf16", "reuse")


# ---------------------------------------------------------------------------
# Backward (fa_bwd) against the fp64 backward oracle


def _run_fwd_bwd(qb, kb, vb, dob, dtype, causal, align, scale):
    import torch
    q, k, v, do = (parity.to_device(x, dtype) for x in (qb, kb, vb, dob))
    o, lse = fa.fa_fwd_ex(q, k, v, causal=causal, causal_align=align, scale=scale)
    dq, dk, dv, delta = fa.fa_bwd(q, k, v, o, do, lse, causal=causal, causal_align=align,
                                  scale=scale)
    torch.cuda.synchronize()
    return (parity.from_device(dq), parity.from_device(dk), parity.from_device(dv),
            delta.cpu().numpy(), parity.from_device(o))


def test_binding_rejects_mismatched_delta_and_workspace():
    """Caller-provided buffers the kernels write are checked before any launch:
    a too-short or wrongly typed delta for fa_bwd, a workspace on the host for
    fa_fwd_splitkv."""
    import torch
    _banner("binding checks of delta and workspace")
    qb, kb, vb = fa_inputs.draw_qkv(1, 2, 64, 64, "bf16", 77)
    q, k, v = (parity.to_device(x, "bf16") for x in (qb, kb, vb))
    o, lse = fa.fa_fwd(q, k, v)
    for bad in (torch.empty((1, 2, 32), dtype=torch.float32, device=q.device),
                torch.empty((1, 2, 64), dtype=torch.float16, device=q.device)):
        with pytest.raises(ValueError):
            fa.fa_bwd(q, k, v, o, o, lse, delta=bad)
    with pytest.raises(ValueError):
        fa.fa_fwd_splitkv(q, k, v, num_splits=2, workspace=torch.empty(1 << 20, dtype=torch.uint8))
    torch.cuda.synchronize()


BWD_SHAPES = [(64, 64), (130, 130), (37, 200), (200, 37), (1, 65), (128, 300), (257, 511)]


@pytest.mark.parametrize("causal,align", MASKS)
@pytest.mark.parametrize("nq,nk", BWD_SHAPES)
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("fp16", 128), ("fp16", 64)])
def test_bwd_parity(dtype, D, nq, nk, causal, align):
    _banner(f"bwd dtype={dtype} D={D} Nq={nq} Nk={nk} causal={causal} {align}")
    B, H = 2, 2
    seed = 7000 + nq * 3 + nk + D + (1 if dtype == "fp16" else 0) + (5 if causal else 0) \
        + (9 if align == "bottom-right" else 0)
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, nq, nk, D, dtype, seed)
    dob = fa_inputs.draw_qkv_cross(B, H, nq, 1, D, dtype, seed + 1)[0]
    scale = parity.default_scale(D)
    dq, dk, dv, delta, o = _run_fwd_bwd(qb, kb, vb, dob, dtype, causal, align, scale)
    q, k, v, do = (fa_inputs.to_f32(x, dtype) for x in (qb, kb, vb, dob))
    dq_r, dk_r, dv_r = oracle.attention_bwd(q, k, v, do, scale, causal, align)
    what = f"bwd {dtype} D={D} {nq}x{nk} {causal} {align}"
    errs = [parity.check_grad(g, r, dtype, f"{what} {n}")
            for n, g, r in (("dQ", dq, dq_r), ("dK", dk, dk_r), ("dV", dv, dv_r))]
    d_ref = (do.astype(np.float64) * o.astype(np.float64)).sum(-1)
    d_err = np.abs(delta - d_ref).max() / max(1e-30, np.abs(d_ref).max())
    print(f"[bwd errors] {what}: dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e} D {d_err:.2e}",
          flush=True)
    assert d_err <= parity.TOL_DELTA, f"{what}: D error {d_err:.3e}"


def test_bwd_unseen_keys_and_rows_are_zero():
    """Top-left causal with more keys than queries: keys j >= Nq are seen by no
    query, so dK and dV are exactly 0 there; bottom-right with more queries
    than keys: rows i < Nq - Nk see no key and get dQ = 0 exactly."""
    import torch
    _banner("bwd unseen keys / rows")
    for nq, nk, align in ((100, 300, "top-left"), (300, 100, "bottom-right")):
        qb, kb, vb = fa_inputs.draw_qkv_cross(1, 2, nq, nk, 128, "bf16", 91)
        dob = fa_inputs.draw_qkv_cross(1, 2, nq, 1, 128, "bf16", 92)[0]
        dq, dk, dv, _, _ = _run_fwd_bwd(qb, kb, vb, dob, "bf16", True, align, 128 ** -0.5)
        if nk > nq:
            assert (dk[:, :, nq:] == 0).all() and (dv[:, :, nq:] == 0).all()
        else:
            assert (dq[:, :, : nq - nk] == 0).all()


BWD_FULL_SIZE = [(fa_inputs.HEADLINE, False), (fa_inputs.HEADLINE, True),
                 ("b2h16_n4000_d128_fp16", False), ("b2h16_n4000_d128_fp16", True),
                 ("b4h16_n4096_d64_bf16", False), ("b4h16_n4096_d64_bf16", True)]


@pytest.mark.parametrize("name,causal", BWD_FULL_SIZE,
                         ids=[f"{n}-{'causal' if c else 'full'}" for n, c in BWD_FULL_SIZE])
def test_bwd_full_size_sampled(name, causal):
    """The backward at a workload's full size, in the launch configuration the
    benchmark times (fa_fwd then fa_bwd over the whole batch): dQ on sampled
    query rows and dK, dV on sampled key rows of three heads, against the
    oracle's element-by-element gradients of those heads."""
    w = fa_inputs.WORKLOADS[name]
    _banner(f"bwd full size {name} causal={causal}")
    qb, kb, vb = fa_inputs.workload_inputs(w)
    dob = fa_inputs.draw_qkv_cross(w.B, w.H, w.N, 1, w.D, w.dtype, w.seed + 1000)[0]
    dq, dk, dv, _, _ = _run_fwd_bwd(qb, kb, vb, dob, w.dtype, causal, "top-left", w.scale)
    rng = np.random.default_rng(w.seed + 2000)
    heads = [(0, 0), (w.B - 1, w.H - 1), (int(rng.integers(w.B)), int(rng.integers(w.H)))]
    edge = np.array([0, 1, 63, 64, 127, 128, w.N - 65, w.N - 64, w.N - 1])
    for b, h in heads:
        rows = np.unique(np.concatenate([edge, rng.integers(0, w.N, 24)]))
        cols = np.unique(np.concatenate([edge, rng.integers(0, w.N, 24)]))
        q, k, v, do = (fa_inputs.to_f32(x[b, h], w.dtype) for x in (qb, kb, vb, dob))
        dq_r, dk_r, dv_r = oracle.attention_bwd_sampled(q, k, v, do, w.scale, causal, rows, cols)
        what = f"bwd {name} causal={causal} head ({b},{h})"
        errs = [parity.check_grad(g, r, w.dtype, f"{what} {n}")
                for n, g, r in (("dQ", dq[b, h, rows], dq_r), ("dK", dk[b, h, cols], dk_r),
                                ("dV", dv[b, h, cols], dv_r))]
        print(f"[bwd full size] {what}: dQ {errs[0]:.2e} dK {errs[1]:.2e} dV {errs[2]:.2e}",
              flush=True)
    assert np.isfinite(dq).all() and np.isfinite(dk).all() and np.isfinite(dv).all()


def test_bwd_bitwise_deterministic():
    import torch
    _banner("bwd determinism")
    qb, kb, vb = fa_inputs.draw_qkv_cross(2, 4, 300, 300, 128, "bf16", 93)
    dob = fa_inputs.draw_qkv_cross(2, 4, 300, 1, 128, "bf16", 94)[0]
    r1 = _run_fwd_bwd(qb, kb, vb, dob, "bf16", True, "top-left", 128 ** -0.5)
    r2 = _run_fwd_bwd(qb, kb, vb, dob, "bf16", True, "top-left", 128 ** -0.5)
    assert all(np.array_equal(a, b) for a, b in zip(r1, r2))


def test_no_lse_output():
    import torch
    _banner("lse = NULL")
    qb, kb, vb = fa_inputs.draw_qkv(1, 2, 300, 64, "bf16", 9)
    q, k, v = (parity.to_device(x, "bf16") for x in (qb, kb, vb))
    o, lse = fa.fa_fwd(q, k, v, causal=True, with_lse=False)
    torch.cuda.synchronize()
    assert lse is None
    o_ref, _ = parity.reference_full(qb, kb, vb, "bf16", 1 / 8, True)
    parity.check(parity.from_device(o), None, o_ref, None, "bf16", "no lse")


# ---------------------------------------------------------------------------
# Closed forms and invariants on the GPU


@pytest.mark.parametrize("dtype", DTYPES)
def test_causal_first_row_is_first_value(dtype):
    """Query 0 sees only key 0: O[0] = V[0] (bit-exact after rounding to a
    16-bit output), LSE[0] = scale * q0 . k0."""
    _banner(f"causal row 0 dtype={dtype}")
    qb, kb, vb = fa_inputs.draw_qkv(2, 2, 200, 128, dtype, 31)
    scale = parity.default_scale(128)
    o, lse = _run(qb, kb, vb, dtype, True, scale)
    v32 = fa_inputs.to_f32(vb, dtype)
    q32, k32 = fa_inputs.to_f32(qb, dtype), fa_inputs.to_f32(kb, dtype)
    for b in range(2):
        for h in range(2):
            if dtype == "fp32":
                assert np.allclose(o[b, h, 0], v32[b, h, 0], rtol=4e-7, atol=0)
            else:
                assert np.array_equal(o[b, h, 0], v32[b, h, 0])
            expect = scale * math.fsum(float(x) * float(y) for x, y in zip(q32[b, h, 0], k32[b, h, 0]))
            assert abs(lse[b, h, 0] - expect) <= 1e-4 * max(1.0, abs(expect))


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_give_means(causal):
    """Q = 0: every visible score is 0, so O is the mean (causal: prefix mean)
    of the value rows and LSE = log(number of visible keys)."""
    _banner(f"Q=0 causal={causal}")
    B, H, N, D, dtype = 1, 2, 333, 64, "bf16"
    _, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 41)
    qb = np.zeros_like(kb)
    o, lse = _run(qb, kb, vb, dtype, causal, 0.125)
    v = fa_inputs.to_f32(vb, dtype).astype(np.float64)
    if causal:
        ref = np.cumsum(v, axis=2) / np.arange(1, N + 1)[None, None, :, None]
        lref = np.log(np.arange(1, N + 1))[None, None, :]
    else:
        ref = np.broadcast_to(v.mean(axis=2, keepdims=True), v.shape)
        lref = np.full((1, 1, N), math.log(N))
    assert np.abs(o - ref).max() <= parity.TOL_O_16
    assert np.abs(lse - lref).max() <= parity.TOL_LSE


def test_key_permutation_invariance():
    _banner("key permutation")
    B, H, N, D, dtype = 1, 2, 300, 128, "fp16"
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 51)
    perm = np.random.default_rng(52).permutation(N)
    o1, l1 = _run(qb, kb, vb, dtype, False, 0.09)
    o2, l2 = _run(qb, kb[:, :, perm].copy(), vb[:, :, perm].copy(), dtype, False, 0.09)
    assert np.abs(o1 - o2).max() <= parity.TOL_O_16
    assert np.abs(l1 - l2).max() <= parity.TOL_LSE


@pytest.mark.parametrize("q_mult", [8.0, 32.0])
def test_amplified_scores_stay_finite(q_mult):
    """Large score spreads stress the running-max rescale ("Building a
    Verifiable FlashAttention Forward", Part 4)."""
    _banner(f"amplified Q x{q_mult}")
    B, H, N, D, dtype = 1, 4, 513, 128, "bf16"
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, 61, q_mult=q_mult, v_dist="uniform")
    for causal in (False, True):
        o, lse = _run(qb, kb, vb, dtype, causal, parity.default_scale(D))
        o_ref, lse_ref = parity.reference_full(qb, kb, vb, dtype, parity.default_scale(D), causal)
        parity.check(o, lse, o_ref, lse_ref, dtype, f"amplified x{q_mult} causal={causal}")


def test_bitwise_deterministic():
    _banner("determinism")
    qb, kb, vb = fa_inputs.draw_qkv(2, 8, 1000, 128, "bf16", 71)
    runs = [_run(qb, kb, vb, "bf16", c, 0.0884) for c in (False, True, False, True)]
    assert np.array_equal(runs[0][0], runs[2][0]) and np.array_equal(runs[0][1], runs[2][1])
    assert np.array_equal(runs[1][0], runs[3][0]) and np.array_equal(runs[1][1], runs[3][1])


# ---------------------------------------------------------------------------
# The workloads at full size, in the benchmark's launch configuration


WORKLOAD_CASES = [(name, c) for name, w in fa_inputs.WORKLOADS.items() for c in w.masks]


@pytest.mark.parametrize("name,causal", WORKLOAD_CASES,
                         ids=[f"{n}-{'causal' if c else 'full'}" for n, c in WORKLOAD_CASES])
def test_workload_full_size(name, causal):
    """Every output element and every LSE of the workload at its full size,
    run as the benchmark runs it (fa_fwd, the default kernel), against the
    fp64 oracle evaluated row by row in chunks."""
    w = fa_inputs.WORKLOADS[name]
    _banner(f"workload {name} causal={causal}")
    qb, kb, vb = fa_inputs.workload_inputs(w)
    o, lse = _run(qb, kb, vb, w.dtype, causal, w.scale)
    oe, le, worst = parity.check_every_row(o, lse, qb, kb, vb, w.dtype, w.scale, causal, name)
    bound = parity.TOL_O_32_NORMWISE if w.dtype == "fp32" else parity.TOL_O_16
    print(f"[parity] {name} causal={causal} every element: O err {oe:.3e} (bound {bound:.0e}, "
          f"margin {bound - oe:.3e}; worst at head/row/d {worst[:3]} where |O_ref| = "
          f"{worst[3]:.3f}), LSE err {le:.3e} (bound {parity.TOL_LSE:.0e})", flush=True)


# ---------------------------------------------------------------------------
# Streams and HIP graphs: the entry points are stream-ordered and make no
# allocating or synchronising call, so they run on any stream and can be
# captured into a graph


def _graph_inputs(seed):
    import torch
    qb, kb, vb = fa_inputs.draw_qkv(2, 4, 520, 128, "bf16", seed)
    dob = fa_inputs.draw_qkv(2, 4, 520, 128, "bf16", seed + 1)[0]
    return tuple(parity.to_device(x, "bf16") for x in (qb, kb, vb, dob))


def test_side_stream_matches_default_stream():
    """Inputs written and attention run on a side stream give bitwise the
    result of the default stream."""
    import torch
    _banner("side stream")
    q, k, v, _ = _graph_inputs(501)
    o_ref, l_ref = fa.fa_fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        q2, k2, v2 = q * 1, k * 1, v * 1          # produced on the side stream
        o, lse = fa.fa_fwd(q2, k2, v2, causal=True, stream=side)
    side.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_graph_capture_replays_match_eager():
    """fa_fwd (both masks), fa_fwd_splitkv (two kernels, preallocated
    workspace) and fa_bwd (two kernels) captured into one HIP graph; the
    inputs are rewritten between replays by eager kernels, and every replay
    must equal, bitwise, the eager calls on the same inputs."""
    import torch
    _banner("graph capture")
    q, k, v, do = _graph_inputs(601)
    o_nc, l_nc = torch.empty_like(q), torch.empty(q.shape[:3], device=q.device)
    o_c, l_c = torch.empty_like(q), torch.empty(q.shape[:3], device=q.device)
    o_s, l_s = torch.empty_like(q), torch.empty(q.shape[:3], device=q.device)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty(q.shape[:3], device=q.device)
    B, H, N, D = q.shape
    need = fa.fa_fwd_splitkv_workspace_size(B, H, N, N, D, 4)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)

    def work(stream):
        fa.fa_fwd(q, k, v, o_nc, l_nc, causal=False, stream=stream)
        fa.fa_fwd(q, k, v, o_c, l_c, causal=True, stream=stream)
        fa.fa_fwd_splitkv(q, k, v, o_s, l_s, causal=True, num_splits=4, workspace=ws,
                          stream=stream)
        fa.fa_bwd(q, k, v, o_c, do, l_c, causal=True, dq=dq, dk=dk, dv=dv, delta=delta,
                  stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work(side)                                 # first calls outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        work(torch.cuda.current_stream())
    torch.cuda.synchronize()
    outs = (o_nc, l_nc, o_c, l_c, o_s, l_s, dq, dk, dv, delta)
    for rep in range(4):
        nq, nk, nv, ndo = _graph_inputs(700 + rep)
        q.copy_(nq), k.copy_(nk), v.copy_(nv), do.copy_(ndo)
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in outs]
        work(torch.cuda.current_stream())           # eager, same inputs
        torch.cuda.synchronize()
        for name, g, e in zip(("o", "lse", "o_causal", "lse_causal", "o_split", "lse_split",
                               "dq", "dk", "dv", "delta"), got, outs):
            assert torch.equal(g, e), f"replay {rep}: {name} differs from the eager call"
    # and the replayed forward is right, not only repeatable
    bits = fa_inputs.draw_qkv(2, 4, 520, 128, "bf16", 703)
    o_ref, lse_ref = oracle.attention(*(fa_inputs.to_f32(x, "bf16") for x in bits), D ** -0.5, True)
    parity.check(parity.from_device(o_c), l_c.cpu().numpy(), o_ref, lse_ref, "bf16", "graph")
