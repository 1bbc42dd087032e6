"""CPU tests of the C ABI: the library loads without a GPU, exports every
function that include/*.h declares, and validates its arguments before any
HIP call (so every error path can be exercised here)."""
import ctypes
import glob
import os
import re

import pytest

import exact_attention_10_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# fake, never dereferenced device addresses (validation runs before any HIP call)
Q, K, V, O, L = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(fa.LIBRARY):
        pytest.fail("HIP library not built: run `python -m exact_attention_10_amd.build`")
    return fa.load_library()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, flags=re.M):
            names.add(m.group(1))
    return sorted(names)


def test_header_declares_expected_entry_points():
    names = declared_functions()
    for n in ("fa_fwd", "fa_fwd_ex", "fa_bwd", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc",
              "fa_fwd_splitkv_workspace_size",
              "fa_splitkv_auto_splits", "fa_fwd_nk", "fa_fwd_variant", "fa_strerror", "fa_version",
              "fa_num_variants", "fa_variant_name"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
        assert n in fa.SIGNATURES, f"{n} has no binding signature"


def test_version_and_strings(lib):
    assert lib.fa_version() >= 100
    for code in (fa.FA_OK, fa.FA_ERR_INVALID_ARG, fa.FA_ERR_UNSUPPORTED, fa.FA_ERR_ALIGNMENT,
                 fa.FA_ERR_HIP, 12345):
        assert isinstance(fa.fa_strerror(code), str) and fa.fa_strerror(code)
    n = fa.fa_num_variants()
    assert n >= 1
    assert all(fa.fa_variant_name(i) for i in range(n))
    assert fa.fa_variant_name(n) == "" and fa.fa_variant_name(-1) == ""


def call(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=4, N=256, D=128, causal=0, scale=0.088,
         dtype=fa.FA_DTYPE_BF16, n_kv=None, variant=None):
    if variant is not None:
        return lib.fa_fwd_variant(q, k, v, o, lse, B, H, N, N if n_kv is None else n_kv, D,
                                  causal, scale, dtype, None, variant)
    if n_kv is not None:
        return lib.fa_fwd_nk(q, k, v, o, lse, B, H, N, n_kv, D, causal, scale, dtype, None)
    return lib.fa_fwd(q, k, v, o, lse, B, H, N, D, causal, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_ERR_INVALID_ARG),
    (dict(H=-1), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-0.1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(D=32), fa.FA_ERR_UNSUPPORTED),
    (dict(dtype=7), fa.FA_ERR_UNSUPPORTED),
    (dict(q=Q + 8), fa.FA_ERR_ALIGNMENT),
    (dict(lse=L + 4), fa.FA_ERR_ALIGNMENT),
    (dict(o=Q), fa.FA_ERR_INVALID_ARG),                 # output aliases an input
    (dict(o=K + 4096), fa.FA_ERR_INVALID_ARG),          # partial overlap
    (dict(lse=O + 64), fa.FA_ERR_INVALID_ARG),          # lse inside o
    (dict(N=1 << 24, D=128, dtype=fa.FA_DTYPE_FP32), fa.FA_ERR_UNSUPPORTED),  # head > 2 GiB
    (dict(n_kv=-1), fa.FA_ERR_INVALID_ARG),
    (dict(n_kv=257), fa.FA_ERR_INVALID_ARG),
    (dict(variant=99), fa.FA_ERR_UNSUPPORTED),
    (dict(variant=-1), fa.FA_ERR_UNSUPPORTED),
])
def test_validation_rejects_before_any_hip_call(lib, kw, code):
    assert call(lib, **kw) == code


def call_ex(lib, q=Q, k=K, v=V, o=O, lse=L, B=2, H=4, Nq=256, Nk=512, D=128, causal=1,
            align=fa.FA_CAUSAL_BOTTOM_RIGHT, scale=0.088, dtype=fa.FA_DTYPE_BF16):
    return lib.fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, D, causal, align, scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(Nq=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-3), fa.FA_ERR_INVALID_ARG),
    (dict(align=2), fa.FA_ERR_INVALID_ARG),
    (dict(align=-1, causal=0), fa.FA_ERR_INVALID_ARG),     # checked even without a mask
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=1 << 24, dtype=fa.FA_DTYPE_FP32), fa.FA_ERR_UNSUPPORTED),   # K head > 2 GiB
    (dict(Nq=1 << 24, dtype=fa.FA_DTYPE_FP32), fa.FA_ERR_UNSUPPORTED),   # Q head > 2 GiB
    (dict(v=V + 8), fa.FA_ERR_ALIGNMENT),
    # o is [2,4,256,128] bf16 = 512 KiB; k and v are [2,4,512,128] = 1 MiB each
    (dict(o=K + (1 << 20) - 4096), fa.FA_ERR_INVALID_ARG),  # o overlaps the end of k
    (dict(k=O + (1 << 19) - 256), fa.FA_ERR_INVALID_ARG),   # k starts inside o
    (dict(lse=V + (1 << 20) - 64), fa.FA_ERR_INVALID_ARG),  # lse inside v's key-length extent
])
def test_cross_attention_validation(lib, kw, code):
    assert call_ex(lib, **kw) == code


WS = 0x60000000   # fake workspace address (256-byte aligned)


def call_split(lib, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Nq=200, Nk=1000, D=64, causal=0,
               align=fa.FA_CAUSAL_TOP_LEFT, scale=0.125, dtype=fa.FA_DTYPE_BF16, ns=4,
               ws=WS, ws_bytes=None):
    if ws_bytes is None:
        ws_bytes = lib.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, ns)
    return lib.fa_fwd_splitkv(q, k, v, o, lse, B, H, Nq, Nk, D, causal, align, scale, dtype, ns,
                              ws, ws_bytes, None)


def test_splitkv_workspace_size(lib):
    # o_part: ns * rows * D fp32, rounded up to 256 bytes; then lse_part: ns * rows fp32
    rows, D, ns = 1 * 2 * 200, 64, 4
    o_bytes = ns * rows * D * 4
    want = (o_bytes + 255) // 256 * 256 + ns * rows * 4
    assert lib.fa_fwd_splitkv_workspace_size(1, 2, 200, 1000, D, ns) == want
    assert lib.fa_fwd_splitkv_workspace_size(1, 2, 200, 1000, D, 1) == 0      # single pass
    assert lib.fa_fwd_splitkv_workspace_size(1, 2, 200, 1000, D, 33) == 0     # invalid
    assert lib.fa_fwd_splitkv_workspace_size(0, 2, 200, 1000, D, 4) == 0      # invalid


def test_splitkv_auto_choice(lib):
    # [1, 8, 2048] queries at D = 128: 128 workgroups, 32 key tiles -> 2 splits
    assert lib.fa_splitkv_auto_splits(1, 8, 2048, 2048, 128) == 2
    # [8, 1, 1024] at D = 64: 16 key tiles are too few to split
    assert lib.fa_splitkv_auto_splits(8, 1, 1024, 1024, 64) == 1
    # a large grid needs no split
    assert lib.fa_splitkv_auto_splits(4, 16, 4096, 4096, 128) == 1
    # one query tile, many keys: one workgroup per CU would be 256, capped at 32
    assert lib.fa_splitkv_auto_splits(1, 1, 1, 1 << 20, 128) == 32
    # one query tile, 64 key tiles at D = 128: 8 splits of 8 tiles
    assert lib.fa_splitkv_auto_splits(1, 1, 100, 4096, 128) == 8


@pytest.mark.parametrize("kw,code", [
    (dict(ns=-1), fa.FA_ERR_INVALID_ARG),
    (dict(ns=33), fa.FA_ERR_INVALID_ARG),
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),
    (dict(ws_bytes=1024), fa.FA_ERR_INVALID_ARG),                # too small
    (dict(ws=WS + 16), fa.FA_ERR_ALIGNMENT),                      # not 256-byte aligned
    (dict(ws=Q), fa.FA_ERR_INVALID_ARG),                          # overlaps q
    (dict(ws=O - 256), fa.FA_ERR_INVALID_ARG),                    # runs into o
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),                          # checked like fa_fwd_ex
    (dict(align=5), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
])
def test_splitkv_validation(lib, kw, code):
    assert call_split(lib, **kw) == code


def call_split_noalloc(lib, q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, Nq=200, Nk=1000, D=64, causal=0,
                       align=fa.FA_CAUSAL_TOP_LEFT, scale=0.125, dtype=fa.FA_DTYPE_BF16, ns=4):
    return lib.fa_fwd_splitkv_noalloc(q, k, v, o, lse, B, H, Nq, Nk, D, causal, align, scale,
                                      dtype, ns, None)


@pytest.mark.parametrize("kw,code", [
    (dict(ns=-1), fa.FA_ERR_INVALID_ARG),
    (dict(ns=33), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(D=96), fa.FA_ERR_UNSUPPORTED),
    (dict(align=5), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(o=Q), fa.FA_ERR_INVALID_ARG),
    (dict(k=K + 8), fa.FA_ERR_ALIGNMENT),
    # partials of 32 splits x 4096 query rows x 128 fp32 (64 MiB) exceed the
    # 32 MiB scratch: refused before any HIP call
    (dict(B=1, H=1, Nq=4096, Nk=1 << 16, D=128, ns=32), fa.FA_ERR_SCRATCH),
])
def test_splitkv_noalloc_validation(lib, kw, code):
    assert call_split_noalloc(lib, **kw) == code
    assert fa.fa_strerror(code)


def test_splitkv_noalloc_scratch_covers_every_automatic_choice(lib):
    """Every split count the library picks by itself (num_splits = 0) fits the
    static scratch: grids of up to 128 query tiles are the only ones split."""
    assert fa.FA_SPLITKV_SCRATCH_BYTES == 32 << 20
    worst = 0
    for D in (64, 128):
        for BH in (1, 2, 3, 5, 8, 16, 31, 64, 100, 127, 128):
            for nq in (1, 100, 128, 129, 1000, 4096, 16384):
                for nk in (64, 1000, 4096, 1 << 16, 1 << 20):
                    need = lib.fa_fwd_splitkv_workspace_size(1, BH, nq, nk, D, 0)
                    worst = max(worst, need)
                    assert need <= fa.FA_SPLITKV_SCRATCH_BYTES, (D, BH, nq, nk, need)
    assert worst > (8 << 20)     # the sweep does reach sizable partials


# fake addresses for the backward's extra tensors: [2,4,256,128] bf16 = 512 KiB each
OO, DO, DQ, DK, DV, DL = 0x90000000, 0xA0000000, 0xB0000000, 0xC0000000, 0xD0000000, 0xE0000000


def call_bwd(lib, q=Q, k=K, v=V, o=OO, do=DO, lse=L, dq=DQ, dk=DK, dv=DV, delta=DL, B=2, H=4,
             Nq=256, Nk=256, D=128, causal=1, align=fa.FA_CAUSAL_TOP_LEFT, scale=0.088,
             dtype=fa.FA_DTYPE_BF16):
    return lib.fa_bwd(q, k, v, o, do, lse, dq, dk, dv, delta, B, H, Nq, Nk, D, causal, align,
                      scale, dtype, None)


@pytest.mark.parametrize("kw,code", [
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(delta=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=None), fa.FA_ERR_INVALID_ARG),
    (dict(do=None), fa.FA_ERR_INVALID_ARG),
    (dict(dk=None), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_DTYPE_FP32), fa.FA_ERR_UNSUPPORTED),     # no fp32 backward
    (dict(D=80), fa.FA_ERR_UNSUPPORTED),
    (dict(align=3), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(dq=Q), fa.FA_ERR_INVALID_ARG),                         # output aliases an input
    (dict(dk=DV), fa.FA_ERR_INVALID_ARG),                        # two outputs alias
    (dict(dv=DO + 4096), fa.FA_ERR_INVALID_ARG),                 # output inside dout
    (dict(delta=L + 64), fa.FA_ERR_INVALID_ARG),                 # delta inside lse
    (dict(delta=DL + 4), fa.FA_ERR_ALIGNMENT),
    (dict(do=DO + 8), fa.FA_ERR_ALIGNMENT),
])
def test_bwd_validation(lib, kw, code):
    assert call_bwd(lib, **kw) == code


def test_lse_may_be_null_for_validation(lib):
    # with lse = NULL, an otherwise invalid call still fails in validation
    assert call(lib, lse=None, D=80) == fa.FA_ERR_UNSUPPORTED


def test_python_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError):
        fa.load_library(str(tmp_path / "missing.so"))


def test_binding_rejects_cpu_tensors(lib):
    torch = pytest.importorskip("torch")
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x)
