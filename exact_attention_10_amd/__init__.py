"""Python binding of the gfx950 FlashAttention-2 forward library.

Argument marshalling only: every step of the attention forward runs in the
HIP kernels of ``libfa_mi355x.so`` (built by ``exact_attention_10_amd.build``).
PyTorch supplies device memory and streams. There is no fallback: if the
library is missing, calls raise ``RuntimeError``.

The functions mirror the C ABI of ``include/fa.h``:

* :func:`fa_fwd` -- O = softmax(scale * Q K^T) V and the row log-sum-exp;
* :func:`fa_fwd_ex` -- the same with separate query and key lengths and a
  top-left or bottom-right causal mask;
* :func:`fa_fwd_splitkv` -- the same result for small grids, with the keys
  of every query tile split over several workgroups and combined;
* :func:`fa_fwd_splitkv_noalloc` -- the same split-KV computation with its
  partials in the library's static scratch array (no allocation);
* :func:`fa_bwd` -- the backward pass: dQ, dK, dV from the forward's inputs,
  output and log-sum-exp;
* :func:`fa_fwd_nk` -- the same with only the first ``n_kv`` keys visible;
* :func:`fa_fwd_variant` -- run a named kernel variant (tuning);
* :func:`fa_num_variants`, :func:`fa_variant_name`, :func:`fa_strerror`,
  :func:`fa_version`.
"""
from __future__ import annotations

import ctypes
import math
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; FA_MI355X_LIBRARY names another build of the same
# sources instead (the tests use it for a host-sanitizer check build)
LIBRARY = os.environ.get("FA_MI355X_LIBRARY") or os.path.join(_HERE, "libfa_mi355x.so")

FA_DTYPE_FP32, FA_DTYPE_FP16, FA_DTYPE_BF16 = 0, 1, 2
FA_CAUSAL_TOP_LEFT, FA_CAUSAL_BOTTOM_RIGHT = 0, 1
_ALIGN = {"top-left": FA_CAUSAL_TOP_LEFT, "bottom-right": FA_CAUSAL_BOTTOM_RIGHT}
FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_ALIGNMENT, FA_ERR_HIP = 0, -1, -2, -3, -4
FA_ERR_SCRATCH = -5
# bytes of the static device array behind fa_fwd_splitkv_noalloc (include/fa.h)
FA_SPLITKV_SCRATCH_BYTES = 32 << 20

# names and argument types of every exported symbol of include/fa.h
_P, _I64, _I, _F = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float
SIGNATURES = {
    "fa_fwd": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I, _F, _I, _P]),
    "fa_fwd_ex": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _F, _I, _P]),
    "fa_fwd_splitkv": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _F, _I, _I,
                            _P, ctypes.c_size_t, _P]),
    "fa_fwd_splitkv_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _F,
                                    _I, _I, _P]),
    "fa_bwd": (_I, [_P] * 10 + [_I64] * 5 + [_I, _I, _F, _I, _P]),
    "fa_fwd_splitkv_workspace_size": (ctypes.c_size_t, [_I64, _I64, _I64, _I64, _I64, _I]),
    "fa_splitkv_auto_splits": (_I, [_I64, _I64, _I64, _I64, _I64]),
    "fa_fwd_nk": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _F, _I, _P]),
    "fa_fwd_variant": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _F, _I, _P, _I]),
    "fa_num_variants": (_I, []),
    "fa_variant_name": (ctypes.c_char_p, [_I]),
    "fa_strerror": (ctypes.c_char_p, [_I]),
    "fa_version": (_I, []),
}

_lib = None


class FAError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def load_library(path: str = LIBRARY):
    """Load the HIP library; raises RuntimeError if it has not been built."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m exact_attention_10_amd.build`")
    # PyTorch ships its own HIP and HSA runtimes. Import it first so that the
    # library binds to the runtime already in the process (same soname)
    # instead of loading the system copies next to torch's: two HSA runtimes
    # in one process do not share the device, and launches then fail.
    import torch  # noqa: F401
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    if path == LIBRARY:
        _lib = lib
    return lib


def _dtype_code(t):
    import torch
    codes = {torch.float32: FA_DTYPE_FP32, torch.float16: FA_DTYPE_FP16,
             torch.bfloat16: FA_DTYPE_BF16}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _check(code: int):
    if code != FA_OK:
        raise FAError(code, fa_strerror(code))


def _prepare(q, k, v, o, lse, with_lse, same_length=True):
    import torch
    if q.dim() != 4 or k.dim() != 4 or v.dim() != 4:
        raise ValueError("q, k, v must be [B, H, N, D]")
    kv_shape = q.shape if same_length else (q.shape[0], q.shape[1], k.shape[2], q.shape[3])
    for name, t, shape in (("q", q, q.shape), ("k", k, kv_shape), ("v", v, kv_shape)):
        if t.shape != shape or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in shape, dtype and device"
                             + ("" if same_length else " (k and v may differ in N)"))
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if o is None:
        o = torch.empty_like(q)
    elif o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() or o.device != q.device:
        raise ValueError("o must be a contiguous tensor like q")
    if lse is None and with_lse:
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    elif lse is not None and (lse.shape != q.shape[:3] or lse.dtype != torch.float32
                              or not lse.is_contiguous() or lse.device != q.device):
        raise ValueError("lse must be a contiguous fp32 [B, H, N] tensor")
    return o, lse


def _stream_handle(q, stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def fa_fwd_variant(q, k, v, o=None, lse=None, *, n_kv=None, causal=False, scale=None,
                   stream=None, variant=0, with_lse=True):
    """Run kernel variant ``variant``; returns (o, lse). See include/fa.h."""
    lib = load_library()
    o, lse = _prepare(q, k, v, o, lse, with_lse)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    n_kv = N if n_kv is None else int(n_kv)
    rc = lib.fa_fwd_variant(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr() if lse is not None else None,
                            B, H, N, n_kv, D, int(bool(causal)), float(scale),
                            _dtype_code(q), _stream_handle(q, stream), int(variant))
    _check(rc)
    return o, lse


def fa_fwd_nk(q, k, v, o=None, lse=None, *, n_kv, causal=False, scale=None, stream=None,
              with_lse=True):
    """Attention with only the first ``n_kv`` keys visible; returns (o, lse)."""
    lib = load_library()
    o, lse = _prepare(q, k, v, o, lse, with_lse)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = lib.fa_fwd_nk(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr() if lse is not None else None,
                       B, H, N, int(n_kv), D, int(bool(causal)), float(scale),
                       _dtype_code(q), _stream_handle(q, stream))
    _check(rc)
    return o, lse


def fa_fwd(q, k, v, o=None, lse=None, *, causal=False, scale=None, stream=None,
           with_lse=True):
    """O = softmax(scale * Q K^T) V over [B, H, N, D] tensors; returns (o, lse).

    ``scale`` defaults to 1/sqrt(D). ``lse`` is fp32 [B, H, N] (natural log) or
    None when ``with_lse`` is False. Asynchronous on ``stream`` (default: the
    current torch stream).
    """
    lib = load_library()
    o, lse = _prepare(q, k, v, o, lse, with_lse)
    B, H, N, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = lib.fa_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                    lse.data_ptr() if lse is not None else None,
                    B, H, N, D, int(bool(causal)), float(scale), _dtype_code(q),
                    _stream_handle(q, stream))
    _check(rc)
    return o, lse


def fa_fwd_ex(q, k, v, o=None, lse=None, *, causal=False, causal_align="top-left",
              scale=None, stream=None, with_lse=True):
    """Attention with separate query and key lengths: q [B, H, Nq, D], k and v
    [B, H, Nk, D]; returns (o [B, H, Nq, D], lse [B, H, Nq]). ``causal_align``
    is "top-left" (query i sees keys j <= i) or "bottom-right"
    (j <= i + Nk - Nq)."""
    lib = load_library()
    if causal_align not in _ALIGN:
        raise ValueError(f"causal_align must be one of {sorted(_ALIGN)}")
    o, lse = _prepare(q, k, v, o, lse, with_lse, same_length=False)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = lib.fa_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                       lse.data_ptr() if lse is not None else None,
                       B, H, Nq, Nk, D, int(bool(causal)), _ALIGN[causal_align], float(scale),
                       _dtype_code(q), _stream_handle(q, stream))
    _check(rc)
    return o, lse


def fa_fwd_splitkv(q, k, v, o=None, lse=None, *, causal=False, causal_align="top-left",
                   scale=None, num_splits=0, workspace=None, stream=None, with_lse=True):
    """Split-KV attention (same result as :func:`fa_fwd_ex`); returns (o, lse).

    ``num_splits`` = 0 lets the library choose. ``workspace`` is a device tensor
    of at least :func:`fa_fwd_splitkv_workspace_size` bytes; when None, one is
    allocated here with torch (the library itself allocates nothing).
    """
    import torch
    lib = load_library()
    if causal_align not in _ALIGN:
        raise ValueError(f"causal_align must be one of {sorted(_ALIGN)}")
    o, lse = _prepare(q, k, v, o, lse, with_lse, same_length=False)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    need = lib.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, int(num_splits))
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    elif workspace is not None and (workspace.device != q.device or not workspace.is_contiguous()):
        raise ValueError("workspace must be a contiguous tensor on q's device")
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    rc = lib.fa_fwd_splitkv(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                            lse.data_ptr() if lse is not None else None,
                            B, H, Nq, Nk, D, int(bool(causal)), _ALIGN[causal_align],
                            float(scale), _dtype_code(q), int(num_splits), ws_ptr, ws_bytes,
                            _stream_handle(q, stream))
    _check(rc)
    return o, lse


def fa_fwd_splitkv_noalloc(q, k, v, o=None, lse=None, *, causal=False, causal_align="top-left",
                           scale=None, num_splits=0, stream=None, with_lse=True):
    """Split-KV attention whose partials live in the library's static scratch
    array (nothing is allocated by the library; see include/fa.h for the limit
    and for why calls on one GPU must not overlap); returns (o, lse). Pass
    ``o`` and ``lse`` to keep this wrapper from allocating them either."""
    lib = load_library()
    if causal_align not in _ALIGN:
        raise ValueError(f"causal_align must be one of {sorted(_ALIGN)}")
    o, lse = _prepare(q, k, v, o, lse, with_lse, same_length=False)
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rc = lib.fa_fwd_splitkv_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr() if lse is not None else None,
                                    B, H, Nq, Nk, D, int(bool(causal)), _ALIGN[causal_align],
                                    float(scale), _dtype_code(q), int(num_splits),
                                    _stream_handle(q, stream))
    _check(rc)
    return o, lse


def fa_bwd(q, k, v, o, dout, lse, *, causal=False, causal_align="top-left", scale=None,
           dq=None, dk=None, dv=None, delta=None, stream=None):
    """Gradients (dq, dk, dv) of the forward for upstream gradient ``dout``.

    ``o`` and ``lse`` are the forward's outputs for the same q, k, v, causal,
    causal_align and scale. Returns (dq, dk, dv, delta) where delta is
    rowsum(dout * o) in fp32. 16-bit dtypes only.
    """
    import torch
    lib = load_library()
    if causal_align not in _ALIGN:
        raise ValueError(f"causal_align must be one of {sorted(_ALIGN)}")
    _prepare(q, k, v, o, lse, True, same_length=False)
    if dout.shape != q.shape or dout.dtype != q.dtype or not dout.is_contiguous() \
            or dout.device != q.device:
        raise ValueError("dout must be a contiguous tensor like q")
    B, H, Nq, D = q.shape
    Nk = k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, ref in (("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        if t.shape != ref.shape or t.dtype != ref.dtype or not t.is_contiguous() \
                or t.device != ref.device:
            raise ValueError(f"{name} must be a contiguous tensor like {name[1:]}")
    if delta is None:
        delta = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif delta.shape != (B, H, Nq) or delta.dtype != torch.float32 or not delta.is_contiguous() \
            or delta.device != q.device:
        raise ValueError("delta must be a contiguous fp32 [B, H, Nq] tensor on q's device")
    rc = lib.fa_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), dout.data_ptr(),
                    lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                    B, H, Nq, Nk, D, int(bool(causal)), _ALIGN[causal_align], float(scale),
                    _dtype_code(q), _stream_handle(q, stream))
    _check(rc)
    return dq, dk, dv, delta


def fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, num_splits=0) -> int:
    return int(load_library().fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, int(num_splits)))


def fa_splitkv_auto_splits(B, H, Nq, Nk, D) -> int:
    return int(load_library().fa_splitkv_auto_splits(B, H, Nq, Nk, D))


def fa_num_variants() -> int:
    return load_library().fa_num_variants()


def fa_variant_name(variant: int) -> str:
    return load_library().fa_variant_name(int(variant)).decode()


def fa_strerror(code: int) -> str:
    return load_library().fa_strerror(int(code)).decode()


def fa_version() -> int:
    return load_library().fa_version()
