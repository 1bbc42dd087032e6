"""GPU test of fa_fwd_splitkv_noalloc, the split-KV entry point that
allocates nothing (its partials live in the library's static scratch array).

Two calls in a row through the C ABI, the second on smaller inputs, each
compared bitwise with fa_fwd_splitkv (same kernels, same split count, a
caller workspace poisoned with NaN) and with the fp64 oracle within the
forward tolerances; then the library's own split choice, and a request too
large for the scratch, refused before anything is launched."""
import numpy as np
import pytest

import exact_attention_10_amd as fa
import fa_inputs
from tests import parity

pytestmark = pytest.mark.gpu

CASES = [
    # (B, H, Nq, Nk, D, dtype, causal, align, num_splits)
    (2, 4, 520, 2100, 128, "bf16", True, "bottom-right", 5),
    (1, 2, 130, 700, 64, "fp16", False, "top-left", 3),
]


def _one(B, H, Nq, Nk, D, dtype, causal, align, ns, seed):
    import torch
    print(f"\n[case] noalloc B={B} H={H} Nq={Nq} Nk={Nk} D={D} {dtype} causal={causal} "
          f"{align} splits={ns}", flush=True)
    qb, kb, vb = fa_inputs.draw_qkv_cross(B, H, Nq, Nk, D, dtype, seed)
    q, k, v = (parity.to_device(x, dtype) for x in (qb, kb, vb))
    scale = parity.default_scale(D)
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa.fa_fwd_splitkv_noalloc(q, k, v, o, lse, causal=causal, causal_align=align, scale=scale,
                              num_splits=ns)
    torch.cuda.synchronize()
    need = fa.fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, D, ns)
    ws = torch.full((max(need, 4) // 4,), float("nan"), dtype=torch.float32, device=q.device)
    o2, l2 = fa.fa_fwd_splitkv(q, k, v, causal=causal, causal_align=align, scale=scale,
                               num_splits=ns, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, l2), "differs from fa_fwd_splitkv"
    o_ref, lse_ref = parity.reference_full_ex(qb, kb, vb, dtype, scale, causal, align)
    oe, le = parity.check(parity.from_device(o), lse.cpu().numpy(), o_ref, lse_ref, dtype,
                          f"noalloc {dtype} D={D}")
    print(f"[parity] noalloc splits={ns}: O err {oe:.3e} LSE err {le:.3e}", flush=True)


def test_noalloc_two_calls_second_smaller():
    for i, case in enumerate(CASES):
        _one(*case, seed=900 + i)


def test_noalloc_automatic_split_choice():
    B, H, Nq, Nk, D = 1, 8, 2048, 2048, 128
    assert fa.fa_splitkv_auto_splits(B, H, Nq, Nk, D) > 1
    _one(B, H, Nq, Nk, D, "bf16", False, "top-left", 0, seed=910)


def test_noalloc_refuses_partials_beyond_the_scratch():
    import torch
    q = torch.zeros((1, 1, 4096, 128), dtype=torch.bfloat16, device="cuda")
    kv = torch.zeros((1, 1, 1 << 16, 128), dtype=torch.bfloat16, device="cuda")
    assert fa.fa_fwd_splitkv_workspace_size(1, 1, 4096, 1 << 16, 128, 32) > \
        fa.FA_SPLITKV_SCRATCH_BYTES
    with pytest.raises(fa.FAError) as e:
        fa.fa_fwd_splitkv_noalloc(q, kv, kv, num_splits=32)
    assert e.value.code == fa.FA_ERR_SCRATCH
