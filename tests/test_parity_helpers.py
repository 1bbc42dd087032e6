"""CPU tests of the GPU-parity checking helpers: the every-row comparison
must pass the oracle's own result rounded to the storage type, and must fail,
naming the right element, when a mistake is planted in it."""
import numpy as np
import pytest

import fa_inputs
import oracle
from tests import parity


def _case(dtype, causal, B=2, H=3, N=150, D=64, seed=11):
    qb, kb, vb = fa_inputs.draw_qkv(B, H, N, D, dtype, seed)
    q, k, v = (fa_inputs.to_f32(x, dtype) for x in (qb, kb, vb))
    o, lse = oracle.attention(q, k, v, D ** -0.5, causal)
    return (qb, kb, vb), o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_every_row_accepts_the_rounded_oracle(causal):
    bits, o, lse = _case("bf16", causal)
    o_b = fa_inputs.to_f32(fa_inputs.round_to_dtype(o.astype(np.float32), "bf16"), "bf16")
    oe, le, worst = parity.check_every_row(o_b, lse.astype(np.float32), *bits, "bf16",
                                           64 ** -0.5, causal, "rounded oracle", chunk=97)
    assert oe <= 2 ** -8 * np.abs(o).max() and le < 1e-6
    assert worst is not None


@pytest.mark.parametrize("where", [(0, 0, 0), (5, 149, 63), (3, 77, 10)])
def test_every_row_finds_a_planted_output_error(where):
    bits, o, lse = _case("bf16", True)
    bad = o.reshape(6, 150, 64).astype(np.float32).copy()
    bad[where] += 0.02
    with pytest.raises(AssertionError, match=r"O max abs error"):
        parity.check_every_row(bad, lse, *bits, "bf16", 64 ** -0.5, True, "planted", chunk=64)
    bad[where] -= 0.02 - 0.005                      # within the bound: passes, located
    oe, _, worst = parity.check_every_row(bad, lse, *bits, "bf16", 64 ** -0.5, True, "planted",
                                          chunk=64)
    assert abs(oe - 0.005) < 1e-6 and worst[:3] == where


def test_every_row_finds_a_planted_lse_error():
    bits, o, lse = _case("fp16", False)
    bad = lse.copy().reshape(-1)
    bad[517] += 2e-3
    with pytest.raises(AssertionError, match=r"LSE max abs error"):
        parity.check_every_row(o, bad, *bits, "fp16", 64 ** -0.5, False, "planted", chunk=100)
    bad[517] = -np.inf
    with pytest.raises(AssertionError, match=r"LSE finiteness"):
        parity.check_every_row(o, bad, *bits, "fp16", 64 ** -0.5, False, "planted", chunk=100)


def test_every_row_fp32_is_normwise():
    bits, o, lse = _case("fp32", False, B=1, H=1, N=128)
    scale = np.abs(o).max()
    bad = o.copy()
    bad[0, 0, 5, 3] += 0.5e-5 * scale
    oe, _, _ = parity.check_every_row(bad, lse, *bits, "fp32", 64 ** -0.5, False, "fp32")
    assert oe == pytest.approx(0.5e-5, rel=1e-3)
    bad[0, 0, 5, 3] += 1e-5 * scale
    with pytest.raises(AssertionError, match=r"normwise"):
        parity.check_every_row(bad, lse, *bits, "fp32", 64 ** -0.5, False, "fp32")
