"""CPU tests of the fp64 oracle: its pins, the tile recurrence, and mutants.

No GPU is involved; these run in the default (not gpu) suite.
"""
import math
import os
import shutil
import subprocess
import tempfile

import numpy as np
import pytest

import fa_inputs
import oracle
from oracle.tiled import tiled_attention
from tests import oracle_bwd_pins, oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


@pytest.mark.parametrize("bm,bn", [(16, 16), (64, 32), (7, 5), (128, 64), (32, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_tiled_recurrence_equals_explicit(bm, bn, causal):
    """The online-softmax recurrence reaches the explicit result (up to
    rounding) for square and non-square tiles, non-divisors of N and a ragged
    key length ("A09 - Advanced Triton & FlashAttention", section 3: the
    rescaled update is an exact identity)."""
    BH, N, D = 2, 150, 16
    rng = np.random.default_rng(bm * 1000 + bn)
    q = rng.standard_normal((BH, N, D)).astype(np.float32) * 3
    k = rng.standard_normal((BH, N, D)).astype(np.float32)
    v = rng.standard_normal((BH, N, D)).astype(np.float32)
    for n_kv in (N, 97):
        o_t, l_t = tiled_attention(q, k, v, 0.25, causal, bm, bn, n_kv=n_kv)
        o_e, l_e = oracle.attention(q, k, v, 0.25, causal, n_kv=n_kv)
        fin = np.isfinite(l_e)
        assert np.array_equal(fin, np.isfinite(l_t))
        assert np.abs(o_t - o_e).max() <= 1e-12
        assert np.abs(l_t[fin] - l_e[fin]).max() <= 1e-12


def test_tiled_recurrence_no_visible_key():
    q = np.ones((1, 8, 4), np.float32)
    o, lse = tiled_attention(q, q, q, 0.5, True, 4, 4, n_kv=0)
    assert (o == 0).all() and np.isneginf(lse).all()


def test_rows_api_rejects_bad_rows():
    q = np.zeros((1, 4, 4), np.float32)
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, q, 1.0, False, [(0, 4)])
    with pytest.raises(ValueError):
        oracle.attention_rows(q, q, q, 1.0, False, [(1, 0)])


def test_thread_count_does_not_change_results():
    BH, N, D = 3, 70, 16
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((BH, N, D)).astype(np.float32) for _ in range(3))
    env = dict(os.environ)
    code = ("import numpy as np, oracle, sys;"
            "a=np.load(sys.argv[1]);"
            "o,l=oracle.attention(a['q'],a['k'],a['v'],0.3,True);"
            "np.save(sys.argv[2], np.concatenate([o.ravel(), l.ravel()]))")
    with tempfile.TemporaryDirectory() as td:
        np.savez(os.path.join(td, "in.npz"), q=q, k=k, v=v)
        outs = []
        for threads in ("1", "5"):
            env["OMP_NUM_THREADS"] = threads
            out = os.path.join(td, f"o{threads}.npy")
            subprocess.run(["python", "-c", code, os.path.join(td, "in.npz"), out],
                           check=True, env=env, cwd=oracle_pins.__file__.rsplit("/tests/", 1)[0])
            outs.append(np.load(out))
        assert np.array_equal(outs[0], outs[1])


# ---------------------------------------------------------------------------
# Mutants: plant a plausible mistake in a copy of the oracle's C source and
# check that at least one pin fails on it.

MUTANTS = {
    "causal_excludes_diagonal": ("if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;",
                                 "if (causal && i + coff < n_vis) n_vis = i + coff;"),
    "causal_offset_dropped": ("if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;",
                              "if (causal && i + 1 < n_vis) n_vis = i + 1;"),
    "key_count_from_query_length": ("int64_t n_vis = n_kv;",
                                    "int64_t n_vis = n_kv < Nq ? n_kv : Nq;"),
    "dropped_scale": ("s[j] = scale * dot;", "s[j] = dot;"),
    "transposed_key_operand": ("dot += (double)qi[d] * (double)kj[d];",
                               "dot += (double)qi[d] * (double)kh[d * Nk + j];"),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "lse_dropped_max": ("lse[r] = m + log(l);", "lse[r] = log(l);"),
    "value_row_index": ("const float *vj = vh + j * D;", "const float *vj = vh + i * D;"),
    "no_max_subtraction": ("double m = s[0];", "double m = 0.0;"),
    "missing_normalisation": ("oi[d] = acc[d] / l;", "oi[d] = acc[d];"),
    "denominator_skips_first_key": ("l += s[j];", "if (j > 0) l += s[j];"),
    "max_ignores_first_key": ("double m = s[0];\n            for (int64_t j = 1;",
                              "double m = s[n_vis - 1];\n            for (int64_t j = n_vis;"),
    "empty_row_not_zero": ("for (int64_t d = 0; d < D; ++d) oi[d] = 0.0;\n                lse[r] = -INFINITY;",
                           "for (int64_t d = 0; d < D; ++d) oi[d] = vh[d];\n                lse[r] = 0.0;"),
}


@pytest.fixture(scope="module")
def mutant_dir():
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    d = tempfile.mkdtemp(prefix="oracle_mutants_")
    yield d
    shutil.rmtree(d, ignore_errors=True)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = open(oracle.SOURCE).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path_c = os.path.join(mutant_dir, f"{name}.c")
    path_so = os.path.join(mutant_dir, f"lib{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    oracle.build(path_c, path_so)
    failed = []
    for pin in oracle_pins.ALL_PINS:
        try:
            pin(lib_path=path_so)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"


# ---------------------------------------------------------------------------
# Input generator


def test_bf16_rounding_is_rne():
    import torch
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 10
    # add exact ties: float32 values whose low 16 bits are 0x8000
    ties = (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties])
    ours = fa_inputs.round_to_dtype(x, "bf16")
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = fa_inputs.to_f32(ours, "bf16")
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_fp16_roundtrip():
    x = np.random.default_rng(1).standard_normal(1000).astype(np.float32)
    bits = fa_inputs.round_to_dtype(x, "fp16")
    assert bits.dtype == np.uint16
    assert np.array_equal(fa_inputs.to_f32(bits, "fp16"), x.astype(np.float16).astype(np.float32))


def test_generator_is_seeded_and_follows_recipe():
    w = fa_inputs.WORKLOADS["b1h32_n16384_d128_bf16_q8"]
    q, k, v = fa_inputs.workload_inputs(w, N=64, H=2)
    q2, _, _ = fa_inputs.workload_inputs(w, N=64, H=2)
    assert np.array_equal(q, q2)
    vf = fa_inputs.to_f32(v, "bf16")
    assert vf.min() >= -1.0 and vf.max() <= 1.0
    qf = fa_inputs.to_f32(q, "bf16")
    assert 6.0 < qf.std() < 10.0
    assert math.isclose(w.scale, 1 / math.sqrt(128))


# ---------------------------------------------------------------------------
# Backward oracle: pins and mutants


@pytest.mark.parametrize("pin", oracle_bwd_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin()


BWD_MUTANTS = {
    "delta_term_dropped": ("dSi[j] = Pi[j] * (dp - Di);", "dSi[j] = Pi[j] * dp;"),
    "delta_sign_flipped": ("dSi[j] = Pi[j] * (dp - Di);", "dSi[j] = Pi[j] * (dp + Di);"),
    "dq_scale_dropped": ("dqh[i * D + d] = scale * acc;", "dqh[i * D + d] = acc;"),
    "dk_uses_keys": ("acc_k += dS[i * Nk + j] * (double)qh[i * D + d];",
                     "acc_k += dS[i * Nk + j] * (double)kh[j * D + d];"),
    "dv_uses_ds": ("acc_v += P[i * Nk + j] * (double)doh[i * D + d];",
                   "acc_v += dS[i * Nk + j] * (double)doh[i * D + d];"),
    "probabilities_unnormalised": ("for (int64_t j = 0; j < n_vis; ++j) Pi[j] = exp(Pi[j] - L);",
                                   "for (int64_t j = 0; j < n_vis; ++j) Pi[j] = exp(Pi[j] - m);"),
    "causal_offset_dropped": ("if (causal && i + coff + 1 < n_vis) n_vis = i + coff + 1;\n"
                              "            double *Pi = P + i * Nk",
                              "if (causal && i + 1 < n_vis) n_vis = i + 1;\n"
                              "            double *Pi = P + i * Nk"),
    "dp_transposed_value": ("for (int64_t d = 0; d < D; ++d) dp += (double)doi[d] * (double)vh[j * D + d];",
                            "for (int64_t d = 0; d < D; ++d) dp += (double)doi[d] * (double)vh[d * Nk + j];"),
    "sampled_dk_scale_dropped": ("for (int64_t d = 0; d < D; ++d) ok[d] *= scale;", ""),
    "sampled_future_rows_kept": ("if (causal && j > i + coff) continue;", "if (causal && j > i) continue;"),
    "sampled_dv_uses_ds": ("ov[d] += p * (double)doi[d];", "ov[d] += ds * (double)doi[d];"),
    "sampled_dq_delta_dropped": ("const double ds = exp(scale * dot - L[i]) * (dp - Dv[i]);",
                                 "const double ds = exp(scale * dot - L[i]) * dp;"),
}


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_mutant_is_caught(name, mutant_dir):
    src = open(oracle.BWD_SOURCE).read()
    old, new = BWD_MUTANTS[name]
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    path_c = os.path.join(mutant_dir, f"bwd_{name}.c")
    path_so = os.path.join(mutant_dir, f"libbwd_{name}.so")
    with open(path_c, "w") as f:
        f.write(src.replace(old, new))
    oracle.build(path_c, path_so)
    failed = []
    for pin in oracle_bwd_pins.ALL_PINS:
        try:
            pin(lib_path=path_so)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches backward mutant {name}"
