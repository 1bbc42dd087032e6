"""Pins for the fp64 backward oracle: facts fixed by calculus and by the
forward oracle (itself pinned), not by the backward oracle's own code.

Each ``pin_*`` raises AssertionError when the backward oracle library at
``lib_path`` disagrees with the fact it checks; ``tests/test_oracle.py`` runs
them against the real library and against planted mistakes in copies of it.
"""
from __future__ import annotations

import numpy as np

import oracle


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def _loss(q, k, v, dout, scale, causal, align):
    """sum(dO * O) with O from the (separately pinned) forward oracle."""
    o, _ = oracle.attention(q, k, v, scale, causal, causal_align=align)
    return float(np.sum(o * dout.astype(np.float64)))


def pin_finite_differences(lib_path=oracle.BWD_LIBRARY):
    """The gradient of sum(dO * O) with respect to chosen elements of Q, K and
    V, by central differences of the forward oracle, for square and
    non-square shapes, causal masks of both alignments, several heads."""
    cases = [((2, 6, 6, 4), False, "top-left"), ((1, 5, 9, 3), True, "bottom-right"),
             ((1, 8, 4, 3), True, "bottom-right"), ((2, 7, 7, 5), True, "top-left")]
    for c, ((BH, nq, nk, D), causal, align) in enumerate(cases):
        q, k, v = _rand((BH, nq, D), 300 + c), _rand((BH, nk, D), 310 + c), _rand((BH, nk, D), 320 + c)
        dout = _rand((BH, nq, D), 330 + c)
        scale = 0.7
        dq, dk, dv = oracle.attention_bwd(q, k, v, dout, scale, causal, align, lib_path=lib_path)
        rng = np.random.default_rng(340 + c)
        for name, x, g in (("Q", q, dq), ("K", k, dk), ("V", v, dv)):
            for _ in range(4):
                idx = tuple(int(rng.integers(0, n)) for n in x.shape)
                h = np.float32(2.0 ** -8)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args = {"Q": (xp, k, v), "K": (q, xp, v), "V": (q, k, xp)}[name]
                argm = {"Q": (xm, k, v), "K": (q, xm, v), "V": (q, k, xm)}[name]
                fd = (_loss(*args, dout, scale, causal, align) - _loss(*argm, dout, scale, causal, align)) \
                    / (float(xp[idx]) - float(xm[idx]))
                err = abs(fd - g[idx])
                assert err <= 2e-5 * max(1.0, abs(g[idx])), \
                    f"d{name}{idx} case {c}: oracle {g[idx]:.9g} vs finite difference {fd:.9g}"


def pin_key_gradients_sum_to_zero(lib_path=oracle.BWD_LIBRARY):
    """Each row of dS sums to 0 over its keys (sum_j P_ij (dP_ij - D_i) =
    D_i - D_i), so the key gradients sum to 0 over the keys: sum_j dK_j = 0;
    and since each row of P sums to 1, sum_j dV_j = sum_i dO_i over the rows
    that see a key."""
    for causal, align, (nq, nk) in ((False, "top-left", (9, 13)), (True, "top-left", (11, 11)),
                                    (True, "bottom-right", (12, 5))):
        q, k, v = _rand((2, nq, 6), 350), _rand((2, nk, 6), 351), _rand((2, nk, 6), 352)
        dout = _rand((2, nq, 6), 353)
        _, dk, dv = oracle.attention_bwd(q, k, v, dout, 0.4, causal, align, lib_path=lib_path)
        assert np.abs(dk.sum(axis=1)).max() <= 1e-12, "sum over keys of dK"
        coff = 0 if align == "top-left" or not causal else nk - nq
        sees = np.array([(not causal) or (i + coff >= 0) for i in range(nq)])
        want = dout[:, sees].astype(np.float64).sum(axis=1)
        assert np.abs(dv.sum(axis=1) - want).max() <= 1e-12, "sum over keys of dV"


def pin_single_key(lib_path=oracle.BWD_LIBRARY):
    """One key: P = 1, so dS = 0 (dQ = dK = 0) and dV_0 = sum_i dO_i."""
    q, k, v, dout = _rand((1, 6, 4), 360), _rand((1, 1, 4), 361), _rand((1, 1, 4), 362), _rand((1, 6, 4), 363)
    dq, dk, dv = oracle.attention_bwd(q, k, v, dout, 0.5, False, lib_path=lib_path)
    assert np.abs(dq).max() <= 1e-14 and np.abs(dk).max() <= 1e-14
    assert np.abs(dv[0, 0] - dout[0].astype(np.float64).sum(axis=0)).max() <= 1e-13


def pin_zero_upstream(lib_path=oracle.BWD_LIBRARY):
    """dO = 0 gives zero gradients."""
    q, k, v = _rand((1, 5, 4), 370), _rand((1, 6, 4), 371), _rand((1, 6, 4), 372)
    grads = oracle.attention_bwd(q, k, v, np.zeros((1, 5, 4), np.float32), 0.5, True, lib_path=lib_path)
    assert all((g == 0).all() for g in grads)


def pin_constant_values(lib_path=oracle.BWD_LIBRARY):
    """Equal value rows make O independent of the scores: dQ = dK = 0."""
    q, k, dout = _rand((1, 7, 4), 380), _rand((1, 7, 4), 381), _rand((1, 7, 4), 382)
    v = np.tile(_rand((1, 1, 4), 383), (1, 7, 1))
    dq, dk, _ = oracle.attention_bwd(q, k, v, dout, 0.5, True, lib_path=lib_path)
    assert np.abs(dq).max() <= 1e-13 and np.abs(dk).max() <= 1e-13


def pin_unseen_rows_and_keys(lib_path=oracle.BWD_LIBRARY):
    """Bottom-right causal with more queries than keys: the first Nq - Nk rows
    see no key and get dQ = 0; under a top-left mask with more keys than
    queries, keys j >= Nq are seen by no query and get dK = dV = 0."""
    q, k, v, dout = _rand((1, 8, 3), 390), _rand((1, 3, 3), 391), _rand((1, 3, 3), 392), _rand((1, 8, 3), 393)
    dq, _, _ = oracle.attention_bwd(q, k, v, dout, 0.5, True, "bottom-right", lib_path=lib_path)
    assert (dq[0, :5] == 0).all() and np.abs(dq[0, 5:]).max() > 0
    q, k, v, dout = _rand((1, 3, 3), 394), _rand((1, 8, 3), 395), _rand((1, 8, 3), 396), _rand((1, 3, 3), 397)
    _, dk, dv = oracle.attention_bwd(q, k, v, dout, 0.5, True, "top-left", lib_path=lib_path)
    assert (dk[0, 3:] == 0).all() and (dv[0, 3:] == 0).all()


def pin_sampled_finite_differences(lib_path=oracle.BWD_LIBRARY):
    """The single-head, selected-output gradients (attention_bwd_sampled)
    against central differences of the forward oracle's sum(dO * O), for
    chosen elements of the selected rows of Q and key rows of K and V, under
    no mask and under causal masks of both alignments."""
    cases = [((7, 9, 4), False, "top-left"), ((9, 6, 3), True, "bottom-right"),
             ((8, 8, 5), True, "top-left")]
    for c, ((nq, nk, D), causal, align) in enumerate(cases):
        q, k, v = _rand((nq, D), 400 + c), _rand((nk, D), 410 + c), _rand((nk, D), 420 + c)
        dout = _rand((nq, D), 430 + c)
        scale = 0.6
        rows, cols = np.array([0, nq // 2, nq - 1]), np.array([0, nk // 3, nk - 1])
        dq, dk, dv = oracle.attention_bwd_sampled(q, k, v, dout, scale, causal, rows, cols,
                                                  causal_align=align, lib_path=lib_path)
        rng = np.random.default_rng(440 + c)
        for name, x, sel, g in (("Q", q, rows, dq), ("K", k, cols, dk), ("V", v, cols, dv)):
            for r in range(len(sel)):
                d = int(rng.integers(0, D))
                idx = (int(sel[r]), d)
                h = np.float32(2.0 ** -8)
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args = {"Q": (xp, k, v), "K": (q, xp, v), "V": (q, k, xp)}[name]
                argm = {"Q": (xm, k, v), "K": (q, xm, v), "V": (q, k, xm)}[name]
                fd = (_loss(*args, dout, scale, causal, align) - _loss(*argm, dout, scale, causal, align)) \
                    / (float(xp[idx]) - float(xm[idx]))
                err = abs(fd - g[r, d])
                assert err <= 2e-5 * max(1.0, abs(g[r, d])), \
                    f"sampled d{name}{idx} case {c}: oracle {g[r, d]:.9g} vs finite difference {fd:.9g}"


def pin_sampled_matches_full(lib_path=oracle.BWD_LIBRARY):
    """The selected-output gradients equal the corresponding rows of the full
    explicit gradients (two separately written evaluations of one
    definition), including rows that see no key and keys no row sees."""
    for nq, nk, causal, align in ((23, 31, False, "top-left"), (30, 17, True, "bottom-right"),
                                  (19, 40, True, "top-left"), (1, 5, True, "bottom-right")):
        q, k, v, dout = _rand((nq, 8), 450), _rand((nk, 8), 451), _rand((nk, 8), 452), _rand((nq, 8), 453)
        dq, dk, dv = oracle.attention_bwd(q[None], k[None], v[None], dout[None], 0.45, causal, align,
                                          lib_path=lib_path)
        rows, cols = np.arange(nq), np.arange(nk)
        sq, sk, sv = oracle.attention_bwd_sampled(q, k, v, dout, 0.45, causal, rows, cols,
                                                  causal_align=align, lib_path=lib_path)
        for what, a, b in (("dQ", sq, dq[0]), ("dK", sk, dk[0]), ("dV", sv, dv[0])):
            assert np.abs(a - b).max() <= 1e-12 * max(1.0, np.abs(b).max()), \
                f"{what} {nq}x{nk} causal={causal} {align}: sampled and full gradients differ"


ALL_PINS = [pin_finite_differences, pin_key_gradients_sum_to_zero, pin_single_key,
            pin_zero_upstream, pin_constant_values, pin_unseen_rows_and_keys,
            pin_sampled_finite_differences, pin_sampled_matches_full]
