"""Pins for the fp64 attention oracle: facts fixed by the pages and by
mathematics, not by the oracle's own code.

Each ``pin_*`` function raises AssertionError when the oracle library at
``lib_path`` disagrees with the fact it checks. ``tests/test_oracle.py`` runs
them against the real oracle and against deliberately broken copies of it
(a dropped term, a wrong sign or index, a transposed operand) to show that
each plausible mistake fails at least one pin.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext

import numpy as np
import scipy.special

import oracle

RNG_SEED = 1234


def _rand(shape, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal(shape) * scale).astype(np.float32)


def decimal_attention(q, k, v, scale, causal, n_kv=None, coff=0, prec=60):
    """Brute force in high-precision decimal straight from the definition:
    O_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij}, LSE_i = ln sum_j e^{s_ij},
    s_ij = scale * q_i . k_j, over visible keys (j < n_kv, and j <= i + coff
    if causal). No max subtraction: exact arithmetic does not need it.
    q: [Nq, D], k, v: [Nk, D] float32. Returns (O, LSE) as float64 arrays.
    """
    Nq, D = q.shape
    Nk = k.shape[0]
    n_kv = Nk if n_kv is None else n_kv
    o = np.zeros((Nq, D))
    lse = np.full(Nq, -np.inf)
    with localcontext() as ctx:
        ctx.prec = prec
        sc = Decimal(float(scale))
        qd = [[Decimal(float(x)) for x in row] for row in q]
        kd = [[Decimal(float(x)) for x in row] for row in k]
        vd = [[Decimal(float(x)) for x in row] for row in v]
        for i in range(Nq):
            vis = [j for j in range(n_kv) if (not causal or j <= i + coff)]
            if not vis:
                continue
            w = {j: (sc * sum(a * b for a, b in zip(qd[i], kd[j]))).exp() for j in vis}
            den = sum(w.values())
            for d in range(D):
                o[i, d] = float(sum(w[j] * vd[j][d] for j in vis) / den)
            lse[i] = float(den.ln())
    return o, lse


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    same_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    with np.errstate(invalid="ignore"):
        err = np.where(same_inf, 0.0, np.abs(a - b))
    bound = tol * np.maximum(1.0, np.where(same_inf, 1.0, np.abs(b)))
    bad = ~(err <= bound)
    assert not bad.any(), f"{what}: max err {np.nanmax(np.where(bad, err, 0))}"


# ---------------------------------------------------------------------------
# Pins


def pin_decimal_brute_force(lib_path=oracle.LIBRARY):
    """Exact-order brute force on tiny inputs (high-precision decimal)."""
    for seed, (N, D), causal, n_kv in [
        (1, (7, 5), False, None), (2, (7, 5), True, None),
        (3, (9, 4), False, 6), (4, (9, 4), True, 5), (5, (1, 3), False, None),
    ]:
        q, k, v = (_rand((N, D), seed * 10 + t) for t in range(3))
        scale = 1.0 / math.sqrt(D)
        o, lse = oracle.attention(q[None], k[None], v[None], scale, causal, n_kv,
                                  lib_path=lib_path)
        o_ref, lse_ref = decimal_attention(q, k, v, scale, causal, n_kv)
        _close(o[0], o_ref, 1e-13, f"O brute force seed {seed}")
        _close(lse[0], lse_ref, 1e-13, f"LSE brute force seed {seed}")


def pin_scipy_softmax(lib_path=oracle.LIBRARY):
    """Library special case: per row, the weights are scipy's softmax of the
    scores and LSE is scipy's logsumexp (scores summed exactly with fsum)."""
    N, D = 12, 6
    q, k, v = (_rand((N, D), 40 + t) for t in range(3))
    scale = 0.37
    for causal in (False, True):
        o, lse = oracle.attention(q[None], k[None], v[None], scale, causal,
                                  lib_path=lib_path)
        for i in range(N):
            n_vis = i + 1 if causal else N
            s = np.array([scale * math.fsum(float(a) * float(b) for a, b in zip(q[i], k[j]))
                          for j in range(n_vis)])
            w = scipy.special.softmax(s)
            o_ref = np.array([math.fsum(w[j] * float(v[j, d]) for j in range(n_vis))
                              for d in range(D)])
            _close(o[0, i], o_ref, 1e-14, "O vs scipy softmax")
            _close(lse[0, i], scipy.special.logsumexp(s), 1e-14, "LSE vs scipy logsumexp")


def pin_rows_sum_to_one(lib_path=oracle.LIBRARY):
    """With V = identity (D = N), O is the probability matrix P itself: each
    row is non-negative, sums to 1, and is exactly 0 on masked keys."""
    N = 24
    q, k = _rand((N, N), 50), _rand((N, N), 51)
    v = np.eye(N, dtype=np.float32)
    for causal in (False, True):
        p, _ = oracle.attention(q[None], k[None], v[None], 0.3, causal, lib_path=lib_path)
        p = p[0]
        assert (p >= 0).all(), "negative probability"
        assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-14 * N, "rows do not sum to 1"
        if causal:
            assert (np.triu(p, 1) == 0).all(), "future key has weight"


def pin_single_key(lib_path=oracle.LIBRARY):
    """N = 1: the only key gets weight 1, so O = V and LSE = scale * q.k."""
    D = 16
    q, k, v = (_rand((1, D), 60 + t) for t in range(3))
    for causal in (False, True):
        o, lse = oracle.attention(q[None], k[None], v[None], 0.25, causal, lib_path=lib_path)
        assert np.array_equal(o[0, 0], v[0].astype(np.float64)), "O != V for one key"
        expect = 0.25 * math.fsum(float(a) * float(b) for a, b in zip(q[0], k[0]))
        _close(lse[0, 0], expect, 1e-15, "LSE for one key")


def pin_constant_values(lib_path=oracle.LIBRARY):
    """Every value row equal to c gives O = c (weights sum to one)."""
    N, D = 33, 8
    q, k = _rand((N, D), 70), _rand((N, D), 71)
    c = _rand((1, D), 72)
    v = np.repeat(c, N, axis=0)
    for causal in (False, True):
        o, _ = oracle.attention(q[None], k[None], v[None], 0.5, causal, lib_path=lib_path)
        _close(o[0], np.repeat(c.astype(np.float64), N, axis=0), 1e-15, "constant V")


def pin_key_permutation(lib_path=oracle.LIBRARY):
    """Non-causal attention is a set function of the (key, value) pairs:
    permuting K and V rows together changes nothing."""
    N, D = 31, 8
    q, k, v = (_rand((N, D), 80 + t) for t in range(3))
    perm = np.random.default_rng(81).permutation(N)
    o1, l1 = oracle.attention(q[None], k[None], v[None], 0.4, False, lib_path=lib_path)
    o2, l2 = oracle.attention(q[None], k[perm][None], v[perm][None], 0.4, False,
                              lib_path=lib_path)
    _close(o1, o2, 1e-14, "O under key permutation")
    _close(l1, l2, 1e-14, "LSE under key permutation")


def pin_zero_queries(lib_path=oracle.LIBRARY):
    """Q = 0: all visible scores are 0, so O is the mean of the visible value
    rows and LSE = log(number of visible keys); causal gives prefix means."""
    N, D = 20, 8
    q = np.zeros((N, D), dtype=np.float32)
    k, v = _rand((N, D), 90), _rand((N, D), 91)
    o, lse = oracle.attention(q[None], k[None], v[None], 0.7, False, lib_path=lib_path)
    _close(o[0], np.repeat(v.astype(np.float64).mean(axis=0, keepdims=True), N, 0),
           1e-14, "Q=0 mean")
    _close(lse[0], np.full(N, math.log(N)), 1e-15, "Q=0 LSE")
    o, lse = oracle.attention(q[None], k[None], v[None], 0.7, True, lib_path=lib_path)
    prefix = np.cumsum(v.astype(np.float64), axis=0) / np.arange(1, N + 1)[:, None]
    _close(o[0], prefix, 1e-14, "Q=0 causal prefix mean")
    _close(lse[0], np.log(np.arange(1, N + 1)), 1e-15, "Q=0 causal LSE")


def pin_causal_first_row(lib_path=oracle.LIBRARY):
    """Under the top-left causal mask query 0 sees only key 0."""
    N, D = 17, 8
    q, k, v = (_rand((N, D), 100 + t) for t in range(3))
    o, lse = oracle.attention(q[None], k[None], v[None], 0.3, True, lib_path=lib_path)
    assert np.array_equal(o[0, 0], v[0].astype(np.float64)), "causal row 0 != V[0]"
    _close(lse[0, 0], 0.3 * math.fsum(float(a) * float(b) for a, b in zip(q[0], k[0])),
           1e-15, "causal row 0 LSE")
    # and row 1 sees exactly keys 0 and 1
    s = [0.3 * math.fsum(float(a) * float(b) for a, b in zip(q[1], k[j])) for j in (0, 1)]
    w = scipy.special.softmax(s)
    _close(o[0, 1], w[0] * v[0].astype(np.float64) + w[1] * v[1].astype(np.float64),
           1e-15, "causal row 1")


def pin_value_shift(lib_path=oracle.LIBRARY):
    """Adding a constant c to every value row adds c to every output."""
    N, D = 19, 8
    q, k, v = (_rand((N, D), 110 + t) for t in range(3))
    v = np.round(v * 256) / 256          # multiples of 2^-8: v + c is exact in fp32
    c = np.float32(3.0)
    for causal in (False, True):
        o1, _ = oracle.attention(q[None], k[None], v[None], 0.3, causal, lib_path=lib_path)
        o2, _ = oracle.attention(q[None], k[None], (v + c)[None], 0.3, causal,
                                 lib_path=lib_path)
        _close(o2 - o1, np.full_like(o1, 3.0), 1e-13, "value shift")


def pin_power_of_two_rescale(lib_path=oracle.LIBRARY):
    """(2Q, scale/2) gives bit-identical scores, hence identical outputs."""
    N, D = 21, 8
    q, k, v = (_rand((N, D), 120 + t) for t in range(3))
    for causal in (False, True):
        o1, l1 = oracle.attention(q[None], k[None], v[None], 0.3, causal, lib_path=lib_path)
        o2, l2 = oracle.attention((2 * q)[None], k[None], v[None], 0.15, causal,
                                  lib_path=lib_path)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), "2Q, scale/2 differs"


def pin_large_scores(lib_path=oracle.LIBRARY):
    """Scores far beyond exp's range (Q amplified 1024x) must stay finite and
    match the exact brute force ("Building a Verifiable FlashAttention
    Forward", Part 4: amplified Q/K and a finiteness check)."""
    N, D = 9, 16
    q = _rand((N, D), 130, scale=1024.0)
    k, v = _rand((N, D), 131), _rand((N, D), 132)
    for causal in (False, True):
        o, lse = oracle.attention(q[None], k[None], v[None], 0.25, causal, lib_path=lib_path)
        assert np.isfinite(o).all() and np.isfinite(lse).all(), "non-finite output"
        o_ref, lse_ref = decimal_attention(q, k, v, 0.25, causal, prec=80)
        _close(o[0], o_ref, 1e-12, "O large scores")
        _close(lse[0], lse_ref, 1e-13, "LSE large scores")


def pin_no_visible_key(lib_path=oracle.LIBRARY):
    """A row that sees no key (key length 0) gives O = 0 and LSE = -inf."""
    N, D = 5, 4
    q, k, v = (_rand((N, D), 140 + t) for t in range(3))
    for causal in (False, True):
        o, lse = oracle.attention(q[None], k[None], v[None], 0.5, causal, n_kv=0,
                                  lib_path=lib_path)
        assert (o == 0).all() and np.isneginf(lse).all(), "empty key set"


def pin_multi_head_rows(lib_path=oracle.LIBRARY):
    """Heads are independent: the rows API over several heads matches each
    head's brute force, for any row order."""
    BH, N, D = 3, 6, 4
    q, k, v = (_rand((BH, N, D), 150 + t) for t in range(3))
    rows = np.array([(2, 5), (0, 0), (1, 3), (2, 0), (0, 5)])
    o, lse = oracle.attention_rows(q, k, v, 0.5, True, rows, lib_path=lib_path)
    for r, (bh, i) in enumerate(rows):
        o_ref, lse_ref = decimal_attention(q[bh], k[bh], v[bh], 0.5, True)
        _close(o[r], o_ref[i], 1e-13, f"head {bh} row {i}")
        _close(lse[r], lse_ref[i], 1e-13, f"head {bh} row {i} LSE")


def pin_cross_attention_brute_force(lib_path=oracle.LIBRARY):
    """Query and key lengths are separate ("Triton: FlashAttention-2 Forward
    Pass", Masks and sentinels: Q rows and the output use the query length,
    the key loop and K/V rows the key length). Several heads, Nq < Nk and
    Nq > Nk, both causal alignments ("How to profile and optimise kernels",
    Round 4: top-left as SDPA's is_causal, bottom-right as FlashAttention
    since 2.1), against the decimal brute force."""
    BH, D = 2, 3
    for seed, (nq, nk) in enumerate([(3, 7), (7, 3), (1, 2), (4, 4)]):
        q = _rand((BH, nq, D), 160 + seed)
        k = _rand((BH, nk, D), 170 + seed)
        v = _rand((BH, nk, D), 180 + seed)
        for causal, align in ((False, "top-left"), (True, "top-left"), (True, "bottom-right")):
            coff = 0 if align == "top-left" else nk - nq
            o, lse = oracle.attention(q, k, v, 0.6, causal, causal_align=align,
                                      lib_path=lib_path)
            for bh in range(BH):
                o_ref, lse_ref = decimal_attention(q[bh], k[bh], v[bh], 0.6, causal, coff=coff)
                what = f"Nq={nq} Nk={nk} causal={causal} {align} head {bh}"
                _close(o[bh], o_ref, 1e-13, what)
                _close(lse[bh], lse_ref, 1e-13, what + " LSE")


def pin_one_query_two_keys(lib_path=oracle.LIBRARY):
    """One query, two keys with equal scores (Q = 0) and value rows 5 and 10:
    O = 7.5 and LSE = ln 2. The pages report a kernel that took the key
    length from Q returning 5 for a one-query, two-key case ("Triton:
    FlashAttention-2 Forward Pass", Masks and sentinels); here 5 is what
    a top-left causal mask gives, since query 0 then sees key 0 only, while
    the bottom-right alignment (offset Nk - Nq = 1) sees both keys."""
    D = 4
    q = np.zeros((1, 1, D), np.float32)
    k = _rand((1, 2, D), 190)
    v = np.array([[[5.0] * D, [10.0] * D]], np.float32)
    for causal, align, o_want, lse_want in (
            (False, "top-left", 7.5, math.log(2.0)),
            (True, "bottom-right", 7.5, math.log(2.0)),
            (True, "top-left", 5.0, 0.0)):
        o, lse = oracle.attention(q, k, v, 0.5, causal, causal_align=align, lib_path=lib_path)
        _close(o[0, 0], np.full(D, o_want), 1e-15, f"one query two keys {causal} {align}")
        _close(lse[0, 0], lse_want, 1e-15, f"one query two keys LSE {causal} {align}")


def pin_bottom_right_rows(lib_path=oracle.LIBRARY):
    """Bottom-right alignment: the last query row sees every key, so it equals
    the non-causal row; with more queries than keys, the first Nq - Nk rows
    see no key at all (O = 0, LSE = -inf) and row Nq - Nk sees key 0 only
    (O = V[0], LSE = scale q.k_0)."""
    D = 4
    for nq, nk in ((3, 8), (8, 3)):
        q = _rand((1, nq, D), 200 + nq)
        k = _rand((1, nk, D), 210 + nq)
        v = _rand((1, nk, D), 220 + nq)
        o_c, l_c = oracle.attention(q, k, v, 0.4, True, causal_align="bottom-right",
                                    lib_path=lib_path)
        o_n, l_n = oracle.attention(q, k, v, 0.4, False, lib_path=lib_path)
        _close(o_c[0, -1], o_n[0, -1], 1e-15, "last row sees every key")
        _close(l_c[0, -1], l_n[0, -1], 1e-15, "last row LSE")
        if nq > nk:
            first = nq - nk
            assert (o_c[0, :first] == 0).all() and np.isneginf(l_c[0, :first]).all(), \
                "rows above the shifted diagonal see no key"
            _close(o_c[0, first], v[0, 0], 0.0, "first visible row is V[0]")
            s0 = 0.4 * math.fsum(float(a) * float(b) for a, b in zip(q[0, first], k[0, 0]))
            _close(l_c[0, first], s0, 1e-15, "first visible row LSE")


ALL_PINS = [
    pin_decimal_brute_force, pin_scipy_softmax, pin_rows_sum_to_one, pin_single_key,
    pin_constant_values, pin_key_permutation, pin_zero_queries, pin_causal_first_row,
    pin_value_shift, pin_power_of_two_rescale, pin_large_scores, pin_no_visible_key,
    pin_multi_head_rows, pin_cross_attention_brute_force, pin_one_query_two_keys,
    pin_bottom_right_rows,
]
