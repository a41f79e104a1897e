"""Checks that pin the fp64 oracle to facts other than itself.

Each ``pin_*`` takes an implementation ``attn(q, k, v, rows, scale, causal)``
returning ``(O[rows], LSE[rows])`` and raises AssertionError when the
implementation violates a fact fixed by the pages or by mathematics:

* softmax rows sum to one (read off with V = identity, so O = P);
* constant V returns V; V-affine and logit-shift equivariance;
* non-causal attention does not depend on the order of the K/V rows;
* closed forms: Q = 0 gives LSE = ln(#visible keys) and O = mean of the visible
  V rows; the first causal row is O_0 = V_0, LSE_0 = scale*q_0.k_0;
* brute force at 50 decimal digits on tiny shapes, with no max-subtraction.

The same functions run against planted mistakes in
``test_oracle_mutants.py`` to show that each mistake trips at least one pin.
"""
from __future__ import annotations

import decimal
from decimal import Decimal

import numpy as np

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _all(attn, q, k, v, scale, causal):
    return attn(q, k, v, np.arange(q.shape[0]), scale, causal)


def pin_rowsum_one(attn):
    """With V = I (d = N), O is P itself: nonnegative, rows sum to one, and the
    causal part above the diagonal is zero."""
    rng = _rng(11)
    for N, causal in ((7, False), (7, True), (33, True)):
        q = rng.standard_normal((N, 5))
        k = rng.standard_normal((N, 5))
        p, _ = _all(attn, q, k, np.eye(N), 0.7, causal)
        assert np.all(p >= -TOL), "negative probability"
        assert np.allclose(p.sum(axis=1), 1.0, atol=TOL, rtol=0), "row sums != 1"
        if causal:
            assert np.all(np.abs(np.triu(p, 1)) <= TOL), "mass on masked keys"


def pin_constant_v(attn):
    rng = _rng(12)
    for causal in (False, True):
        N, d = 19, 6
        q = rng.standard_normal((N, d)) * 3
        k = rng.standard_normal((N, d)) * 3
        v0 = rng.standard_normal(d)
        o, _ = _all(attn, q, k, np.tile(v0, (N, 1)), 0.5, causal)
        assert np.allclose(o, v0[None, :], atol=TOL, rtol=0), "constant V not returned"


def pin_permutation_invariance(attn):
    rng = _rng(13)
    N, d = 23, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, lse = _all(attn, q, k, v, 0.35, False)
    perm = rng.permutation(N)
    o2, lse2 = _all(attn, q, k[perm], v[perm], 0.35, False)
    assert np.allclose(o, o2, atol=TOL, rtol=0), "O depends on K/V order"
    assert np.allclose(lse, lse2, atol=TOL, rtol=0), "LSE depends on K/V order"


def pin_zero_query_closed_form(attn):
    """Q = 0: every visible logit is 0, so LSE_i = ln(#visible keys) and O_i is
    the plain mean of the visible V rows (prefix mean when causal)."""
    rng = _rng(14)
    N, d = 29, 4
    q = np.zeros((N, d))
    k, v = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    o, lse = _all(attn, q, k, v, 0.9, False)
    assert np.allclose(lse, np.log(N), atol=TOL, rtol=0), "LSE(Q=0) != ln N"
    assert np.allclose(o, v.mean(axis=0)[None, :], atol=TOL, rtol=0)
    o, lse = _all(attn, q, k, v, 0.9, True)
    cnt = np.arange(1, N + 1)
    assert np.allclose(lse, np.log(cnt), atol=TOL, rtol=0), "causal LSE(Q=0) != ln(i+1)"
    prefix = np.cumsum(v, axis=0) / cnt[:, None]
    assert np.allclose(o, prefix, atol=TOL, rtol=0), "causal O(Q=0) != prefix mean"


def pin_first_causal_row(attn):
    rng = _rng(15)
    N, d = 17, 9
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o, lse = attn(q, k, v, np.array([0]), 0.6, True)
    assert np.allclose(o[0], v[0], atol=TOL, rtol=0), "O_0 != V_0"
    assert abs(lse[0] - 0.6 * float(q[0] @ k[0])) <= TOL, "LSE_0 != scale*q0.k0"


def pin_logit_shift(attn):
    """K' = K + 1 w^T adds scale*q_i.w to every logit of row i: O unchanged,
    LSE_i shifted by scale*q_i.w (any mask)."""
    rng = _rng(16)
    N, d = 21, 7
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    w = rng.standard_normal(d)
    for causal in (False, True):
        o, lse = _all(attn, q, k, v, 0.45, causal)
        o2, lse2 = _all(attn, q, k + w[None, :], v, 0.45, causal)
        assert np.allclose(o, o2, atol=1e-11, rtol=0), "O changed by a logit shift"
        assert np.allclose(lse2, lse + 0.45 * (q @ w), atol=1e-11, rtol=0)


def pin_v_affine(attn):
    rng = _rng(17)
    N, d = 15, 5
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    a = rng.standard_normal((d, 3))
    b = rng.standard_normal(3)
    for causal in (False, True):
        o, _ = _all(attn, q, k, v, 0.8, causal)
        o2, _ = _all(attn, q, k, v @ a + b[None, :], 0.8, causal)
        assert np.allclose(o2, o @ a + b[None, :], atol=1e-11, rtol=0), "V-affine"


def brute_force_decimal(q, k, v, scale, causal, digits=50):
    """o_i = sum_j e^{s_ij} v_j / sum_j e^{s_ij}, LSE_i = ln sum_j e^{s_ij}, with
    s_ij = scale * q_i . k_j, evaluated in Decimal with ``digits`` digits and no
    max-subtraction. Inputs are converted exactly from binary floats."""
    ctx = decimal.Context(prec=digits)
    N, d = len(q), len(q[0])
    sc = Decimal(float(scale))
    out_o, out_l = [], []
    for i in range(N):
        ws, num = [], [Decimal(0)] * len(v[0])
        for j in range(len(k)):
            if causal and j > i:
                continue
            s = sum((Decimal(float(q[i][t])) * Decimal(float(k[j][t])) for t in range(d)),
                    Decimal(0))
            e = ctx.exp(ctx.multiply(sc, s))
            ws.append(e)
            num = [ctx.add(num[c], ctx.multiply(e, Decimal(float(v[j][c]))))
                   for c in range(len(v[0]))]
        z = sum(ws, Decimal(0))
        out_o.append([float(ctx.divide(x, z)) for x in num])
        out_l.append(float(ctx.ln(z)))
    return np.array(out_o), np.array(out_l)


def pin_brute_force(attn):
    rng = _rng(18)
    for (N, Nk, d, dv), causal, scale in (((5, 5, 3, 2), False, 0.61),
                                          ((6, 6, 4, 3), True, 1.3),
                                          ((3, 7, 2, 4), False, 0.25),
                                          ((8, 8, 4, 4), True, 0.5)):
        q = rng.standard_normal((N, d))
        k = rng.standard_normal((Nk, d))
        v = rng.standard_normal((Nk, dv))
        o, lse = _all(attn, q, k, v, scale, causal)
        bo, bl = brute_force_decimal(q, k, v, scale, causal)
        assert np.allclose(o, bo, atol=1e-13, rtol=0), "O != decimal brute force"
        assert np.allclose(lse, bl, atol=1e-13, rtol=0), "LSE != decimal brute force"


def pin_causal_last_row(attn):
    """The last causal row sees every key, so it equals the non-causal row."""
    rng = _rng(19)
    N, d = 12, 6
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    o1, l1 = attn(q, k, v, np.array([N - 1]), 0.7, True)
    o2, l2 = attn(q, k, v, np.array([N - 1]), 0.7, False)
    assert np.allclose(o1, o2, atol=TOL, rtol=0) and np.allclose(l1, l2, atol=TOL, rtol=0)


ALL_PINS = [
    pin_rowsum_one,
    pin_constant_v,
    pin_permutation_invariance,
    pin_zero_query_closed_form,
    pin_first_causal_row,
    pin_logit_shift,
    pin_v_affine,
    pin_brute_force,
    pin_causal_last_row,
]


def failing_pins(attn):
    """Names of the pins ``attn`` fails (an exception of any kind counts)."""
    bad = []
    for pin in ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(attn)
        except Exception:  # noqa: BLE001 - a crash is a failed pin too
            bad.append(pin.__name__)
    return bad
