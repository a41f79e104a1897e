"""Checks that pin the fp64 backward oracle to facts other than itself.

Each ``pin_*`` takes an implementation ``bwd(q, k, v, do, scale, causal)``
returning ``(dQ, dK, dV, D)`` and raises AssertionError when it violates a fact
fixed by mathematics:

* central finite differences of the scalar ``sum(O * dO)`` (the forward is
  the separately pinned forward oracle), on tiny shapes, causal and not;
* every softmax row sums to one, so ``sum_j dV_j = sum_i dO_i`` and every row
  of dS sums to zero, so ``sum_j dK_j = 0``;
* adding one vector to every key leaves P, hence all gradients, unchanged;
* Q = 0 gives uniform weights over the visible keys: ``dV_j`` is the sum of
  ``dO_i / n_i`` over the queries i that see key j, and ``D_i`` is
  ``dO_i`` dotted with the mean of the visible V rows.

``test_oracle_bwd.py`` runs them on the oracle; the same functions run
against planted mistakes in that file to show each mistake trips a pin.
"""
from __future__ import annotations

import numpy as np

import oracle


def _rng(seed):
    return np.random.default_rng(seed)


def _loss(q, k, v, do, scale, causal):
    o, _ = oracle.attention_rows(q, k, v, np.arange(q.shape[0]), scale, causal)
    return float(np.sum(o * do))


def pin_finite_differences(bwd):
    rng = _rng(31)
    h = 1e-5
    for Nq, Nk, d, causal in ((5, 5, 3, False), (5, 5, 3, True), (4, 6, 2, False), (6, 6, 4, True)):
        q = rng.standard_normal((Nq, d))
        k = rng.standard_normal((Nk, d))
        v = rng.standard_normal((Nk, d))
        do = rng.standard_normal((Nq, d))
        scale = 0.6
        dq, dk, dv, _ = bwd(q, k, v, do, scale, causal)
        for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
            num = np.zeros_like(x)
            for idx in np.ndindex(x.shape):
                xp, xm = x.copy(), x.copy()
                xp[idx] += h
                xm[idx] -= h
                args_p = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
                args_m = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
                num[idx] = (_loss(*args_p, do, scale, causal) - _loss(*args_m, do, scale, causal)) / (2 * h)
            assert np.allclose(g, num, atol=1e-7, rtol=1e-6), \
                f"{name} differs from finite differences (causal={causal}): {np.max(np.abs(g - num))}"


def pin_column_sums(bwd):
    rng = _rng(32)
    for N, causal in ((9, False), (9, True), (17, True)):
        q, k, v, do = (rng.standard_normal((N, 4)) for _ in range(4))
        dq, dk, dv, _ = bwd(q, k, v, do, 0.8, causal)
        assert np.allclose(dv.sum(axis=0), do.sum(axis=0), atol=1e-12), "sum_j dV_j != sum_i dO_i"
        assert np.allclose(dk.sum(axis=0), 0.0, atol=1e-12), "sum_j dK_j != 0"


def pin_key_shift(bwd):
    rng = _rng(33)
    for N, causal in ((8, False), (8, True)):
        q, k, v, do = (rng.standard_normal((N, 3)) for _ in range(4))
        c = rng.standard_normal(3)
        a = bwd(q, k, v, do, 0.9, causal)
        b = bwd(q, k + c[None, :], v, do, 0.9, causal)
        for x, y, name in zip(a, b, ("dQ", "dK", "dV", "D")):
            assert np.allclose(x, y, atol=1e-11), f"{name} changes when every key is shifted"


def pin_zero_query(bwd):
    rng = _rng(34)
    for N, causal in ((7, False), (7, True)):
        q = np.zeros((N, 3))
        k, v, do = (rng.standard_normal((N, 3)) for _ in range(3))
        _, _, dv, delta = bwd(q, k, v, do, 0.5, causal)
        n = np.arange(1, N + 1) if causal else np.full(N, N)
        want_dv = np.zeros_like(v)
        mean_v = np.zeros_like(do)
        for i in range(N):
            vis = range(i + 1) if causal else range(N)
            for j in vis:
                want_dv[j] += do[i] / n[i]
            mean_v[i] = v[list(vis)].mean(axis=0)
        assert np.allclose(dv, want_dv, atol=1e-12), "dV for uniform weights"
        assert np.allclose(delta, np.sum(do * mean_v, axis=1), atol=1e-12), "D for uniform weights"


PINS = (pin_finite_differences, pin_column_sums, pin_key_shift, pin_zero_query)


def failing_pins(bwd):
    bad = []
    for pin in PINS:
        try:
            pin(bwd)
        except AssertionError:
            bad.append(pin.__name__)
    return bad
