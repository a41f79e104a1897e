"""The backward oracle against its pins, and planted mistakes against the pins."""
import numpy as np
import pytest

import oracle
from oracle.attention_bwd import attention_bwd_head
from tests import oracle_bwd_pins as pins


@pytest.mark.parametrize("pin", pins.PINS, ids=lambda p: p.__name__)
def test_backward_oracle_pin(pin):
    pin(attention_bwd_head)


def test_bhnd_matches_head():
    rng = np.random.default_rng(35)
    q, k, v, do = (rng.standard_normal((2, 3, 10, 4)) for _ in range(4))
    dq, dk, dv, delta = oracle.attention_bwd_bhnd(q, k, v, do, 0.5, True)
    a = attention_bwd_head(q[1, 2], k[1, 2], v[1, 2], do[1, 2], 0.5, True)
    for x, y in zip((dq[1, 2], dk[1, 2], dv[1, 2], delta[1, 2]), a):
        np.testing.assert_array_equal(x, y)


def _mutant(kind):
    def bwd(q, k, v, do, scale, causal):
        q, k, v, do = (np.asarray(a, dtype=np.float64) for a in (q, k, v, do))
        rows = np.arange(q.shape[0])
        o, lse = oracle.attention_rows(q, k, v, rows, scale, causal)
        s = scale * (q @ k.T)
        if causal and kind != "no_mask":
            s = np.where(np.arange(k.shape[0])[None, :] > rows[:, None], -np.inf, s)
        p = np.exp(s - lse[:, None])
        dv = p.T @ do
        dp = do @ v.T
        delta = np.sum(do * o, axis=1)
        if kind == "delta_from_dp":
            delta = np.sum(dp, axis=1)
        ds = p * (dp - delta[:, None]) if kind != "ds_sign" else p * (dp + delta[:, None])
        if kind == "ds_no_p":
            ds = dp - delta[:, None]
        dq = scale * (ds @ k)
        dk = scale * (ds.T @ q)
        if kind == "dq_no_scale":
            dq = ds @ k
        if kind == "dk_swapped":
            dk = scale * (ds @ q)           # dS instead of dS^T (square shapes only)
        if kind == "dv_from_dp":
            dv = dp.T @ do
        if kind == "dq_uses_v":
            dq = scale * (ds @ v)
        return dq, dk, dv, delta
    return bwd


MUTANTS = ["no_mask", "delta_from_dp", "ds_sign", "ds_no_p", "dq_no_scale", "dk_swapped",
           "dv_from_dp", "dq_uses_v"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_planted_mistake_is_caught(kind):
    bwd = _mutant(kind)
    try:
        bad = pins.failing_pins(bwd)
    except ValueError:
        bad = ["shape error"]     # a transposed operand that cannot even multiply
    assert bad, f"mutant {kind} passed every backward pin"


def test_unmutated_copy_passes():
    assert pins.failing_pins(_mutant("none")) == []


@pytest.mark.parametrize("causal", [False, True])
def test_sampled_matches_full(causal):
    rng = np.random.default_rng(36)
    N, d = 70, 8
    q, k, v, do = (rng.standard_normal((N, d)) for _ in range(4))
    rows = np.array([0, 1, 33, 69])
    keys = np.array([0, 5, 64, 69])
    dq, dk, dv, _ = attention_bwd_head(q, k, v, do, 0.4, causal)
    sq, sk, sv = oracle.attention_bwd_sampled(q, k, v, do, rows, keys, 0.4, causal)
    np.testing.assert_allclose(sq, dq[rows], atol=1e-12)
    np.testing.assert_allclose(sk, dk[keys], atol=1e-12)
    np.testing.assert_allclose(sv, dv[keys], atol=1e-12)
