"""The fp64 oracle against facts fixed by the pages and by mathematics."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(oracle.attention_rows)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_online_recurrences_equal_two_pass(causal, seed):
    """Both online update rules ("FlashAttention · InkStack" 1.1.2 and 2.1),
    with random key-block splits of 1..97, reach the two-pass result."""
    rng = np.random.default_rng(100 + seed)
    N, d = 211, 16
    q, k, v = (rng.standard_normal((N, d)) * 2 for _ in range(3))
    o, lse = oracle.attention_head(q, k, v, 0.3, causal)
    splits = []
    left = N
    while left:
        s = int(min(left, rng.integers(1, 98)))
        splits.append(s)
        left -= s
    for fn in (oracle.online_attention_head, oracle.online_attention_head_fa1):
        o2, lse2 = fn(q, k, v, 0.3, causal, splits)
        np.testing.assert_allclose(o2, o, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse2, lse, atol=1e-12, rtol=0)
    # one key at a time is the recurrence of the MUSA guide's online softmax
    o3, lse3 = oracle.online_attention_head(q, k, v, 0.3, causal)
    np.testing.assert_allclose(o3, o, atol=1e-12, rtol=0)
    np.testing.assert_allclose(lse3, lse, atol=1e-12, rtol=0)


def test_rows_match_full_head():
    rng = np.random.default_rng(3)
    N, d = 300, 8
    q, k, v = (rng.standard_normal((N, d)) for _ in range(3))
    rows = np.array([0, 1, 17, 255, 256, 299])
    for causal in (False, True):
        o, lse = oracle.attention_head(q, k, v, 0.4, causal)
        o2, lse2 = oracle.attention_rows(q, k, v, rows, 0.4, causal)
        # same arithmetic, possibly another BLAS blocking: equal to rounding
        np.testing.assert_allclose(o2, o[rows], atol=1e-14, rtol=0)
        np.testing.assert_allclose(lse2, lse[rows], atol=1e-14, rtol=0)


def test_bhnd_is_per_head():
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((2, 3, 20, 4)) for _ in range(3))
    o, lse = oracle.attention_bhnd(q, k, v, 0.5, True)
    assert o.shape == (2, 3, 20, 4) and lse.shape == (2, 3, 20)
    o11, l11 = oracle.attention_head(q[1, 2], k[1, 2], v[1, 2], 0.5, True)
    np.testing.assert_array_equal(o[1, 2], o11)
    np.testing.assert_array_equal(lse[1, 2], l11)


def test_large_logits_do_not_overflow():
    """Safe softmax: logits near 1e3 (e^1000 overflows fp64) stay finite."""
    N, d = 9, 2
    q = np.full((N, d), 30.0)
    k = np.full((N, d), 30.0)
    k[3] = 31.0
    v = np.arange(N * d, dtype=np.float64).reshape(N, d)
    o, lse = oracle.attention_head(q, k, v, 1.0, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    # key 3 dominates by e^{60}: O ~= V_3
    np.testing.assert_allclose(o, np.tile(v[3], (N, 1)), atol=1e-20, rtol=1e-12)
