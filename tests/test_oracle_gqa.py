"""Pins of the grouped-query / key-value-history oracle to the pinned
single-head oracle and to closed forms."""
import numpy as np
import pytest

import oracle


def _r(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("causal", [False, True])
def test_reduces_to_mha(causal):
    """Hkv = H and Nq = Nk: the plain per-head oracle."""
    q, k, v = _r(1, 2, 3, 20, 8), _r(2, 2, 3, 20, 8), _r(3, 2, 3, 20, 8)
    o, l = oracle.attention_gqa(q, k, v, 0.4, causal)
    o2, l2 = oracle.attention_bhnd(q, k, v, 0.4, causal)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(l, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_grouped_equals_repeated_kv(causal):
    """Each group of H/Hkv query heads sees one K/V head: the same as repeating
    K and V H/Hkv times along the head axis."""
    q, k, v = _r(4, 2, 8, 11, 6), _r(5, 2, 2, 11, 6), _r(6, 2, 2, 11, 6)
    o, l = oracle.attention_gqa(q, k, v, 0.7, causal)
    kr, vr = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, l2 = oracle.attention_bhnd(q, kr, vr, 0.7, causal)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    np.testing.assert_allclose(l, l2, atol=1e-14)


def test_last_rows_of_full_causal():
    """The Nq queries are the last Nq positions: their results equal the last
    Nq rows of causal attention over all Nk positions."""
    Nk, Nq = 37, 5
    qf, k, v = _r(7, 1, 2, Nk, 4), _r(8, 1, 2, Nk, 4), _r(9, 1, 2, Nk, 4)
    of, lf = oracle.attention_bhnd(qf, k, v, 0.5, True)
    o, l = oracle.attention_gqa(qf[:, :, Nk - Nq:], k, v, 0.5, True)
    np.testing.assert_allclose(o, of[:, :, Nk - Nq:], atol=1e-14)
    np.testing.assert_allclose(l, lf[:, :, Nk - Nq:], atol=1e-14)


def test_single_query_sees_every_key():
    """Nq = 1: the causal mask hides nothing; Q = 0 gives the mean of V and
    LSE = ln Nk."""
    k, v = _r(10, 1, 1, 50, 4), _r(11, 1, 1, 50, 4)
    q = np.zeros((1, 3, 1, 4))
    for causal in (False, True):
        o, l = oracle.attention_gqa(q, k, v, 0.3, causal)
        np.testing.assert_allclose(o[0, :, 0], np.tile(v[0, 0].mean(0), (3, 1)), atol=1e-14)
        np.testing.assert_allclose(l, np.log(50.0), atol=1e-14)
