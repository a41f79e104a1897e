"""Pins of the variable-length (packed token-major) oracle: to the pinned
grouped-query oracle sequence by sequence, to the isolation of sequences, and
to closed forms at Q = 0 including queries that see no key."""
import numpy as np
import pytest

import oracle

LENS_Q = [3, 0, 5, 1, 4]
LENS_K = [3, 2, 9, 0, 2]      # sequence 4 (causal) has more queries than keys


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def _pack(seed, H, Hkv, d):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((sum(LENS_Q), H, d))
    k = rng.standard_normal((sum(LENS_K), Hkv, d))
    v = rng.standard_normal((sum(LENS_K), Hkv, d))
    return q, k, v


@pytest.mark.parametrize("causal", [False, True])
def test_each_sequence_is_grouped_attention(causal):
    """A sequence with Nq <= Nk equals attention_gqa of its own tokens."""
    q, k, v = _pack(1, 6, 2, 8)
    cq, ck = _cu(LENS_Q), _cu(LENS_K)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 0.35, causal)
    for b in (0, 2):
        qs = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]
        ks = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        vs = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
        og, lg = oracle.attention_gqa(qs, ks, vs, 0.35, causal)
        np.testing.assert_allclose(o[cq[b]:cq[b + 1]], og[0].transpose(1, 0, 2), atol=1e-14)
        np.testing.assert_allclose(l[cq[b]:cq[b + 1]], lg[0].T, atol=1e-14)


@pytest.mark.parametrize("causal", [False, True])
def test_sequences_are_isolated(causal):
    """Changing every token of the other sequences leaves a sequence's output
    bit for bit unchanged."""
    q, k, v = _pack(2, 4, 4, 8)
    cq, ck = _cu(LENS_Q), _cu(LENS_K)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 0.5, causal)
    q2, k2, v2 = _pack(3, 4, 4, 8)
    b = 2
    q2[cq[b]:cq[b + 1]] = q[cq[b]:cq[b + 1]]
    k2[ck[b]:ck[b + 1]] = k[ck[b]:ck[b + 1]]
    v2[ck[b]:ck[b + 1]] = v[ck[b]:ck[b + 1]]
    o2, l2 = oracle.attention_varlen(q2, k2, v2, cq, ck, 0.5, causal)
    np.testing.assert_array_equal(o2[cq[b]:cq[b + 1]], o[cq[b]:cq[b + 1]])
    np.testing.assert_array_equal(l2[cq[b]:cq[b + 1]], l[cq[b]:cq[b + 1]])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_queries_closed_form(causal):
    """Q = 0: every visible score is 0, so LSE = ln(#visible keys) and O is the
    mean of the visible V rows; a query that sees no key has O = 0 and
    LSE = -inf."""
    H, Hkv, d = 4, 2, 3
    _, k, v = _pack(4, H, Hkv, d)
    q = np.zeros((sum(LENS_Q), H, d))
    cq, ck = _cu(LENS_Q), _cu(LENS_K)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 0.7, causal)
    for b, (nq, nk) in enumerate(zip(LENS_Q, LENS_K)):
        for i in range(nq):
            n_vis = nk if not causal else max(0, min(nk, i + (nk - nq) + 1))
            t = cq[b] + i
            for h in range(H):
                if n_vis == 0:
                    assert l[t, h] == -np.inf and np.all(o[t, h] == 0)
                else:
                    assert abs(l[t, h] - np.log(n_vis)) < 1e-14
                    want = v[ck[b]:ck[b] + n_vis, h // (H // Hkv)].mean(axis=0)
                    np.testing.assert_allclose(o[t, h], want, atol=1e-14)


def test_permuting_sequences_permutes_outputs():
    H, Hkv, d = 2, 1, 5
    q, k, v = _pack(5, H, Hkv, d)
    cq, ck = _cu(LENS_Q), _cu(LENS_K)
    o, l = oracle.attention_varlen(q, k, v, cq, ck, 0.4, True)
    order = [3, 0, 4, 2, 1]
    qp = np.concatenate([q[cq[b]:cq[b + 1]] for b in order])
    kp = np.concatenate([k[ck[b]:ck[b + 1]] for b in order])
    vp = np.concatenate([v[ck[b]:ck[b + 1]] for b in order])
    cqp = _cu([LENS_Q[b] for b in order])
    ckp = _cu([LENS_K[b] for b in order])
    op, lp = oracle.attention_varlen(qp, kp, vp, cqp, ckp, 0.4, True)
    np.testing.assert_array_equal(op, np.concatenate([o[cq[b]:cq[b + 1]] for b in order]))
    np.testing.assert_array_equal(lp, np.concatenate([l[cq[b]:cq[b + 1]] for b in order]))


def _mutant_global_keys(q, k, v, cu_q, cu_k, scale, causal):
    """Planted mistake: every sequence attends to all keys of the batch."""
    n = len(cu_q) - 1
    return oracle.attention_varlen(q, k, v, [0] + [len(q)] * n, [0] + [len(k)] * n, scale, causal)


def _mutant_top_left(q, k, v, cu_q, cu_k, scale, causal):
    """Planted mistake: the causal diagonal aligned top-left (j <= i)."""
    o, l = oracle.attention_varlen(q, k, v, cu_q, cu_k, scale, False)
    if not causal:
        return o, l
    o, l = o.copy(), l.copy()
    for b in range(len(cu_q) - 1):
        q0, q1, k0 = int(cu_q[b]), int(cu_q[b + 1]), int(cu_k[b])
        nk = int(cu_k[b + 1]) - k0
        for i in range(q1 - q0):
            n_vis = min(nk, i + 1)
            if n_vis == 0:
                continue
            kk = {0: k0, 1: k0 + n_vis}
            oo, ll = oracle.attention_varlen(q[q0 + i:q0 + i + 1], k[kk[0]:kk[1]], v[kk[0]:kk[1]],
                                             [0, 1], [0, n_vis], scale, False)
            o[q0 + i], l[q0 + i] = oo[0], ll[0]
    return o, l


@pytest.mark.parametrize("mutant", [_mutant_global_keys, _mutant_top_left])
def test_planted_mistakes_fail_a_pin(mutant):
    H, Hkv, d = 4, 2, 3
    _, k, v = _pack(4, H, Hkv, d)
    q = np.zeros((sum(LENS_Q), H, d))
    cq, ck = _cu(LENS_Q), _cu(LENS_K)
    o, l = mutant(q, k, v, cq, ck, 0.7, True)
    ok = True
    for b, (nq, nk) in enumerate(zip(LENS_Q, LENS_K)):
        for i in range(nq):
            n_vis = max(0, min(nk, i + (nk - nq) + 1))
            t = cq[b] + i
            want = -np.inf if n_vis == 0 else np.log(n_vis)
            if not np.allclose(l[t], want, atol=1e-12):
                ok = False
    assert not ok, "the Q = 0 closed form did not catch the planted mistake"
