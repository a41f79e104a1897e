"""Planted mistakes in the oracle (on the CPU) must each fail at least one pin.

Every mutant below is the oracle's ``attention_rows`` with one plausible
mistake: a dropped term, a wrong sign or index, a transposed operand, a wrong
mask or log base. If a mutant passed every pin, the pins would not pin that part
of the oracle. The online recurrence gets the same treatment against the
online == two-pass identity, including the inverted rescale printed in one of
the pages' listings (the FA3 walkthrough's Algorithm 1 rescale step, read as a
garble there).
"""
import numpy as np
import pytest

import oracle
from tests.oracle_pins import failing_pins


def _mk(score_fn=None, mask="gt", softmax="ok", out="ok", lse="ln"):
    def attn(q, k, v, rows, scale, causal):
        q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
        rows = np.asarray(rows, dtype=np.int64)
        s = score_fn(q, k, rows, scale) if score_fn else scale * (q[rows] @ k.T)
        if causal:
            keys = np.arange(k.shape[0])[None, :]
            r = rows[:, None]
            bad = {"gt": keys > r, "ge": keys >= r, "lt": keys < r,
                   "off1": keys > r + 1}[mask]
            s = np.where(bad, -np.inf, s)
        m = np.max(s, axis=1)
        e = np.exp(s - m[:, None])
        ell = e.sum(axis=1)
        if softmax == "ok":
            p = e / ell[:, None]
        elif softmax == "no_norm":
            p = e
        elif softmax == "num_unshifted":
            p = np.exp(s) / ell[:, None]
        elif softmax == "axis0":
            e0 = np.exp(s - np.max(s, axis=0, keepdims=True))
            p = e0 / e0.sum(axis=0, keepdims=True)
        elif softmax == "sq":
            p = e * e / (e * e).sum(axis=1, keepdims=True)
        o = {"ok": lambda: p @ v,
             "pt": lambda: (p.T @ v[: p.shape[0]]) if p.shape[0] == p.shape[1] else p @ v[::-1],
             "vrev": lambda: p @ v[::-1]}[out]()
        lse_v = {"ln": lambda: m + np.log(ell), "log2": lambda: m + np.log2(ell),
                 "drop": lambda: m, "nolog": lambda: m + ell,
                 "sign": lambda: m - np.log(ell)}[lse]()
        return o, lse_v
    return attn


MUTANTS = {
    "transposed_scores": _mk(score_fn=lambda q, k, r, sc: sc * (k @ q.T)[r]
                             if q.shape[0] == k.shape[0] else sc * (q[r] @ k[::-1].T)),
    "no_scale": _mk(score_fn=lambda q, k, r, sc: q[r] @ k.T),
    "scale_twice": _mk(score_fn=lambda q, k, r, sc: sc * sc * (q[r] @ k.T)),
    "sqrt_scale": _mk(score_fn=lambda q, k, r, sc: np.sqrt(sc) * (q[r] @ k.T)),
    "negated_scores": _mk(score_fn=lambda q, k, r, sc: -sc * (q[r] @ k.T)),
    "mask_includes_diagonal": _mk(mask="ge"),
    "mask_wrong_direction": _mk(mask="lt"),
    "mask_off_by_one": _mk(mask="off1"),
    "missing_normalisation": _mk(softmax="no_norm"),
    "numerator_not_shifted": _mk(softmax="num_unshifted"),
    "softmax_over_queries": _mk(softmax="axis0"),
    "squared_weights": _mk(softmax="sq"),
    "pv_transposed": _mk(out="pt"),
    "v_rows_reversed": _mk(out="vrev"),
    "lse_log2": _mk(lse="log2"),
    "lse_dropped_log": _mk(lse="drop"),
    "lse_sum_not_log": _mk(lse="nolog"),
    "lse_sign": _mk(lse="sign"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    assert failing_pins(MUTANTS[name]), f"mutant {name} passed every pin"


def test_true_oracle_passes_every_pin():
    assert failing_pins(oracle.attention_rows) == []


def _online(variant):
    """Deferred-normalisation recurrence with one planted mistake."""
    def run(q, k, v, scale, causal, splits):
        N = q.shape[0]
        rows = np.arange(N)
        m = np.full(N, -np.inf)
        ell = np.zeros(N)
        acc = np.zeros((N, v.shape[1]))
        start = 0
        for size in splits:
            blk = slice(start, start + size)
            s = scale * (q @ k[blk].T)
            if causal:
                s = np.where(np.arange(start, start + size)[None, :] > rows[:, None], -np.inf, s)
            m_new = np.maximum(m, s.max(axis=1))
            ref = np.where(np.isfinite(m_new), m_new, 0.0)
            alpha = np.exp(m - ref)
            if variant == "inverted_alpha":
                alpha = np.where(np.isfinite(m), np.exp(ref - m), 0.0)
            p = np.exp(s - ref[:, None])
            ell = (ell if variant == "ell_not_rescaled" else alpha * ell) + p.sum(axis=1)
            acc = (acc if variant == "o_not_rescaled" else alpha[:, None] * acc) + p @ v[blk]
            m = m if variant == "max_not_updated" and start else m_new
            start += size
        return acc / ell[:, None], m + np.log(ell)
    return run


@pytest.mark.parametrize("variant", ["inverted_alpha", "ell_not_rescaled",
                                     "o_not_rescaled", "max_not_updated"])
def test_online_mutant_is_caught(variant):
    rng = np.random.default_rng(7)
    N, d = 64, 8
    q, k, v = (rng.standard_normal((N, d)) * 2 for _ in range(3))
    o, lse = oracle.attention_head(q, k, v, 0.5, True)
    with np.errstate(all="ignore"):
        o2, lse2 = _online(variant)(q, k, v, 0.5, True, [5, 11, 16, 32])
    assert not (np.allclose(o2, o, atol=1e-9) and np.allclose(lse2, lse, atol=1e-9))
