"""Pins of the longest-first batch order oracle (``oracle.varlen_lpt_order``).

The order is the FA4 walkthrough's variable-length preprocessing: sequences
sorted by the estimated time of their heaviest work tile, heaviest first,
given to the kernel as a permutation virtual index -> actual sequence. Each
pin is a function of the order function, so that planted mistakes (an inverse
permutation, an ascending sort, unstable ties, sequences without queries
counted, weights by total length) can be shown to fail at least one.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "varlen_lpt_order.json")


def _cu(lens):
    return np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)


def pin_page_example(order_fn):
    """The page's worked example: input order 0, 1, 2, 3 runs as 1, 2, 3, 0
    (virtual i -> actual order[i])."""
    g = json.load(open(GOLDEN))
    return order_fn(g["cu_seqlens_q"], g["cu_seqlens_k"], g["max_seqlen_q"], g["max_seqlen_k"],
                    g["num_splits"]) == g["virtual_to_actual"]


def pin_closed_forms(order_fn):
    return all([
        # equal lengths, or lengths already decreasing: the identity
        order_fn(_cu([3] * 5), _cu([200] * 5), 3, 200, 1) == [0, 1, 2, 3, 4],
        order_fn(_cu([1] * 4), _cu([900, 500, 130, 10]), 1, 900, 1) == [0, 1, 2, 3],
        # increasing lengths: reversed
        order_fn(_cu([1] * 4), _cu([10, 130, 500, 900]), 1, 900, 1) == [3, 2, 1, 0],
        # a sequence without queries has no tile and goes last
        order_fn(_cu([0, 1, 1]), _cu([5000, 64, 128]), 1, 5000, 1) == [2, 1, 0],
        # many queries do not make a tile longer: only the keys it streams count
        order_fn(_cu([900, 1]), _cu([64, 128]), 900, 128, 1) == [1, 0],
        # keys split in ranges of 128: both heaviest tiles stream two blocks
        order_fn(_cu([1, 1]), _cu([1000, 100]), 1, 1000, 8) == [0, 1],
    ])


def pin_invariants(order_fn):
    """A permutation, weights (recomputed from the definition here: blocks of
    the heaviest tile) non-increasing along it, equal weights in input order."""
    for seed in range(6):
        rng = np.random.default_rng(seed)
        B = int(rng.integers(2, 60))
        lq = rng.integers(0, 300, size=B)
        lk = rng.choice([0, 1, 64, 65, 128, 700, 1000], size=B)
        splits = int(rng.integers(1, 4))
        mq, mk = int(lq.max()), int(lk.max())
        order = order_fn(_cu(lq), _cu(lk), mq, mk, splits)
        split_keys = math.ceil(math.ceil(mk / splits) / 64) * 64
        w = [0 if lq[b] == 0 else math.ceil(min(int(lk[b]), split_keys) / 64) for b in range(B)]
        if sorted(order) != list(range(B)):
            return False
        for i in range(B - 1):
            a, b = order[i], order[i + 1]
            if w[a] < w[b] or (w[a] == w[b] and a > b):
                return False
    return True


PINS = [pin_page_example, pin_closed_forms, pin_invariants]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_meets_pin(pin):
    assert pin(oracle.varlen_lpt_order)


def test_weights_count_blocks_of_the_heaviest_tile():
    # 65 keys are two 64-key blocks; lengths past the stated maxima are clamped
    assert oracle.varlen_tile_weights(_cu([2, 2, 2]), _cu([64, 65, 300]), 2, 200) == [1, 2, 4]


def _mutant(kind):
    def order_fn(cu_q, cu_k, mq, mk, splits):
        w = oracle.varlen_tile_weights(cu_q, cu_k, mq, mk, splits)
        B = len(w)
        if kind == "ascending":
            return sorted(range(B), key=lambda b: (w[b], b))
        if kind == "inverse":
            o = sorted(range(B), key=lambda b: (-w[b], b))
            inv = [0] * B
            for v, b in enumerate(o):
                inv[b] = v
            return inv
        if kind == "unstable":
            return sorted(range(B), key=lambda b: (-w[b], -b))
        if kind == "count_empty":
            wk = [math.ceil(min(int(cu_k[b + 1] - cu_k[b]), mk) / 64) for b in range(B)]
            return sorted(range(B), key=lambda b: (-wk[b], b))
        if kind == "total_tokens":
            wt = [int(cu_q[b + 1] - cu_q[b]) + int(cu_k[b + 1] - cu_k[b]) for b in range(B)]
            return sorted(range(B), key=lambda b: (-wt[b], b))
        raise ValueError(kind)
    return order_fn


@pytest.mark.parametrize("kind", ["ascending", "inverse", "unstable", "count_empty",
                                  "total_tokens"])
def test_planted_mistake_fails_a_pin(kind):
    fn = _mutant(kind)
    assert not all(pin(fn) for pin in PINS), f"mutant {kind} passes every pin"
