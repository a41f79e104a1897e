"""CPU oracle for the longest-first order of a variable-length batch.

TEST INFRASTRUCTURE ONLY (see the package docstring). Only ``tests/``, the
smoke check and the benchmark's CPU-baseline leg may use it.

The FA4 walkthrough's variable-length section describes a preprocessing step
that estimates, for every sequence of the batch, the execution time of its
heaviest work tile, sorts the sequences by that estimate from the heaviest
down, and hands the attention kernel a permutation "virtual index -> actual
sequence": the kernel walks virtual sequences 0, 1, 2, ... and reads the data
of the actual sequence the permutation names, so that the longest tiles start
first (longest-processing-time order) without moving any tensor.

Readings taken here (the page gives the idea, not a formula):

* a work tile is one query tile of one sequence (over one key range when the
  keys are split); its execution time is proportional to the number of
  64-key K/V blocks it streams. The heaviest tile of sequence b streams
  ceil(min(Nk_b, split_keys) / 64) blocks when it has a query (with the
  bottom-right causal mask the last query row sees every key), and nothing
  when Nq_b = 0;
* lengths are those the attention kernel uses: offsets clamped to the
  totals and lengths to the stated maxima;
* sequences of equal weight keep their input order (a stable sort), so the
  permutation is unique.
"""
from __future__ import annotations

import math


def varlen_tile_weights(cu_q, cu_k, max_q: int, max_k: int, num_splits: int = 1,
                        block: int = 64) -> list[int]:
    """K/V blocks streamed by the heaviest work tile of each sequence."""
    B = len(cu_q) - 1
    total_q, total_k = int(cu_q[B]), int(cu_k[B])
    per = -(-max_k // num_splits) if max_k > 0 else 0
    split_keys = -(-per // block) * block
    w = []
    for b in range(B):
        q0 = min(max(int(cu_q[b]), 0), total_q)
        q1 = min(max(int(cu_q[b + 1]), q0), total_q)
        k0 = min(max(int(cu_k[b]), 0), total_k)
        k1 = min(max(int(cu_k[b + 1]), k0), total_k)
        nq, nk = min(q1 - q0, max_q), min(k1 - k0, max_k)
        w.append(0 if nq <= 0 else math.ceil(min(nk, split_keys) / block))
    return w


def varlen_lpt_order(cu_q, cu_k, max_q: int, max_k: int, num_splits: int = 1,
                     block: int = 64) -> list[int]:
    """The permutation virtual index -> actual sequence, heaviest tile first,
    ties in input order."""
    w = varlen_tile_weights(cu_q, cu_k, max_q, max_k, num_splits, block)
    return sorted(range(len(w)), key=lambda b: (-w[b], b))
