"""GPU parity of fa_fwd_varlen (sequences of different lengths packed
token-major) against the fp64 variable-length oracle.

Tolerances as for fa_fwd: max|dO| <= 4e-3 (f16) / 1.6e-2 (bf16), |dLSE| <=
1e-3 on rows that see at least one key; rows that see none must be O = 0 and
LSE = -inf exactly. Cases cover ragged lengths across tile boundaries, empty
query and key sequences, causal sequences with more queries than keys,
grouped heads, key splits, and a prefill-sized batch.
"""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import TOL_LSE, TOL_O, say

pytestmark = pytest.mark.gpu


def run_varlen(case, splits, max_q=None, max_k=None, ordered=False):
    import torch
    import io_aware_softmax_fa_amd as fa
    tdt = torch.float16 if case.dtype == fi.F16 else torch.bfloat16
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()
               for a in (case.q, case.k, case.v))
    cq = torch.from_numpy(case.cu_q).cuda()
    ck = torch.from_numpy(case.cu_k).cuda()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((q.shape[0], case.H), float("nan"), device="cuda")
    mq = max(case.lens_q) if max_q is None else max_q
    mk = max(case.lens_k) if max_k is None else max_k
    order = fa.varlen_order(cq, ck, mq, mk, splits) if ordered else None
    fa.forward_varlen(q, k, v, cq, ck, mq, mk, case.causal, case.scale, num_splits=splits, out=o,
                      lse=lse, order=order)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_varlen(case, splits, label=""):
    say(f"[gpu-varlen] {label} lens_q={case.lens_q[:8]}{'...' if len(case.lens_q) > 8 else ''} "
        f"lens_k={case.lens_k[:8]}{'...' if len(case.lens_k) > 8 else ''} H={case.H} "
        f"Hkv={case.Hkv} d={case.d} dtype={fi.DTYPE_NAMES[case.dtype]} causal={case.causal} "
        f"splits={splits} seed={case.seed}")
    o, lse = run_varlen(case, splits)
    ro, rl = oracle.attention_varlen(case.exact("q"), case.exact("k"), case.exact("v"),
                                     case.cu_q, case.cu_k, case.scale, case.causal)
    empty = np.isneginf(rl)
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0), "rows with no key"
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse[~empty])), "non-finite output"
    do = float(np.max(np.abs(o - ro))) if o.size else 0.0
    dl = float(np.max(np.abs(lse[~empty] - rl[~empty]))) if (~empty).any() else 0.0
    say(f"      max|dO|={do:.3e} max|dLSE|={dl:.3e} empty rows={int(empty.sum())}")
    assert do <= TOL_O[case.dtype] and dl <= TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("dtype,d", [(fi.F16, 64), (fi.BF16, 128)])
def test_ragged_batch(causal, dtype, d):
    lens = (1, 63, 64, 65, 127, 128, 129, 300)
    check_varlen(fi.make_varlen_case(lens, lens, 4, 4, d, dtype, causal, seed=601), 1, "ragged")


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_history(splits, causal):
    """Chunked prefill / decode mix: each sequence's queries are the last ones
    of a longer key history; 8 query heads over 2 K/V heads."""
    lq = (1, 5, 40, 200, 1, 17)
    lk = (700, 5, 333, 257, 64, 1000)
    check_varlen(fi.make_varlen_case(lq, lk, 8, 2, 128, fi.BF16, causal, seed=602), splits,
                 "history")


@pytest.mark.parametrize("causal", [False, True])
def test_empty_sequences_and_rows_without_keys(causal):
    """Empty query sequences, empty key sequences (O = 0, LSE = -inf), and
    causal sequences with more queries than keys (their first rows see no
    key)."""
    lq = (0, 10, 7, 0, 130, 3)
    lk = (5, 0, 20, 0, 60, 3)
    check_varlen(fi.make_varlen_case(lq, lk, 6, 3, 64, fi.F16, causal, seed=603), 1, "empty")
    check_varlen(fi.make_varlen_case(lq, lk, 6, 3, 64, fi.F16, causal, seed=604), 4, "empty-split")


def test_max_seqlen_above_every_length():
    """A grid sized for longer sequences than the batch holds: the extra tiles
    and ranges must do nothing."""
    case = fi.make_varlen_case((30, 90), (50, 90), 4, 2, 128, fi.BF16, True, seed=605)
    o, lse = run_varlen(case, 2, max_q=500, max_k=900)
    ro, rl = oracle.attention_varlen(case.exact("q"), case.exact("k"), case.exact("v"),
                                     case.cu_q, case.cu_k, case.scale, True)
    assert float(np.max(np.abs(o - ro))) <= TOL_O[fi.BF16]
    assert float(np.max(np.abs(lse - rl))) <= TOL_LSE


def test_equals_dense_forward_bitwise():
    """One sequence of N tokens with H = Hkv, unsplit, computes exactly what
    fa_fwd computes on the same data in [B, H, N, d] layout (the same tiles,
    in the same order)."""
    import torch
    import io_aware_softmax_fa_amd as fa
    N, H, d = 700, 4, 128
    case = fi.make_varlen_case((N,), (N,), H, H, d, fi.BF16, True, seed=606)
    o, lse = run_varlen(case, 1)
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)[None]).view(np.int16))
               .view(torch.bfloat16).cuda() for a in (case.q, case.k, case.v))
    od, ld = fa.forward(q, k, v, True, case.scale)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(o, od[0].float().cpu().numpy().transpose(1, 0, 2))
    np.testing.assert_array_equal(lse, ld[0].cpu().numpy().T)


def test_prefill_batch_b8_mixed_lengths_bf16():
    """A prefill-sized batch: 8 sequences of 100..3000 tokens (seeded), 32
    query heads over 8 K/V heads, d = 128, causal; every row against the oracle."""
    rng = np.random.default_rng(607)
    lens = tuple(int(x) for x in rng.integers(100, 3001, size=8))
    check_varlen(fi.make_varlen_case(lens, lens, 32, 8, 128, fi.BF16, True, seed=607), 1,
                 "prefill")


def test_bench_workload_sampled():
    """The benchmark's variable-length workload in the launch it times (the
    longest-first order, then the ordered call): 16 causal sequences with
    lengths uniform in [512, 8192] (seed 620), H=32 over Hkv=8, d=128, bf16.
    Four heads of every sequence are checked at 64 sampled query rows each
    (always the first and last row), against the oracle's full sums over the
    sequence's keys."""
    import torch
    import io_aware_softmax_fa_amd as fa
    lens = [int(x) for x in np.random.default_rng(620).integers(512, 8193, size=16)]
    case = fi.make_varlen_case(lens, lens, 32, 8, 128, fi.BF16, True, seed=620)
    say(f"[gpu-varlen] bench workload: 16 sequences, total {sum(lens)} tokens")
    o, lse = run_varlen(case, 1, ordered=True)
    q, k, v = case.exact("q"), case.exact("k"), case.exact("v")
    rng = np.random.default_rng(621)
    worst_o = worst_l = 0.0
    for b, n in enumerate(lens):
        q0, k0 = int(case.cu_q[b]), int(case.cu_k[b])
        rows = np.unique(np.concatenate([[0, n - 1], rng.integers(0, n, size=62)]))
        for h in (0, 7, 20, 31):
            kh = h // 4
            ro, rl = oracle.attention_rows(q[q0:q0 + n, h], k[k0:k0 + n, kh], v[k0:k0 + n, kh],
                                           rows, case.scale, True)
            worst_o = max(worst_o, float(np.max(np.abs(o[q0 + rows, h] - ro))))
            worst_l = max(worst_l, float(np.max(np.abs(lse[q0 + rows, h] - rl))))
    say(f"      max|dO|={worst_o:.3e} max|dLSE|={worst_l:.3e}")
    assert worst_o <= TOL_O[fi.BF16] and worst_l <= TOL_LSE


# ---------------------------------------------- longest-first sequence order --

def _order_case(lens_q, lens_k, max_q, max_k, splits, label):
    """fa_varlen_order on the GPU against the order oracle, entry by entry."""
    import torch
    import io_aware_softmax_fa_amd as fa
    cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    say(f"[gpu-order] {label} B={len(lens_q)} max_q={max_q} max_k={max_k} splits={splits}")
    got = fa.varlen_order(torch.from_numpy(cu_q).cuda(), torch.from_numpy(cu_k).cuda(), max_q,
                          max_k, splits, total_q=int(cu_q[-1]), total_k=int(cu_k[-1]))
    torch.cuda.synchronize()
    want = oracle.varlen_lpt_order(cu_q, cu_k, max_q, max_k, splits)
    assert got.cpu().tolist() == want


def test_order_page_example():
    import json
    import os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "varlen_lpt_order.json")))
    lq = np.diff(g["cu_seqlens_q"]).tolist()
    lk = np.diff(g["cu_seqlens_k"]).tolist()
    _order_case(lq, lk, g["max_seqlen_q"], g["max_seqlen_k"], g["num_splits"], "page example")


@pytest.mark.parametrize("B", [1, 7, 256, 257, 3000])
@pytest.mark.parametrize("splits", [1, 3])
def test_order_matches_oracle(B, splits):
    """Random lengths with many equal weights (ties keep input order), empty
    query and key sequences, lengths past the stated maxima (clamped), and
    batches over one and several 256-sequence chunks."""
    rng = np.random.default_rng(700 + B + splits)
    lq = rng.choice([0, 1, 5, 130, 1000], size=B)
    lk = rng.choice([0, 1, 63, 64, 65, 500, 4096, 9000], size=B)
    _order_case(lq, lk, 900, 8192, splits, "random")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("splits", [1, 3])
def test_ordered_run_equals_input_order(causal, splits):
    """The order changes which sequences run first, not what any output row
    holds: O and LSE equal the input-order run bit for bit (and the oracle)."""
    import torch
    import io_aware_softmax_fa_amd as fa
    lens_q = (300, 1, 0, 700, 64, 129, 5, 1000)
    lens_k = (300, 900, 40, 700, 64, 129, 2000, 1000)
    case = fi.make_varlen_case(lens_q, lens_k, 8, 2, 128, fi.BF16, causal, seed=710 + splits)
    say(f"[gpu-order] ordered run causal={causal} splits={splits}")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
               for a in (case.q, case.k, case.v))
    cq, ck = torch.from_numpy(case.cu_q).cuda(), torch.from_numpy(case.cu_k).cuda()
    mq, mk = max(lens_q), max(lens_k)
    order = fa.varlen_order(cq, ck, mq, mk, splits)
    outs = []
    for ordr in (None, order):
        o = torch.full_like(q, float("nan"))
        lse = torch.full((q.shape[0], 8), float("nan"), device="cuda")
        fa.forward_varlen(q, k, v, cq, ck, mq, mk, causal, case.scale, num_splits=splits, out=o,
                          lse=lse, order=ordr)
        torch.cuda.synchronize()
        outs.append((o.cpu(), lse.cpu()))
    assert order.cpu().tolist() != list(range(len(lens_q)))      # the order does move sequences
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
    check_varlen(case, splits, "input order")
