"""GPU: the allocation-free split-KV entry point (fa_fwd_kv_noalloc) against
fa_fwd_kv with a caller workspace, through the C ABI.

Both run the same kernels with the same key ranges, so the outputs must be
equal bit for bit; the smaller case is also held to the fp64 oracle at the
bf16/fp16 tolerances. Two calls in a row, the second smaller than the first,
show that the shared static scratch carries nothing from one call into the
next (every partial a call reads, it wrote)."""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import TOL_LSE, TOL_O, say

pytestmark = pytest.mark.gpu


def _dev(a, dtype):
    import torch
    tdt = torch.float16 if dtype == fi.F16 else torch.bfloat16
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()


def _run_both(case, splits):
    import torch
    import io_aware_softmax_fa_amd as fa
    q, k, v = (_dev(a, case.dtype) for a in (case.q, case.k, case.v))
    B, H, Nq, d = q.shape
    o1 = torch.full_like(q, float("nan"))
    l1 = torch.full((B, H, Nq), float("nan"), device="cuda")
    o2, l2 = torch.full_like(o1, float("nan")), torch.full_like(l1, float("nan"))
    ws = torch.empty(max(fa.fa_fwd_kv_workspace(B, H, Nq, d, splits) // 4, 1), dtype=torch.float32,
                     device="cuda")
    fa.forward_kv_noalloc(q, k, v, case.causal, case.scale, num_splits=splits, out=o1, lse=l1)
    fa.forward_kv(q, k, v, case.causal, case.scale, num_splits=splits, out=o2, lse=l2, workspace=ws)
    torch.cuda.synchronize()
    return (o1.float().cpu().numpy(), l1.cpu().numpy(), o2.float().cpu().numpy(),
            l2.cpu().numpy())


def test_noalloc_matches_workspace_entry_two_calls():
    # first call: the benchmark's decode step (B=8, H=32 over Hkv=8, one query,
    # 32768 keys, bf16, causal), 8 ranges; second: a smaller grouped prefill
    big = fi.make_kv_case(8, 32, 8, 1, 32768, 128, fi.BF16, True, seed=530)
    small = fi.make_kv_case(2, 8, 2, 4, 3000, 64, fi.F16, True, seed=531)
    for case, splits, label in ((big, 8, "decode"), (small, 3, "small")):
        say(f"[gpu-noalloc] {label} B={case.B} H={case.H} Hkv={case.Hkv} Nq={case.Nq} "
            f"Nk={case.Nk} d={case.d} splits={splits}")
        o1, l1, o2, l2 = _run_both(case, splits)
        assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
        np.testing.assert_array_equal(o1, o2)
        np.testing.assert_array_equal(l1, l2)
        if label == "small":
            ro, rl = oracle.attention_gqa(case.exact("q"), case.exact("k"), case.exact("v"),
                                          case.scale, case.causal)
            do, dl = float(np.max(np.abs(o1 - ro))), float(np.max(np.abs(l1 - rl)))
            say(f"      vs oracle: max|dO|={do:.3e} max|dLSE|={dl:.3e}")
            assert do <= TOL_O[case.dtype] and dl <= TOL_LSE


def test_noalloc_rejects_partials_past_the_scratch():
    import torch
    import io_aware_softmax_fa_amd as fa
    q = torch.zeros((4, 32, 64, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((4, 8, 4096, 128), dtype=torch.bfloat16, device="cuda")
    need = fa.fa_fwd_kv_workspace(4, 32, 64, 128, 8)
    assert need > fa.FA_NOALLOC_SCRATCH_BYTES
    with pytest.raises(fa.FaError) as e:
        fa.forward_kv_noalloc(q, k, k, True, num_splits=8)
    assert e.value.code == fa.FA_ERR_TOO_LARGE
    # the default split count is lowered to what the scratch holds
    o, lse = fa.forward_kv_noalloc(q, k, k, True)
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all() and torch.isfinite(lse).all()
