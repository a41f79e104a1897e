"""The entry points inside a captured HIP graph: each call queues only
kernels on the caller's stream (no allocation, no memset, no host sync), so
a graph captured around it replays the same results. Each graph is replayed
several times with eager work and synchronisation between replays, and every
replay must equal the eager result bit for bit."""
import numpy as np
import pytest

import fa_inputs as fi
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu


def _replays_match(fn, outs, eager, n=3):
    import torch
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    for i in range(n):
        for t in outs:
            t.fill_(float("nan") if t.is_floating_point() else 0)
        torch.cuda.synchronize()
        g.replay()
        junk = torch.randn(1 << 20, device="cuda").sum()   # eager work between replays
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), f"replay {i} differs from the eager result"
        del junk


@pytest.mark.parametrize("causal", [True, False])
def test_forward_in_graph(causal):
    """Causal at this length runs 128-row tiles, non-causal 256-row tiles."""
    import torch
    import io_aware_softmax_fa_amd as fa
    case = fi.make_case(2, 4, 700, 128, fi.BF16, causal, seed=800)
    say(f"[gpu-graph] fa_fwd B=2 H=4 N=700 d=128 bf16 causal={causal}")
    q, k, v = to_device(case)
    o, lse = torch.empty_like(q), torch.empty((2, 4, 700), device="cuda")
    eo, el = fa.forward(q, k, v, causal, case.scale)
    torch.cuda.synchronize()
    _replays_match(lambda: fa.forward(q, k, v, causal, case.scale, out=o, lse=lse), (o, lse),
                   (eo, el))


def test_split_kv_and_merge_in_graph():
    import torch
    import io_aware_softmax_fa_amd as fa
    case = fi.make_kv_case(2, 8, 2, 1, 5000, 128, fi.BF16, True, seed=801)
    say("[gpu-graph] fa_fwd_kv B=2 H=8 Hkv=2 Nq=1 Nk=5000 splits=4")
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
               for a in (case.q, case.k, case.v))
    ws = torch.empty(fa.fa_fwd_kv_workspace(2, 8, 1, 128, 4) // 4, device="cuda")
    o, lse = torch.empty_like(q), torch.empty((2, 8, 1), device="cuda")
    eo, el = fa.forward_kv(q, k, v, True, case.scale, num_splits=4, workspace=ws)
    torch.cuda.synchronize()
    _replays_match(lambda: fa.forward_kv(q, k, v, True, case.scale, num_splits=4, out=o, lse=lse,
                                         workspace=ws), (o, lse), (eo, el))


def test_backward_in_graph():
    import torch
    import io_aware_softmax_fa_amd as fa
    case = fi.make_case(1, 2, 500, 64, fi.F16, False, seed=802)
    say("[gpu-graph] fa_bwd B=1 H=2 N=500 d=64 f16")
    q, k, v = to_device(case)
    bits, _ = fi.make_dout(case, case.seed)
    g = torch.from_numpy(bits.view(np.int16)).view(torch.float16).cuda()
    o, lse = fa.forward(q, k, v, False, case.scale)
    ws = torch.empty(2 * 500 * 2, device="cuda")
    dq, dk, dv = (torch.empty_like(q) for _ in range(3))
    e = fa.backward(q, k, v, o, lse, g, False, case.scale, workspace=ws)
    e = tuple(t.clone() for t in e)
    torch.cuda.synchronize()
    _replays_match(lambda: fa.backward(q, k, v, o, lse, g, False, case.scale, dq=dq, dk=dk, dv=dv,
                                       workspace=ws), (dq, dk, dv), e)
