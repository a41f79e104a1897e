"""GPU parity of the backward pass (fa_bwd through the C ABI) against the fp64
backward oracle.

The GPU backward consumes the GPU forward's O and LSE, as a training step
would; the oracle rebuilds everything from the exact inputs. Tolerance, per
gradient tensor: max|d(grad)| <= TOL_BWD[dtype] * max|grad| (or the size of the
terms it sums, where the gradient vanishes). Derivation: P and dS are rounded
to the input type before the products that consume them (relative u = 2^-9
for bf16, 2^-12 for f16, per element) and each gradient is rounded once on
output (same u). The largest term is D = rowsum(dO * O), which the
definition ("FlashAttention · InkStack" 1.2.1) forms from the forward's O,
here the rounded O the forward returns: D_i picks up an error of up to
u * sum_d |dO_id O_id| (typically u * sqrt(d) |dO_i| |O_i| / sqrt(3)), and dQ_i
then moves by scale * dD_i * |sum_j P_ij k_j|. In rows with few visible keys
(early causal rows) O_i is close to one V row and the dS_ij nearly cancel, so
this term dominates: with N(0,1) data at d = 128 it reaches about 1.5% of
max|dQ| (row 1 of a causal head). Hence 3e-2 for bf16; f16's u is 8x smaller.
"""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import say, to_device

pytestmark = pytest.mark.gpu

TOL_BWD = {fi.F16: 5e-3, fi.BF16: 3e-2}


def run_bwd(case, dout_bits):
    import torch
    import io_aware_softmax_fa_amd as fa
    q, k, v = to_device(case)
    tdt = torch.float16 if case.dtype == fi.F16 else torch.bfloat16
    g = torch.from_numpy(np.ascontiguousarray(dout_bits).view(np.int16)).view(tdt).cuda()
    o, lse = fa.forward(q, k, v, case.causal, case.scale)
    dq, dk, dv = (torch.full_like(q, float("nan")) for _ in range(3))
    fa.backward(q, k, v, o, lse, g, case.causal, case.scale, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]


def check_bwd(case, label=""):
    say(f"[gpu-bwd] {label} B={case.B} H={case.H} N={case.N} d={case.d} "
        f"dtype={fi.DTYPE_NAMES[case.dtype]} causal={case.causal} seed={case.seed}")
    bits, g = fi.make_dout(case, case.seed)
    got = run_bwd(case, bits)
    ref = oracle.attention_bwd_bhnd(case.exact("q"), case.exact("k"), case.exact("v"), g,
                                    case.scale, case.causal)[:3]
    # A gradient can vanish exactly (one visible key: dS = 0, so dQ = dK = 0);
    # its scale is then that of the terms it sums: scale*|dO||V||K or Q| for
    # dQ and dK, |dO| for dV.
    q, k, v = (np.max(np.abs(case.exact(w))) for w in "qkv")
    gmax = np.max(np.abs(g))
    floors = (case.scale * gmax * v * k, case.scale * gmax * v * q, gmax)
    worst = 0.0
    for name, a, r, fl in zip(("dQ", "dK", "dV"), got, ref, floors):
        assert np.all(np.isfinite(a)), f"non-finite {name}"
        rel = float(np.max(np.abs(a - r)) / max(np.max(np.abs(r)), fl))
        say(f"      {name}: max|d|/max|ref| = {rel:.3e}  (max|ref| {np.max(np.abs(r)):.3e})")
        worst = max(worst, rel)
    assert worst <= TOL_BWD[case.dtype], f"backward error {worst:.3e} > {TOL_BWD[case.dtype]}"


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_grid(dtype, d, causal):
    check_bwd(fi.make_case(2, 3, 384, d, dtype, causal, seed=301), label="grid")


@pytest.mark.parametrize("N", [1, 2, 31, 63, 65, 100, 127, 129, 200, 255, 257, 700])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_ragged(N, causal):
    d = 128 if N % 2 else 64
    dt = fi.BF16 if N % 2 else fi.F16
    check_bwd(fi.make_case(1, 2, N, d, dt, causal, seed=400 + N), label="ragged")


@pytest.mark.parametrize("dtype,d", [(fi.F16, 64), (fi.BF16, 128), (fi.F16, 128), (fi.BF16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_sharp_softmax(dtype, d, causal):
    """Scale 1 on N(0,1) Q and K (logits sqrt(d) times wider than at the
    default scale): P is nearly one-hot in most rows, P = exp(S - LSE) is
    rebuilt from LSEs of tens, and dS nearly cancels. V at a quarter of unit
    spread, as in the forward's sharp case."""
    N = 400
    rng = np.random.default_rng(310 + 2 * d + dtype)
    q = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    k = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    v = rng.standard_normal((1, 2, N, d), dtype=np.float32) * np.float32(0.25)
    case = fi.from_exact(q, k, v, dtype, causal, scale=1.0)
    case.seed = 311
    check_bwd(case, label="sharp")


def test_bwd_b2_h4_n2048_d128_bf16_causal():
    check_bwd(fi.make_case(2, 4, 2048, 128, fi.BF16, True, seed=302), label="n2048")


def test_bwd_deterministic():
    case = fi.make_case(1, 2, 640, 128, fi.BF16, True, seed=303)
    bits, _ = fi.make_dout(case, case.seed)
    a = run_bwd(case, bits)
    b = run_bwd(case, bits)
    for x, y in zip(a, b):
        np.testing.assert_array_equal(x, y)


def test_bwd_workspace_holds_delta():
    """The first B*H*N workspace values are -D = -rowsum(dO * O) of the O the
    forward wrote (recomputed here on the host from those device values)."""
    import torch
    import io_aware_softmax_fa_amd as fa
    case = fi.make_case(1, 2, 300, 64, fi.F16, False, seed=304)
    bits, _ = fi.make_dout(case, case.seed)
    q, k, v = to_device(case)
    g = torch.from_numpy(bits.view(np.int16)).view(torch.float16).cuda()
    o, lse = fa.forward(q, k, v, False, case.scale)
    ws = torch.empty(2 * case.B * case.H * case.N, dtype=torch.float32, device="cuda")
    fa.backward(q, k, v, o, lse, g, False, case.scale, workspace=ws)
    torch.cuda.synchronize()
    want = -(o.double() * g.double()).sum(-1).flatten().cpu().numpy()
    got = ws[: case.B * case.H * case.N].double().cpu().numpy()
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("causal", [False, True])
def test_bwd_b2_h32_n8192_d128_bf16_sampled(causal):
    """The benchmark's backward workload at full size, in the launch the
    benchmark times; two heads are checked at 256 sampled query rows (dQ) and
    256 sampled key rows (dK, dV), each against the full sums of the oracle."""
    case = fi.make_case(2, 32, 8192, 128, fi.BF16, causal, seed=3)
    say(f"[gpu-bwd] full size causal={causal}")
    bits, g = fi.make_dout(case, case.seed)
    got = run_bwd(case, bits)
    q, k, v = case.exact("q"), case.exact("k"), case.exact("v")
    for b, h in ((0, 0), (1, 31)):
        rows = fi.sample_rows(case.seed, b, h, case.N)
        keys = fi.sample_rows(case.seed + 1, b, h, case.N)
        ref = oracle.attention_bwd_sampled(q[b, h], k[b, h], v[b, h], g[b, h], rows, keys,
                                           case.scale, causal)
        outs = (got[0][b, h][rows], got[1][b, h][keys], got[2][b, h][keys])
        for name, a, r in zip(("dQ", "dK", "dV"), outs, ref):
            rel = float(np.max(np.abs(a - r)) / np.max(np.abs(r)))
            say(f"      head ({b},{h}) {name}: max|d|/max|ref| = {rel:.3e}")
            assert rel <= TOL_BWD[fi.BF16], f"{name} error {rel:.3e}"
