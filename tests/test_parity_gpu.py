"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Tolerances (max over all compared elements): |dO| <= 4e-3 for fp16 inputs,
1.6e-2 for bf16, 6e-2 for fp8; |dLSE| <= 1e-3. The workloads up to N = 8192
(including the B=2 H=32 N=8192 bf16 pair and the B=4 H=16 N=8192 fp8 case)
compare every row of every head; only the long sequences (N = 32768 and
131072, and the extra long d = 64 heads) compare a seeded sample of 256 rows
per head (always including rows 0, 1, N-1 and the rows either side of two
256-row tile boundaries). All run at the full sizes and in the launch
configuration the benchmark times.
"""
import numpy as np
import pytest

import fa_inputs as fi
from tests.gpu_util import TOL_LSE, TOL_O, check, run_gpu, say, to_device

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ the workloads --

def test_tiny_single_head_fp16():
    check(fi.make_case(1, 1, 256, 64, fi.F16, False, seed=1), label="tiny")


@pytest.mark.parametrize("causal", [False, True])
def test_b4_h16_n2048_d64_fp16(causal):
    check(fi.make_case(4, 16, 2048, 64, fi.F16, causal, seed=2), label="n2048")


@pytest.mark.parametrize("causal", [False, True])
def test_b2_h32_n8192_d128_bf16(causal):
    """The headline workload, every row of all 64 heads."""
    check(fi.make_case(2, 32, 8192, 128, fi.BF16, causal, seed=3), label="n8192")


def test_b1_h16_n32768_d128_bf16_causal():
    check(fi.make_case(1, 16, 32768, 128, fi.BF16, True, seed=41), rows_per_head=256,
          label="n32768")


def test_b1_h4_n131072_d128_bf16_causal():
    check(fi.make_case(1, 4, 131072, 128, fi.BF16, True, seed=42), rows_per_head=256,
          label="n131072")


def test_one_head_of_a_million_keys():
    """The largest head tested: N = 2^20 keys, causal, d = 128, bf16 (768 MB
    of Q, K and V; 4096 query tiles of one head, 64-bit element offsets past
    2^31), against the oracle on 64 seeded rows (rows 0, 1, N-1 and the
    first tile boundaries among them). Drawing the inputs takes most of the
    test's time (about 45 s on the host)."""
    say("[gpu] N=2^20 one head: drawing inputs")
    case = fi.make_case(1, 1, 1 << 20, 128, fi.BF16, True, seed=44)
    check(case, rows_per_head=64, label="n1m")


# ------------------------------------------------------------- edge cases --

@pytest.mark.parametrize("N", [1, 2, 63, 65, 100, 199, 200, 255, 257, 511, 700, 1025])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_ragged_lengths(N, d, causal):
    dt = fi.F16 if d == 64 else fi.BF16
    check(fi.make_case(2, 2, N, d, dt, causal, seed=1000 + N), label="ragged")


@pytest.mark.parametrize("dtype,N", [(fi.F16, 16384), (fi.BF16, 8192)])
def test_d64_long_heads(dtype, N):
    """d = 64 without a mask over long heads (the 64-row waves, 256-row tiles,
    many K/V tiles per workgroup): 256 seeded rows of each of 6 heads, the
    tile edges among them."""
    check(fi.make_case(1, 6, N, 64, dtype, False, seed=13), rows_per_head=256,
          label=f"d64 long N={N}")


@pytest.mark.parametrize("B,H,N,d,dtype", [(3, 40, 1000, 128, fi.BF16), (2, 72, 1537, 128, fi.F16),
                                           (1, 75, 900, 128, fi.BF16), (2, 80, 800, 64, fi.F16),
                                           (1, 150, 1100, 64, fi.BF16)])
def test_more_tiles_than_resident_workgroups(B, H, N, d, dtype):
    """Without a mask and with more 256-row tiles than the chip holds at once
    (256 workgroups at d = 128, 512 at d = 64 on 256 compute units): tiles
    that run in several rounds on one compute unit, ragged last tiles (N not a
    multiple of 256), and tile counts that are (480, 1008, 640) and are not
    (300, 750) a multiple of the 8 XCDs. 64 seeded rows of every head, the
    tile edges among them."""
    check(fi.make_case(B, H, N, d, dtype, False, seed=B * 1000 + H), rows_per_head=64,
          label=f"many tiles B={B} H={H} N={N} d={d}")


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
@pytest.mark.parametrize("d", [64, 128])
def test_every_dtype_and_head_dim(dtype, d):
    for causal in (False, True):
        check(fi.make_case(1, 3, 1280, d, dtype, causal, seed=7), label="grid")


@pytest.mark.parametrize("d,dtype", [(128, fi.BF16), (64, fi.F16)])
@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_form(causal, d, dtype):
    """Q = 0: LSE_i = ln(#visible keys) exactly in real arithmetic, O_i = mean
    of the visible V rows (every head; d = 64 without a mask runs the
    64-row waves)."""
    N = 777
    rng = np.random.default_rng(9)
    q = np.zeros((1, 2, N, d), np.float32)
    k = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    v = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    case = fi.from_exact(q, k, v, dtype, causal)
    say(f"[gpu] Q=0 closed form d={d} causal={causal}")
    o, lse = run_gpu(case)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    for h in range(2):
        np.testing.assert_allclose(lse[0, h], np.log(cnt), atol=TOL_LSE, rtol=0)
        vx = case.exact("v")[0, h]
        want = np.cumsum(vx, axis=0) / cnt[:, None] if causal else np.tile(vx.mean(0), (N, 1))
        assert np.max(np.abs(o[0, h] - want)) <= TOL_O[dtype]


@pytest.mark.parametrize("causal", [True, False])
def test_constant_v_returns_v(causal):
    N, d = 1000, 64
    rng = np.random.default_rng(10)
    q = rng.standard_normal((1, 1, N, d), dtype=np.float32) * 3
    k = rng.standard_normal((1, 1, N, d), dtype=np.float32) * 3
    v0 = rng.standard_normal(d).astype(np.float32)
    v = np.broadcast_to(v0, (1, 1, N, d)).copy()
    case = fi.from_exact(q, k, v, fi.F16, causal)
    say(f"[gpu] constant V causal={causal}")
    o, _ = run_gpu(case)
    want = case.exact("v")[0, 0, 0]
    assert np.max(np.abs(o[0, 0] - want[None, :])) <= TOL_O[fi.F16]


def test_first_causal_row_is_v0():
    case = fi.make_case(1, 2, 300, 128, fi.BF16, True, seed=12)
    say("[gpu] first causal row")
    o, lse = run_gpu(case)
    v0 = case.exact("v")[:, :, 0]
    q0, k0 = case.exact("q")[:, :, 0], case.exact("k")[:, :, 0]
    # a single visible key: P = 1 exactly, so O_0 is V_0 rounded to bf16, i.e. V_0
    np.testing.assert_array_equal(o[:, :, 0], v0)
    np.testing.assert_allclose(lse[:, :, 0], case.scale * np.sum(q0 * k0, -1), atol=TOL_LSE, rtol=0)


@pytest.mark.parametrize("dtype,d", [(fi.F16, 64), (fi.BF16, 128), (fi.F16, 128), (fi.BF16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_sharp_softmax(dtype, d, causal):
    """Logits sqrt(d) times wider than at the default scale (scale = 1 on
    N(0,1) Q and K): rows are dominated by a few keys, the running reference
    value moves in many 32-key units and P covers the whole exponent range
    down to underflow. V is drawn at a quarter of unit spread so that |O|
    stays below 1, the magnitude the output tolerances were set for."""
    N = 1000
    rng = np.random.default_rng(50 + 2 * d + dtype)
    q = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    k = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    v = rng.standard_normal((1, 2, N, d), dtype=np.float32) * np.float32(0.25)
    check(fi.from_exact(q, k, v, dtype, causal, scale=1.0), label="sharp")


@pytest.mark.parametrize("scale", [1e-3, 4.0])
@pytest.mark.parametrize("dtype,d", [(fi.BF16, 128), (fi.F16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_extreme_scales(scale, dtype, d, causal):
    """Logit multipliers far from 1/sqrt(d) on N(0,1) inputs: 1e-3 makes every
    row nearly uniform (P close to 1 for every key, row sums up to N), 4.0
    makes the logits' spread about 45 (each row dominated by one key, the
    reference value moving often, almost every other P underflowing to 0).
    V at a quarter of unit spread keeps |O| below 1, where the tolerances
    were set."""
    N = 700
    rng = np.random.default_rng(70 + d + int(scale > 1) + 2 * causal)
    q = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    k = rng.standard_normal((1, 2, N, d), dtype=np.float32)
    v = rng.standard_normal((1, 2, N, d), dtype=np.float32) * np.float32(0.25)
    check(fi.from_exact(q, k, v, dtype, causal, scale=scale), label=f"scale {scale}")


@pytest.mark.parametrize("slope", [0.22, -0.22])
@pytest.mark.parametrize("dtype,d", [(fi.BF16, 128), (fi.F16, 64)])
@pytest.mark.parametrize("causal", [False, True])
def test_drifting_scores(slope, dtype, d, causal):
    """Scores that rise (slope > 0) or fall along the keys by about ten
    base-2 units per 32-key unit. Rising: every unit of every row holds a new
    maximum, so the reference value moves in every unit (the rescale path
    on every step). Falling: the first unit holds the maximum and the later
    probabilities underflow to zero. Q = u + noise, K_j = slope*j*u + noise
    for a unit vector u, so q_i . k_j ~ slope * j; scale = 1."""
    N = 700
    rng = np.random.default_rng(60 + d + (slope > 0))
    u = np.full(d, 1.0 / np.sqrt(d), np.float32)
    q = np.float32(0.3) * rng.standard_normal((1, 2, N, d), dtype=np.float32) + u
    k = (np.float32(0.3) * rng.standard_normal((1, 2, N, d), dtype=np.float32)
         + (np.float32(slope) * np.arange(N, dtype=np.float32))[:, None] * u)
    v = rng.standard_normal((1, 2, N, d), dtype=np.float32) * np.float32(0.25)
    check(fi.from_exact(q, k, v, dtype, causal, scale=1.0), label=f"drift {slope:+}")


def _round_to(a, dtype):
    """Round real values to f16 or bf16 (RNE) and back to float64."""
    a32 = np.asarray(a, dtype=np.float32)
    if dtype == fi.F16:
        return a32.astype(np.float16).astype(np.float64)
    return fi.bf16_bits_to_f32(fi.f32_to_bf16_bits(a32)).astype(np.float64)


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
def test_outlier_rmse(dtype):
    """The accuracy experiment of the FA3 walkthrough's numerical-error
    section, for 16-bit inputs: Q, K, V drawn from N(0,1) + N(0,100) *
    Bernoulli(0.001), RMSE of O against fp64 attention of the same rounded
    inputs. The page reports 1.9e-4 for fp16 FlashAttention (it gives no
    shape), 1.7x below a standard implementation that keeps its intermediate
    results in fp16. Here, at B=1 H=4 N=2048 d=128:

    - the RMSE is at most 1.25x that of a CPU model of this kernel's rounding
      (P rounded to the input type before P.V, the row sum over the unrounded
      P, O rounded once; everything else exact). The kernel's reference value
      may lag a row's maximum by up to a factor 256 (it moves only when a
      unit's row sum passes 256), so its largest P is rounded too, where
      with the exact maximum it is 1; the model therefore scales each row's
      P by a seeded factor drawn log-uniformly from [1, 256) before rounding.
      With the exact maximum instead, the model's RMSE is 1.5x lower. For f16
      the RMSE is also at most the page's 1.9e-4;
    - it is below the RMSE of a model of the standard implementation, which
      stores the scores and the normalised probabilities in the input type.
    """
    import oracle
    case = fi.make_case(1, 4, 2048, 128, dtype, False, seed=760, dist="outlier")
    say(f"[gpu] outlier RMSE B=1 H=4 N=2048 d=128 dtype={fi.DTYPE_NAMES[dtype]} seed=760")
    o, lse = run_gpu(case)
    q, k, v = case.exact("q"), case.exact("k"), case.exact("v")
    se = se_fa = se_std = 0.0
    worst_l = 0.0
    lag = np.exp2(np.random.default_rng(761).uniform(0.0, 8.0, size=(case.H, case.N, 1)))
    for h in range(case.H):
        ro, rl = oracle.attention_rows(q[0, h], k[0, h], v[0, h], np.arange(case.N), case.scale,
                                       False)
        se += float(np.sum((o[0, h] - ro) ** 2))
        worst_l = max(worst_l, float(np.max(np.abs(lse[0, h] - rl))))
        s = case.scale * (q[0, h] @ k[0, h].T)
        p = np.exp(s - s.max(axis=1, keepdims=True)) * lag[h]
        fa_model = _round_to((_round_to(p, dtype) @ v[0, h]) / p.sum(axis=1, keepdims=True), dtype)
        se_fa += float(np.sum((fa_model - ro) ** 2))
        s16 = _round_to(s, dtype)
        p16 = np.exp(s16 - s16.max(axis=1, keepdims=True))
        std_model = _round_to(_round_to(p16 / p16.sum(axis=1, keepdims=True), dtype) @ v[0, h], dtype)
        se_std += float(np.sum((std_model - ro) ** 2))
    n = o.size
    rmse, rmse_fa, rmse_std = ((x / n) ** 0.5 for x in (se, se_fa, se_std))
    say(f"      RMSE {rmse:.3e} (model of this kernel's rounding {rmse_fa:.3e}, of a standard "
        f"implementation with 16-bit intermediates {rmse_std:.3e}); max|dLSE|={worst_l:.3e}")
    assert rmse <= 1.25 * rmse_fa, f"RMSE {rmse} > 1.25 x model {rmse_fa}"
    assert rmse < rmse_std
    if dtype == fi.F16:
        assert rmse <= 1.9e-4
    assert worst_l <= TOL_LSE


def test_deterministic():
    import torch
    case = fi.make_case(2, 4, 1500, 128, fi.BF16, True, seed=13)
    t = to_device(case)
    say("[gpu] determinism")
    o1, l1 = run_gpu(case, tensors=t)
    o2, l2 = run_gpu(case, tensors=t)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)
    del t
    torch.cuda.empty_cache()


def test_non_default_stream():
    import torch
    import io_aware_softmax_fa_amd as fa
    case = fi.make_case(1, 2, 512, 64, fi.F16, False, seed=14)
    q, k, v = to_device(case)
    ref_o, ref_l = fa.forward(q, k, v, False, case.scale)
    s = torch.cuda.Stream()
    say("[gpu] side stream")
    with torch.cuda.stream(s):
        o, l = fa.forward(q, k, v, False, case.scale)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(o, ref_o) and torch.equal(l, ref_l)


def test_empty_problem():
    import torch
    import io_aware_softmax_fa_amd as fa
    q = torch.empty((2, 3, 0, 64), dtype=torch.float16, device="cuda")
    o, lse = fa.forward(q, q.clone(), q.clone())
    torch.cuda.synchronize()
    assert o.shape == (2, 3, 0, 64) and lse.shape == (2, 3, 0)


def test_binding_rejects_bad_tensors():
    import torch
    import io_aware_softmax_fa_amd as fa
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(ValueError):
        fa.forward(q, q.transpose(2, 3), q)
    with pytest.raises(TypeError):
        fa.forward(q.float(), q.float(), q.float())
    with pytest.raises(fa.FaError) as e:
        z = torch.zeros((1, 1, 64, 96), dtype=torch.float16, device="cuda")
        fa.forward(z, z, z)
    assert e.value.code == fa.FA_ERR_UNSUPPORTED


# ------------------------------------------------------------------- fp8 --

def test_b4_h16_n8192_d128_fp8():
    """e4m3 Q/K/V with per-tensor scales amax/448, P quantised to e4m3; every
    row of all 64 heads against the 6e-2 gate."""
    check(fi.make_case(4, 16, 8192, 128, fi.FP8_E4M3, False, seed=5), label="fp8 n8192")


@pytest.mark.parametrize("N", [1, 63, 64, 65, 199, 200, 201, 255, 257, 700, 1025])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_fp8_ragged_lengths(N, d, causal):
    # Short and causal rows are dominated by a few keys, where e4m3 rounding of P
    # alone can pass 6e-2 (that gate is stated for the N=8192 workload above);
    # these cases are held to the bound derived from the e4m3 arithmetic.
    # N = 199..201 and 255: the tile count is a multiple of the 4-tile loop and a
    # wave straddles N, which once exposed the last GEMM1 running with idle lanes
    check(fi.make_case(2, 2, N, d, fi.FP8_E4M3, causal, seed=2000 + N), label="fp8 ragged",
          fp8_derived=True)


@pytest.mark.parametrize("B,H,N,d", [(2, 8, 1000, 128), (4, 4, 700, 64), (1, 16, 2048, 128)])
def test_fp8_causal_head_bundles(B, H, N, d):
    """fp8 causal launches whose heads split over the 8 XCDs take the head
    bundles (tiles interleaved longest first across an XCD's bundle, the last
    bundle possibly short); held to the e4m3-derived bound."""
    check(fi.make_case(B, H, N, d, fi.FP8_E4M3, True, seed=2100 + N + d), label="fp8 bundles",
          fp8_derived=True)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_zero_query_closed_form(causal):
    """q codes all zero: LSE_i = ln(#visible keys), O_i = mean of visible V rows."""
    N, d = 600, 128
    case = fi.make_case(1, 2, N, d, fi.FP8_E4M3, causal, seed=21)
    case.q = np.zeros_like(case.q)
    say(f"[gpu] fp8 Q=0 closed form causal={causal}")
    o, lse = run_gpu(case)
    cnt = np.arange(1, N + 1) if causal else np.full(N, N)
    np.testing.assert_allclose(lse[0, 1], np.log(cnt), atol=TOL_LSE, rtol=0)
    vx = case.exact("v")[0, 1]
    want = np.cumsum(vx, axis=0) / cnt[:, None] if causal else np.tile(vx.mean(0), (N, 1))
    assert np.max(np.abs(o[0, 1] - want)) <= TOL_O[fi.FP8_E4M3]


def test_fp8_deterministic():
    case = fi.make_case(1, 4, 1000, 128, fi.FP8_E4M3, True, seed=22)
    t = to_device(case)
    say("[gpu] fp8 determinism")
    o1, l1 = run_gpu(case, tensors=t)
    o2, l2 = run_gpu(case, tensors=t)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


@pytest.mark.parametrize("causal", [False, True])
def test_many_heads_short_sequences(causal):
    """2048 (batch, head) pairs of 33 rows: one ragged tile per head, a grid
    of 2048 workgroups spread over the XCDs by the head-grouped order."""
    check(fi.make_case(64, 32, 33, 128, fi.BF16, causal, seed=90), rows_per_head=8,
          label="many heads")


@pytest.mark.parametrize("B,H", [(1, 3), (3, 5)])
def test_head_counts_not_a_multiple_of_eight(B, H):
    """Heads that do not split evenly over the 8 XCDs take the other branch of
    the tile order (causal: all heads' tiles longest first)."""
    for causal in (False, True):
        check(fi.make_case(B, H, 700, 64, fi.F16, causal, seed=91 + H), label="odd heads")


@pytest.mark.parametrize("B,H,N,causal", [(1, 3, 700, False), (3, 5, 1000, False),
                                          (1, 3, 8292, True), (2, 8, 8192, True),
                                          (1, 2, 8191, True), (1, 2, 16383, True)])
def test_wide_tiles(B, H, N, causal):
    """The 256-row tiles (eight waves) of the plain d = 128 forward: head
    counts that do not split over the 8 XCDs, ragged last tiles, causal
    problems at and just above the length from which they are used (where
    waves past their diagonal also stop computing early), and one just below
    it (128-row tiles)."""
    rows = None if N < 4096 else 256
    check(fi.make_case(B, H, N, 128, fi.BF16, causal, seed=95 + N), rows_per_head=rows,
          label="wide tiles")


@pytest.mark.parametrize("B,H,N,dtype", [(1, 3, 700, fi.F16), (3, 5, 1000, fi.BF16),
                                         (2, 4, 257, fi.F16), (1, 1, 4100, fi.BF16)])
def test_wide_tiles_d64(B, H, N, dtype):
    """The 256-row tiles of the plain d = 64 forward without a mask (two
    workgroups of eight waves per CU): head counts that do not split over the
    8 XCDs and ragged last tiles, one of them a single row past a tile."""
    rows = None if N < 4096 else 256
    check(fi.make_case(B, H, N, 64, dtype, False, seed=131 + N), rows_per_head=rows,
          label="wide tiles d64")


@pytest.mark.parametrize("B,H,N,d,dtype", [(5, 8, 4096, 128, fi.BF16), (2, 8, 2000, 64, fi.F16),
                                           (3, 16, 1100, 128, fi.BF16)])
def test_causal_head_bundles(B, H, N, d, dtype):
    """Causal launches whose heads split over the 8 XCDs run each XCD's
    heads in bundles, tiles interleaved longest first: a short last bundle
    (5 heads per XCD in bundles of 4), a ragged N, and bundles of all of an
    XCD's heads. (The B=2 H=32 N=8192 causal workload runs bundles of 4 over
    256-row tiles.)"""
    rows = None if N <= 2048 else 64
    check(fi.make_case(B, H, N, d, dtype, True, seed=97 + N), rows_per_head=rows,
          label="head bundles")
