"""GPU parity of fa_fwd_kv (grouped query heads over a key/value history,
optionally split over key ranges) against the fp64 grouped-query oracle.

Tolerances as for fa_fwd: max|dO| <= 4e-3 (f16) / 1.6e-2 (bf16), |dLSE| <=
1e-3. Cases cover multi-head (Hkv = H), grouped and multi-query heads, single-
and multi-token decode against long histories, chunked prefill (Nq < Nk,
causal), ragged lengths, and 1..16 key splits including splits that fall
wholly past the causal diagonal.
"""
import numpy as np
import pytest

import fa_inputs as fi
import oracle
from tests.gpu_util import TOL_LSE, TOL_O, say

pytestmark = pytest.mark.gpu


def run_kv(case, splits):
    import torch
    import io_aware_softmax_fa_amd as fa
    tdt = torch.float16 if case.dtype == fi.F16 else torch.bfloat16
    q, k, v = (torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()
               for a in (case.q, case.k, case.v))
    o = torch.full_like(q, float("nan"))
    lse = torch.full((case.B, case.H, case.Nq), float("nan"), device="cuda")
    fa.forward_kv(q, k, v, case.causal, case.scale, num_splits=splits, out=o, lse=lse)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_kv(case, splits, label=""):
    say(f"[gpu-kv] {label} B={case.B} H={case.H} Hkv={case.Hkv} Nq={case.Nq} Nk={case.Nk} "
        f"d={case.d} dtype={fi.DTYPE_NAMES[case.dtype]} causal={case.causal} splits={splits} "
        f"seed={case.seed}")
    o, lse = run_kv(case, splits)
    ro, rl = oracle.attention_gqa(case.exact("q"), case.exact("k"), case.exact("v"), case.scale,
                                  case.causal)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "non-finite output"
    do, dl = float(np.max(np.abs(o - ro))), float(np.max(np.abs(lse - rl)))
    say(f"      max|dO|={do:.3e} max|dLSE|={dl:.3e}")
    assert do <= TOL_O[case.dtype] and dl <= TOL_LSE


@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("causal", [False, True])
def test_mha_equals_fa_fwd_shape(splits, causal):
    check_kv(fi.make_kv_case(1, 4, 4, 300, 300, 128, fi.BF16, causal, seed=501), splits, "mha")


@pytest.mark.parametrize("H,Hkv", [(8, 2), (8, 1), (32, 8)])
@pytest.mark.parametrize("causal", [False, True])
def test_grouped_prefill(H, Hkv, causal):
    check_kv(fi.make_kv_case(2, H, Hkv, 200, 520, 64, fi.F16, causal, seed=502), 1, "gqa")


@pytest.mark.parametrize("Nq", [1, 4, 16])
@pytest.mark.parametrize("splits", [1, 2, 8, 16])
@pytest.mark.parametrize("causal", [False, True])
def test_decode(Nq, splits, causal):
    check_kv(fi.make_kv_case(2, 16, 4, Nq, 4000, 128, fi.BF16, causal, seed=503 + Nq), splits,
             "decode")


@pytest.mark.parametrize("Nk", [1, 63, 65, 777])
def test_ragged_history(Nk):
    check_kv(fi.make_kv_case(1, 6, 3, 1, Nk, 64, fi.F16, True, seed=510 + Nk), 4, "ragged")


def test_chunked_prefill_splits_past_diagonal():
    """Nq = 256 of Nk = 1024, causal, 8 key ranges of 128: the first query tile's
    last ranges lie wholly past its diagonal and must merge as empty."""
    check_kv(fi.make_kv_case(1, 4, 4, 256, 1024, 128, fi.BF16, True, seed=520), 8, "chunk")


@pytest.mark.parametrize("B,H,Hkv,Nq,Nk", [(1, 8, 2, 700, 700), (2, 6, 3, 513, 1000),
                                             (1, 4, 1, 300, 300)])
def test_wide_tiles_grouped(B, H, Hkv, Nq, Nk):
    """Non-causal grouped-query attention in one key range with at least 1024
    rows per K/V head runs on 256-row tiles (eight waves): ragged last
    tiles, queries shorter than the history, and multi-query heads."""
    check_kv(fi.make_kv_case(B, H, Hkv, Nq, Nk, 128, fi.BF16, False, seed=550 + Nq), 1, "wide")


@pytest.mark.parametrize("slope", [0.1, -0.1])
@pytest.mark.parametrize("splits", [1, 8])
def test_decode_drifting_scores(slope, splits):
    """Scores that rise (or fall) steadily along a 3000-key history, scale 1:
    the key ranges' partial LSEs then differ by up to a few hundred, so the
    merge weights of all but one range underflow, and inside each range the
    reference value moves in every unit (rising) or P underflows (falling).
    Q = u + noise, K_j = slope*j*u + noise for a unit vector u."""
    B, H, Hkv, Nq, Nk, d = 1, 8, 2, 4, 3000, 128
    rng = np.random.default_rng(540 + (slope > 0) + 2 * splits)
    u = np.full(d, 1.0 / np.sqrt(d), np.float32)
    q = np.float32(0.3) * rng.standard_normal((B, H, Nq, d), dtype=np.float32) + u
    k = (np.float32(0.3) * rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
         + (np.float32(slope) * np.arange(Nk, dtype=np.float32))[:, None] * u)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32) * np.float32(0.25)
    case = fi.KvCase(B, H, Hkv, Nq, Nk, d, fi.BF16, True, 1.0, -1)
    case.q, case.k, case.v = (fi.f32_to_bf16_bits(a) for a in (q, k, v))
    check_kv(case, splits, f"drift {slope:+}")


def test_b8_h32_hkv8_decode_32k_bf16():
    """A long-history decode step: B=8, H=32 over Hkv=8, one query, Nk=32768,
    with the split count the binding picks."""
    case = fi.make_kv_case(8, 32, 8, 1, 32768, 128, fi.BF16, True, seed=530)
    import io_aware_softmax_fa_amd as fa
    check_kv(case, fa.default_splits(8, 32, 8, 1, 32768), "decode32k")


def test_mqa_decode_one_kv_head():
    """Multi-query attention: 64 query heads over one K/V head, one query,
    a 5000-key history, the binding's split count."""
    import io_aware_softmax_fa_amd as fa
    case = fi.make_kv_case(2, 64, 1, 1, 5000, 128, fi.BF16, True, seed=540)
    check_kv(case, fa.default_splits(2, 64, 1, 1, 5000), "mqa")


def test_splits_beyond_key_tiles():
    """More key ranges than 64-key tiles: most ranges are empty and must
    merge as such."""
    check_kv(fi.make_kv_case(1, 4, 2, 3, 100, 64, fi.F16, True, seed=541), 16, "many-splits")


_N1M = {}


@pytest.mark.parametrize("splits", [None, 1])
def test_decode_over_a_million_keys(splits):
    """The longest history tested: one query per head over Nk = 2^20 keys
    (causal, grouped 8 over 2 K/V heads, d = 128, bf16; 64-bit element
    offsets past 2^31 in K and V), with the binding's default split count
    (256 key ranges of 4096 keys, merged) and with one range that streams the
    whole history. Drawing the inputs takes most of the test's time."""
    if "case" not in _N1M:
        say("[gpu-kv] Nk=2^20 decode: drawing inputs")
        _N1M["case"] = fi.make_kv_case(1, 8, 2, 1, 1 << 20, 128, fi.BF16, True, seed=530)
    check_kv(_N1M["case"], splits, "n1m")
