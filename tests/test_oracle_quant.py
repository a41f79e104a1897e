"""Pins of the FP8 quantisation oracle (e4m3 rounding, block scales, the
random-sign Hadamard transform) to independent implementations and closed
forms."""
import numpy as np
import pytest
import scipy.linalg
import torch

import fa_inputs as fi
from oracle import quant as Q


def test_code_table_matches_torch_float8():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = Q.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    np.testing.assert_array_equal(np.isnan(ours), nan)
    np.testing.assert_array_equal(ours[~nan], ref[~nan])
    assert Q.e4m3_value(0x7E) == 448.0 and Q.e4m3_value(0x01) == 2.0 ** -9


def _grid_points():
    """Every finite e4m3 value, every midpoint between neighbours, points just
    either side of each midpoint, and random values, all within +-448."""
    v = np.unique(np.abs(Q.e4m3_decode(np.arange(0x7F))))
    mids = (v[:-1] + v[1:]) / 2
    eps = np.float32(1e-6)
    pts = np.concatenate([v, mids, mids * (1 + eps), mids * (1 - eps),
                          np.random.default_rng(9).uniform(0, 448, 2000)])
    pts = pts.astype(np.float32)
    return np.concatenate([pts, -pts])


def test_rounding_matches_torch_within_range():
    x = _grid_points()
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(Q.e4m3_encode(x), ref)


def test_rounding_matches_the_input_encoder():
    """The input generator's encoder (a separate implementation: nearest of
    the sorted code values) agrees everywhere, saturation included."""
    x = np.concatenate([_grid_points(), np.float32([449, 464, 480, 1e6, -1e6, -500])])
    np.testing.assert_array_equal(Q.e4m3_encode(x), fi.e4m3_encode(x))


def test_saturation_and_ties():
    assert list(Q.e4m3_round([449.0, 464.0, 1e30, -1e30])) == [448, 448, 448, -448]
    # ties go to the even mantissa: 1 + 1/16 -> 1, 1 + 3/16 -> 1.25, 232 -> 224
    assert list(Q.e4m3_round([1.0625, 1.1875, 232.0])) == [1.0, 1.25, 224.0]
    # below half the smallest subnormal: 0; exactly half: tie to even (0)
    assert list(Q.e4m3_round([2.0 ** -11, 2.0 ** -10, 2.0 ** -10 * 1.001])) == [0, 0, 2.0 ** -9]


@pytest.mark.parametrize("d", [1, 2, 8, 64, 128])
def test_hadamard_is_sylvester_and_orthogonal(d):
    h = Q.hadamard(d)
    np.testing.assert_array_equal(h, scipy.linalg.hadamard(d))
    np.testing.assert_array_equal(h @ h.T, d * np.eye(d))


def test_incoherent_transform_keeps_scores_and_spreads_outliers():
    rng = np.random.default_rng(10)
    d = 128
    signs = rng.choice([-1.0, 1.0], d)
    q, k = rng.standard_normal((9, d)), rng.standard_normal((7, d))
    np.testing.assert_allclose(Q.incoherent(q, signs) @ Q.incoherent(k, signs).T, q @ k.T,
                               atol=1e-12)
    # one outlier of 100 in dim 5: every transformed dim gets magnitude 100/sqrt(d)
    x = np.zeros(d)
    x[5] = 100.0
    np.testing.assert_allclose(np.abs(Q.incoherent(x, signs)), 100 / np.sqrt(d), atol=1e-12)
    # a different sign vector is a different transform
    assert not np.allclose(Q.incoherent(q, signs), Q.incoherent(q, -signs))


def test_block_quantize_closed_forms():
    rng = np.random.default_rng(11)
    x = fi.bf16_bits_to_f32(fi.f32_to_bf16_bits(rng.standard_normal(2 * 200 * 16).astype(
        np.float32))).reshape(2, 200, 16)
    x[1, 70, 3] = 300.0                       # an outlier in block 1 of head 1
    codes, s = Q.block_quantize_f32(x, 64)
    assert s.shape == (2, 4)
    for h in range(2):
        for i in range(4):
            blk = x[h, 64 * i:64 * (i + 1)]
            amax = np.max(np.abs(blk))
            assert s[h, i] == np.float32(np.float32(amax) / np.float32(448))
            # the largest element of a block encodes as +-448
            j = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert abs(Q.e4m3_value(int(codes[h, 64 * i + j[0], j[1]]))) == 448.0
    deq = Q.dequantize_blocks(codes, s, 64)
    # error within half a code step (relative 2^-4, or 2^-10 * s for subnormals)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * np.repeat(s, 64, axis=-1)[:, :200, None])
    assert np.all(np.abs(deq - x) <= bound * (1 + 1e-6))
    # the outlier coarsens only its own block
    c2, s2 = Q.block_quantize_f32(np.where(np.arange(200)[None, :, None] == 70, 0.0, x), 64)
    np.testing.assert_array_equal(s2[:, [0, 2, 3]], s[:, [0, 2, 3]])
    assert s2[1, 1] < s[1, 1] / 10
    # one block spanning the whole tensor is per-tensor quantisation
    c1, s1 = Q.block_quantize_f32(x[1:], 256)
    pc, ps = fi.quantize_e4m3_per_tensor(x[1])
    assert s1[0, 0] == ps
    np.testing.assert_array_equal(c1[0], pc)
