"""Host encoders and the seeded generator (no GPU)."""
import numpy as np
import pytest
import torch

import fa_inputs as fi


def _probe_values():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * 7,
        rng.standard_normal(20000).astype(np.float32) * 1e-3,
        np.array([0.0, -0.0, 1.0, -1.0, 65504.0, 3.0e38, 1e-40], dtype=np.float32),
    ])
    return x


def test_bf16_rne_matches_torch():
    x = _probe_values()
    # every bf16 midpoint in [1, 2): ties must go to even
    mids = (np.arange(0x3F80, 0x4000, dtype=np.uint32) << 16) + 0x8000
    x = np.concatenate([x, mids.view(np.float32)])
    ours = fi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    back = fi.bf16_bits_to_f32(ours)
    np.testing.assert_array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_f16_rne_matches_torch():
    x = _probe_values()
    np.testing.assert_array_equal(
        fi.f32_to_f16(x).view(np.uint16),
        torch.from_numpy(x).to(torch.float16).view(torch.int16).numpy().view(np.uint16))


def test_e4m3_decode_table():
    t = fi.E4M3_VALUES
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert t[0x01] == 2.0 ** -9 and t[0x08] == 2.0 ** -6 and t[0x38] == 1.0
    # every finite code decodes to what torch's float8_e4m3fn holds
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy()
    finite = ~np.isnan(t)
    np.testing.assert_array_equal(t[finite].astype(np.float32), ref[finite])


def test_e4m3_encode_roundtrip_and_midpoints():
    t = fi.E4M3_VALUES
    finite = [c for c in range(256) if not np.isnan(t[c])]
    np.testing.assert_array_equal(fi.e4m3_encode(t[finite]), np.array(finite, dtype=np.uint8))
    pos = t[:0x7F]
    mids = (pos[:-1] + pos[1:]) / 2
    got = fi.e4m3_encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)      # ties to the even code
    np.testing.assert_array_equal(got, want.astype(np.uint8))
    assert fi.e4m3_encode(np.array([1e6]))[0] == 0x7E       # saturates
    assert fi.e4m3_encode(np.array([-1e6]))[0] == 0xFE


def test_e4m3_encode_matches_torch_in_range():
    x = _probe_values()
    x = x[np.abs(x) <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(fi.e4m3_encode(x), ref)


def test_per_tensor_scale():
    x = np.random.default_rng(1).standard_normal(10000).astype(np.float32)
    c, s = fi.quantize_e4m3_per_tensor(x)
    assert s == np.float32(np.abs(x).max() / np.float32(448))
    deq = fi.e4m3_decode(c) * s
    assert np.max(np.abs(deq - x)) <= np.abs(x).max() * 2.0 ** -4


def test_make_case_is_seeded_and_ordered():
    a = fi.make_case(1, 2, 64, 64, fi.BF16, seed=5)
    b = fi.make_case(1, 2, 64, 64, fi.BF16, seed=5)
    np.testing.assert_array_equal(a.q, b.q)
    rng = np.random.default_rng(5)
    q = rng.standard_normal(1 * 2 * 64 * 64, dtype=np.float32)
    k = rng.standard_normal(1 * 2 * 64 * 64, dtype=np.float32)
    np.testing.assert_array_equal(a.k.ravel(), fi.f32_to_bf16_bits(k))
    np.testing.assert_array_equal(a.exact("q").ravel(),
                                  fi.bf16_bits_to_f32(fi.f32_to_bf16_bits(q)).astype(np.float64))
    assert a.scale == np.float32(0.125)


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16, fi.FP8_E4M3])
def test_exact_values_are_representable(dtype):
    c = fi.make_case(1, 1, 32, 64, dtype, seed=2)
    x = c.exact("v")
    assert x.shape == (1, 1, 32, 64) and np.all(np.isfinite(x))
    if dtype == fi.FP8_E4M3:
        assert np.max(np.abs(x)) <= 448 * c.descale[2] * (1 + 1e-6)


def test_sample_rows():
    r = fi.sample_rows(41, 0, 3, 32768)
    assert len(r) == 256 and len(set(r.tolist())) == 256
    for must in (0, 1, 32767, 255, 256, 511, 512):
        assert must in r
    np.testing.assert_array_equal(r, fi.sample_rows(41, 0, 3, 32768))
    assert not np.array_equal(r, fi.sample_rows(41, 0, 4, 32768))
    np.testing.assert_array_equal(fi.sample_rows(1, 0, 0, 100), np.arange(100))
