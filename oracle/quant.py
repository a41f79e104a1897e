"""fp64 CPU oracle for the FP8 accuracy variants: e4m3 rounding, per-block
quantisation and the incoherent (random-sign Hadamard) transform.

TEST INFRASTRUCTURE ONLY (see the package docstring). Only ``tests/``, the
smoke check and the benchmark's CPU-baseline leg may use it.

Sources ("FlashAttention 完全拆解（三）" FP8 section, "FlashAttention 深度解析"
accuracy passages, and "FlashAttention · InkStack" 3.3.1-3.3.3):

* Scaling: an fp16/bf16 block X is stored as e4m3 codes of X / s with
  s = amax(|X|) / 448, 448 being the largest finite e4m3 value; the value a
  code stands for is code * s.
* Block quantisation: every block of rows (the query tile Q_i, the key and
  value tiles K_j, V_j) has its own s, so an outlier only coarsens its block.
* Incoherent processing: before quantising, Q and K of a head are multiplied
  by the same orthogonal M = diag(signs) * H_d / sqrt(d), with H_d the
  Sylvester-Hadamard matrix and random signs +-1; Q M (K M)^T = Q K^T, so the
  scores are unchanged while an outlier's energy spreads over all d dims.

OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; exponent field 0
holds the subnormals m/8 * 2^-6; 0x7F and 0xFF are NaN; there is no infinity.
Encoding rounds to nearest, ties to even mantissa, and saturates at +-448.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_value(code: int) -> float:
    """The real number an e4m3fn code stands for (NaN for 0x7F, 0xFF)."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field, mant = (code >> 3) & 0xF, code & 0x7
    if exp_field == 0xF and mant == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * mant * 2.0 ** -9            # (m / 8) * 2^-6
    return sign * (8 + mant) * 2.0 ** (exp_field - 10)   # (1 + m/8) * 2^(e-7)


_VALUE_OF = np.array([e4m3_value(c) for c in range(256)])
_CODE_OF = {v: c for c, v in enumerate(_VALUE_OF[:0x7F])}   # non-negative values -> code


def e4m3_round(x) -> np.ndarray:
    """Round reals to the nearest e4m3 value (ties to even mantissa), with
    saturation at +-448: the grid spacing at magnitude a is 2^(e-3) with
    e = max(floor(log2 a), -6), and rounding to that grid with ties to even
    multiples is np.rint on the exactly scaled value."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    step = np.exp2(e - 3.0)
    r = np.rint(a / step) * step                   # a / step is exact (power of two)
    r = np.minimum(r, E4M3_MAX)
    return np.copysign(r, x)


def e4m3_encode(x) -> np.ndarray:
    """Codes of ``e4m3_round(x)`` (sign bit set for negative inputs, so -0.0
    and negatives that round to 0 give 0x80)."""
    x = np.asarray(x, dtype=np.float64)
    r = np.abs(e4m3_round(x))
    codes = np.vectorize(lambda v: _CODE_OF[float(v)], otypes=[np.int64])(r) if r.size else \
        np.zeros(r.shape, dtype=np.int64)
    return (codes | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    return _VALUE_OF[np.asarray(codes, dtype=np.uint8)]


def hadamard(d: int) -> np.ndarray:
    """Sylvester construction: H_1 = [1], H_2n = [[H_n, H_n], [H_n, -H_n]]."""
    assert d >= 1 and d & (d - 1) == 0
    h = np.ones((1, 1))
    while h.shape[0] < d:
        h = np.block([[h, h], [h, -h]])
    return h


def incoherent(x, signs) -> np.ndarray:
    """x M with M = diag(signs) H_d / sqrt(d), over the last axis (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    m = np.asarray(signs, dtype=np.float64)[:, None] * hadamard(d) / np.sqrt(d)
    return x @ m


def block_scales(x, block_rows: int) -> np.ndarray:
    """s = amax / 448 per block of ``block_rows`` rows of each [.., N, d] matrix
    (the last block may be short), in fp64; a block of zeros gets s = 1."""
    x = np.asarray(x, dtype=np.float64)
    N = x.shape[-2]
    nb = -(-N // block_rows)
    out = np.empty(x.shape[:-2] + (nb,))
    for i in range(nb):
        amax = np.max(np.abs(x[..., i * block_rows:(i + 1) * block_rows, :]), axis=(-2, -1))
        out[..., i] = np.where(amax > 0, amax / E4M3_MAX, 1.0)
    return out


def block_quantize_f32(x, block_rows: int):
    """Block quantisation with the scale and the ratio formed in float32, the
    precision the GPU quantiser works in: s = fl32(amax / 448), code =
    e4m3(fl32(x / s)). For inputs exactly representable in float32 (fp16,
    bf16 values) both divisions are single correctly rounded float32
    operations, so the codes are fixed exactly. Returns (codes, scales)."""
    x = np.asarray(x, dtype=np.float32)
    N = x.shape[-2]
    nb = -(-N // block_rows)
    scales = np.empty(x.shape[:-2] + (nb,), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    for i in range(nb):
        blk = x[..., i * block_rows:(i + 1) * block_rows, :]
        amax = np.max(np.abs(blk), axis=(-2, -1))
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[..., i] = s
        ratio = (blk / s[..., None, None]).astype(np.float32)
        codes[..., i * block_rows:(i + 1) * block_rows, :] = e4m3_encode(ratio)
    return codes, scales


def dequantize_blocks(codes, scales, block_rows: int) -> np.ndarray:
    """code value * its block's scale, in fp64."""
    v = e4m3_decode(codes)
    s = np.repeat(np.asarray(scales, dtype=np.float64), block_rows, axis=-1)[..., :v.shape[-2]]
    return v * s[..., None]
