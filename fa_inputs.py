"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the tests, the benchmark and the oracle side of the
checks. It draws the random Q/K/V values and encodes them into the storage
formats the GPU path consumes (fp16, bf16, OCP e4m3fn with a per-tensor
scale). It holds none of the attention arithmetic.

Recipe (every caller uses exactly this):

* values: ``numpy.random.default_rng(seed).standard_normal(B*H*N*d,
  dtype=float32)``, drawn in the order Q, K, V, C-order ``[B][H][N][d]``;
* fp16 / bf16: round-to-nearest-even from the float32 draws;
* fp8: per-tensor scale ``s = amax(|x|) / 448`` in float32, codes
  ``e4m3fn(x / s)`` rounded to nearest even, saturating at 448 (the per-tensor
  scaling of FlashAttention · InkStack, section 3.3.3, "Scaling").

The exact values a kernel sees are recovered with ``decode_*`` and are what the
oracle is fed, upcast to float64.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

E4M3_MAX = 448.0

# dtype codes of the C ABI (include/fa.h)
F16, BF16, FP8_E4M3 = 0, 1, 2
DTYPE_NAMES = {F16: "f16", BF16: "bf16", FP8_E4M3: "fp8_e4m3"}


# ---------------------------------------------------------------- encoders --

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round to nearest, ties to even."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    """float32 -> float16, round to nearest even (numpy's cast)."""
    return np.asarray(x, dtype=np.float32).astype(np.float16)


def _e4m3_table() -> np.ndarray:
    """Value of every e4m3fn code 0..255 (NaN for 0x7F and 0xFF)."""
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = math.nan
        elif e == 0:
            vals[code] = sign * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()
_E4M3_POS = E4M3_VALUES[:0x7F]  # codes 0x00..0x7E: 0 .. 448, increasing


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)].astype(np.float32)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """float -> e4m3fn codes: round to nearest, ties to even code, saturate to
    +-448, NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")  # first value >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _E4M3_POS[lo]
    dhi = _E4M3_POS[hi] - a
    take_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(take_hi, hi, lo).astype(np.uint8)
    code = np.where(a == _E4M3_POS[hi], hi, code).astype(np.uint8)
    neg = np.signbit(x)
    code = code | (neg.astype(np.uint8) << 7)
    code = np.where(np.isnan(x), np.uint8(0x7F), code)
    return code.astype(np.uint8)


def quantize_e4m3_per_tensor(x: np.ndarray) -> tuple[np.ndarray, np.float32]:
    """Per-tensor e4m3 quantisation: s = amax/448 (float32), codes = e4m3(x/s)."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
    s = np.float32(amax / np.float32(E4M3_MAX)) if amax > 0 else np.float32(1.0)
    return e4m3_encode((x / s).astype(np.float32)), s


# --------------------------------------------------------------- the cases --

@dataclass
class Case:
    """One seeded attention problem, in device storage format and as the exact
    values that storage format holds (float64, for the oracle)."""
    B: int
    H: int
    N: int
    d: int
    dtype: int
    causal: bool
    scale: float
    seed: int
    # device-format host arrays: uint16 bits (f16/bf16) or uint8 codes (fp8)
    q: np.ndarray = field(repr=False, default=None)
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)
    descale: tuple = (1.0, 1.0, 1.0)

    def exact(self, which: str) -> np.ndarray:
        """The exact real values of q/k/v as float64, shape [B,H,N,d]."""
        a = getattr(self, which)
        if self.dtype == F16:
            x = a.view(np.float16).astype(np.float64)
        elif self.dtype == BF16:
            x = bf16_bits_to_f32(a).astype(np.float64)
        else:
            s = {"q": 0, "k": 1, "v": 2}[which]
            x = e4m3_decode(a).astype(np.float64) * np.float64(self.descale[s])
        return x.reshape(self.B, self.H, self.N, self.d)


def default_scale(d: int) -> float:
    """1/sqrt(d) as the float32 the kernels receive."""
    return float(np.float32(1.0 / math.sqrt(d)))


def make_case(B, H, N, d, dtype, causal=False, seed=0, scale=None,
              dist="normal") -> Case:
    """Draw Q, K, V (in that order) and encode them for ``dtype``.

    ``dist="normal"`` is iid N(0,1); ``dist="outlier"`` is
    N(0,1) + N(0,100)*Bernoulli(0.001), the outlier mix the FA3 walkthrough
    ("FlashAttention 完全拆解（三）", numerical-error section) uses for its RMSE
    table; the Bernoulli and the second normal are drawn after Q, K, V.
    """
    n = B * H * N * d
    rng = np.random.default_rng(seed)
    draws = [rng.standard_normal(n, dtype=np.float32) for _ in range(3)]
    if dist == "outlier":
        for i in range(3):
            mask = rng.random(n, dtype=np.float32) < np.float32(0.001)
            big = rng.standard_normal(n, dtype=np.float32) * np.float32(10.0)
            draws[i] = (draws[i] + np.where(mask, big, np.float32(0))).astype(np.float32)
    elif dist != "normal":
        raise ValueError(dist)
    case = Case(B, H, N, d, dtype, bool(causal),
                default_scale(d) if scale is None else float(scale), seed)
    enc = []
    descale = []
    for x in draws:
        if dtype == F16:
            enc.append(f32_to_f16(x).view(np.uint16))
            descale.append(1.0)
        elif dtype == BF16:
            enc.append(f32_to_bf16_bits(x))
            descale.append(1.0)
        elif dtype == FP8_E4M3:
            c, s = quantize_e4m3_per_tensor(x)
            enc.append(c)
            descale.append(float(s))
        else:
            raise ValueError(dtype)
    shape = (B, H, N, d)
    case.q, case.k, case.v = (e.reshape(shape) for e in enc)
    case.descale = tuple(descale)
    return case


def from_exact(q, k, v, dtype, causal=False, scale=None) -> Case:
    """A Case from given real arrays [B,H,N,d] (used by structured tests such as
    constant-V or Q=0). Values are encoded for ``dtype`` (fp16/bf16 only)."""
    q, k, v = (np.asarray(a, dtype=np.float32) for a in (q, k, v))
    B, H, N, d = q.shape
    case = Case(B, H, N, d, dtype, bool(causal),
                default_scale(d) if scale is None else float(scale), -1)
    if dtype == F16:
        case.q, case.k, case.v = (f32_to_f16(a).view(np.uint16) for a in (q, k, v))
    elif dtype == BF16:
        case.q, case.k, case.v = (f32_to_bf16_bits(a) for a in (q, k, v))
    else:
        raise ValueError("from_exact supports f16/bf16")
    return case


def sample_rows(seed: int, b: int, h: int, N: int, count: int = 256,
                tile: int = 256) -> np.ndarray:
    """Distinct query rows of one head to verify at long N: rows 0, 1, N-1,
    the rows either side of the first two tile boundaries, and the rest drawn
    uniformly from ``default_rng([seed, 7, b, h])``. Sorted."""
    if N <= count:
        return np.arange(N)
    must = {0, 1, N - 1}
    for t in (tile, 2 * tile):
        for r in (t - 1, t):
            if 0 <= r < N:
                must.add(r)
    rng = np.random.default_rng([seed, 7, b, h])
    rows = set(must)
    while len(rows) < count:
        rows.update(int(r) for r in rng.integers(0, N, size=count))
    rows = sorted(rows)
    keep = sorted(must) + [r for r in rows if r not in must]
    return np.array(sorted(keep[:count]), dtype=np.int64)


def make_dout(case: Case, seed: int):
    """An upstream gradient dO for ``case`` (f16/bf16 only): iid N(0,1) float32
    from ``default_rng([seed, 11])``, encoded like the case's inputs. Returns
    (device-format bits [B,H,N,d], exact float64 values)."""
    n = case.B * case.H * case.N * case.d
    x = np.random.default_rng([seed, 11]).standard_normal(n, dtype=np.float32)
    shape = (case.B, case.H, case.N, case.d)
    if case.dtype == F16:
        bits = f32_to_f16(x).view(np.uint16)
        exact = bits.view(np.float16).astype(np.float64)
    elif case.dtype == BF16:
        bits = f32_to_bf16_bits(x)
        exact = bf16_bits_to_f32(bits).astype(np.float64)
    else:
        raise ValueError("dO is drawn for f16/bf16 cases only")
    return bits.reshape(shape), exact.reshape(shape)


@dataclass
class KvCase:
    """A grouped-query problem over a key/value history: q [B,H,Nq,d] and
    k, v [B,Hkv,Nk,d] in device format, with their exact values."""
    B: int
    H: int
    Hkv: int
    Nq: int
    Nk: int
    d: int
    dtype: int
    causal: bool
    scale: float
    seed: int
    q: np.ndarray = field(repr=False, default=None)
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)

    def exact(self, which: str) -> np.ndarray:
        a = getattr(self, which)
        if self.dtype == F16:
            return a.view(np.float16).astype(np.float64)
        return bf16_bits_to_f32(a).astype(np.float64).reshape(a.shape)


def make_kv_case(B, H, Hkv, Nq, Nk, d, dtype, causal=False, seed=0, scale=None) -> KvCase:
    """Draw Q [B,H,Nq,d], then K and V [B,Hkv,Nk,d] (in that order), iid N(0,1)
    float32 from ``default_rng(seed)``, rounded to f16 or bf16."""
    rng = np.random.default_rng(seed)
    shapes = ((B, H, Nq, d), (B, Hkv, Nk, d), (B, Hkv, Nk, d))
    case = KvCase(B, H, Hkv, Nq, Nk, d, dtype, bool(causal),
                  default_scale(d) if scale is None else float(scale), seed)
    enc = []
    for shp in shapes:
        x = rng.standard_normal(int(np.prod(shp)), dtype=np.float32)
        if dtype == F16:
            enc.append(f32_to_f16(x).view(np.uint16).reshape(shp))
        elif dtype == BF16:
            enc.append(f32_to_bf16_bits(x).reshape(shp))
        else:
            raise ValueError("grouped cases are f16/bf16")
    case.q, case.k, case.v = enc
    return case


@dataclass
class VarlenCase:
    """B sequences of different lengths packed token-major: q [Tq,H,d] and
    k, v [Tk,Hkv,d] in device format, offsets cu_q, cu_k (B+1 int32)."""
    lens_q: tuple
    lens_k: tuple
    H: int
    Hkv: int
    d: int
    dtype: int
    causal: bool
    scale: float
    seed: int
    cu_q: np.ndarray = field(repr=False, default=None)
    cu_k: np.ndarray = field(repr=False, default=None)
    q: np.ndarray = field(repr=False, default=None)
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)

    def exact(self, which: str) -> np.ndarray:
        a = getattr(self, which)
        if self.dtype == F16:
            return a.view(np.float16).astype(np.float64)
        return bf16_bits_to_f32(a).astype(np.float64).reshape(a.shape)


def make_varlen_case(lens_q, lens_k, H, Hkv, d, dtype, causal=False, seed=0,
                     scale=None) -> VarlenCase:
    """Draw Q [sum(lens_q),H,d], then K and V [sum(lens_k),Hkv,d] (in that
    order), iid N(0,1) float32 from ``default_rng(seed)``, rounded to f16 or
    bf16; offsets are the running sums of the lengths."""
    lens_q, lens_k = tuple(int(x) for x in lens_q), tuple(int(x) for x in lens_k)
    assert len(lens_q) == len(lens_k)
    rng = np.random.default_rng(seed)
    Tq, Tk = sum(lens_q), sum(lens_k)
    case = VarlenCase(lens_q, lens_k, H, Hkv, d, dtype, bool(causal),
                      default_scale(d) if scale is None else float(scale), seed)
    case.cu_q = np.concatenate([[0], np.cumsum(lens_q)]).astype(np.int32)
    case.cu_k = np.concatenate([[0], np.cumsum(lens_k)]).astype(np.int32)
    enc = []
    for shp in ((Tq, H, d), (Tk, Hkv, d), (Tk, Hkv, d)):
        x = rng.standard_normal(int(np.prod(shp)), dtype=np.float32)
        if dtype == F16:
            enc.append(f32_to_f16(x).view(np.uint16).reshape(shp))
        elif dtype == BF16:
            enc.append(f32_to_bf16_bits(x).reshape(shp))
        else:
            raise ValueError("variable-length cases are f16/bf16")
    case.q, case.k, case.v = enc
    return case


def quantize_e4m3_blocks(x: np.ndarray, block_rows: int) -> tuple[np.ndarray, np.ndarray]:
    """Per-block e4m3 quantisation of [..., N, d]: for each block of
    ``block_rows`` rows, s = amax/448 (float32; 1 for a zero block) and
    codes = e4m3(x/s) with x/s in float32. Returns (codes, scales [..., nblk])."""
    x = np.asarray(x, dtype=np.float32)
    N = x.shape[-2]
    nb = -(-N // block_rows)
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-2] + (nb,), dtype=np.float32)
    for i in range(nb):
        sl = slice(i * block_rows, (i + 1) * block_rows)
        amax = np.max(np.abs(x[..., sl, :]), axis=(-2, -1)).astype(np.float32)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1)).astype(np.float32)
        scales[..., i] = s
        codes[..., sl, :] = e4m3_encode((x[..., sl, :] / s[..., None, None]).astype(np.float32))
    return codes, scales


@dataclass
class Fp8BlockCase:
    """e4m3 codes of Q, K, V [B,H,N,d] with block scales (Q per 128 rows, K
    and V per 64 rows), and the exact values they stand for."""
    B: int
    H: int
    N: int
    d: int
    causal: bool
    scale: float
    seed: int
    q: np.ndarray = field(repr=False, default=None)
    k: np.ndarray = field(repr=False, default=None)
    v: np.ndarray = field(repr=False, default=None)
    qs: np.ndarray = field(repr=False, default=None)
    ks: np.ndarray = field(repr=False, default=None)
    vs: np.ndarray = field(repr=False, default=None)
    dtype: int = FP8_E4M3

    def exact(self, which: str) -> np.ndarray:
        codes = getattr(self, which)
        s, rows = {"q": (self.qs, 128), "k": (self.ks, 64), "v": (self.vs, 64)}[which]
        per_row = np.repeat(s.astype(np.float64), rows, axis=-1)[..., :self.N]
        return e4m3_decode(codes).astype(np.float64) * per_row[..., None]


def make_fp8_block_case(B, H, N, d, causal=False, seed=0, dist="normal") -> Fp8BlockCase:
    """The draws of ``make_case`` (same seed, same order, same distributions),
    quantised per block on the host: Q per 128 rows, K and V per 64 rows."""
    n = B * H * N * d
    rng = np.random.default_rng(seed)
    draws = [rng.standard_normal(n, dtype=np.float32) for _ in range(3)]
    if dist == "outlier":
        for i in range(3):
            mask = rng.random(n, dtype=np.float32) < np.float32(0.001)
            big = rng.standard_normal(n, dtype=np.float32) * np.float32(10.0)
            draws[i] = (draws[i] + np.where(mask, big, np.float32(0))).astype(np.float32)
    case = Fp8BlockCase(B, H, N, d, bool(causal), default_scale(d), seed)
    shape = (B, H, N, d)
    case.q, case.qs = quantize_e4m3_blocks(draws[0].reshape(shape), 128)
    case.k, case.ks = quantize_e4m3_blocks(draws[1].reshape(shape), 64)
    case.v, case.vs = quantize_e4m3_blocks(draws[2].reshape(shape), 64)
    return case
