"""The C-ABI library on a machine without a GPU: it loads, exports every
function include/fa.h declares, and rejects bad arguments on the host before
any HIP call (these calls never reach the device)."""
import ctypes
import os
import re

import pytest

import fa_inputs
import io_aware_softmax_fa_amd as fa
from io_aware_softmax_fa_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def _header_text():
    with open(HEADER) as f:
        return f.read()


def _declared_functions():
    text = re.sub(r"/\*.*?\*/", "", _header_text(), flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, re.M)))


def _header_defines():
    return {m.group(1): int(m.group(2)) for m in
            re.finditer(r"#define\s+(FA_\w+)\s+\(?(-?\d+)\)?", _header_text())}


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert names == ["fa_bwd", "fa_fwd", "fa_fwd_fp8", "fa_fwd_fp8_block", "fa_fwd_kv",
                     "fa_fwd_kv_noalloc", "fa_fwd_kv_workspace", "fa_fwd_varlen", "fa_fwd_varlen_workspace",
                     "fa_quantize_fp8", "fa_strerror", "fa_varlen_order", "fa_version"]
    h = ctypes.CDLL(_lib.LIB_PATH)
    for n in names:
        assert hasattr(h, n), n


def test_constants_agree_with_header():
    d = _header_defines()
    assert d["FA_OK"] == fa.FA_OK == 0
    assert d["FA_ERR_INVALID_ARG"] == fa.FA_ERR_INVALID_ARG
    assert d["FA_ERR_UNSUPPORTED"] == fa.FA_ERR_UNSUPPORTED
    assert d["FA_ERR_LAUNCH"] == fa.FA_ERR_LAUNCH
    assert d["FA_ERR_TOO_LARGE"] == fa.FA_ERR_TOO_LARGE
    assert d["FA_F16"] == fa.FA_F16 == fa_inputs.F16
    assert d["FA_BF16"] == fa.FA_BF16 == fa_inputs.BF16
    assert d["FA_FP8_E4M3"] == fa.FA_FP8_E4M3 == fa_inputs.FP8_E4M3
    assert fa.version() == d["FA_VERSION"]


def test_strerror():
    for c in (0, -1, -2, -3, 7):
        assert isinstance(fa.strerror(c), str) and fa.strerror(c)
    assert fa.strerror(0) == "success"


# fake, never-dereferenced device addresses (16-byte aligned, disjoint)
MB = 1 << 20
Q, K, V, O, L = (0x100000000 + i * 256 * MB for i in range(5))
GOOD = dict(q=Q, k=K, v=V, o=O, lse=L, B=1, H=2, N=128, d=64, scale=0.125, causal=0,
            dtype=fa.FA_BF16, stream=None)


def call(**kw):
    a = dict(GOOD, **kw)
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                     a["scale"], a["causal"], a["dtype"], a["stream"])


def call8(**kw):
    a = dict(GOOD, **kw)
    ds = a.get("descale", (0.01, 0.01, 0.01))
    return fa.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], *ds, a["B"], a["H"], a["N"],
                         a["d"], a["scale"], a["causal"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(v=0), dict(o=0), dict(lse=0),
    dict(q=Q + 2), dict(o=O + 8), dict(lse=L + 4),
    dict(B=-1), dict(H=-3), dict(N=-1), dict(d=0),
    dict(scale=0.0), dict(scale=-1.0), dict(scale=float("inf")), dict(scale=float("nan")),
    dict(causal=2), dict(causal=-1), dict(dtype=3), dict(dtype=-1),
    dict(o=Q), dict(o=Q + 64), dict(lse=K + 16), dict(lse=O + 128),
    dict(B=1 << 30, H=1 << 30, N=1 << 20),
])
def test_invalid_arguments(kw):
    assert call(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=32), dict(d=96), dict(d=256), dict(dtype=fa.FA_FP8_E4M3)])
def test_unsupported(kw):
    assert call(**kw) == fa.FA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(N=0),
                                dict(N=0, q=0, k=0, v=0, o=0, lse=0)])
def test_empty_problem_is_a_no_op(kw):
    assert call(**kw) == fa.FA_OK
    assert call8(**kw) == fa.FA_OK


@pytest.mark.parametrize("kw", [dict(q=0), dict(descale=(0.0, 1.0, 1.0)),
                                dict(descale=(1.0, float("nan"), 1.0)),
                                dict(descale=(1.0, 1.0, -2.0)), dict(scale=0.0),
                                dict(o=K + 4096)])
def test_fp8_invalid_arguments(kw):
    assert call8(**kw) == fa.FA_ERR_INVALID_ARG


def test_fp8_unsupported_head_dim():
    assert call8(d=96) == fa.FA_ERR_UNSUPPORTED


# backward: fake addresses for q, k, v, o, dout, lse, dq, dk, dv, workspace
BQ, BK, BV, BO, BG, BL, BDQ, BDK, BDV, BW = (0x200000000 + i * 256 * MB for i in range(10))
BGOOD = dict(q=BQ, k=BK, v=BV, o=BO, dout=BG, lse=BL, dq=BDQ, dk=BDK, dv=BDV, ws=BW, B=1, H=2,
             N=128, d=128, scale=0.088, causal=1, dtype=fa.FA_BF16, stream=None)


def callb(**kw):
    a = dict(BGOOD, **kw)
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["dout"], a["lse"], a["dq"], a["dk"],
                     a["dv"], a["ws"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                     a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(dout=0), dict(lse=0), dict(dq=0), dict(ws=0), dict(dv=BDV + 4),
    dict(B=-1), dict(scale=0.0), dict(causal=3), dict(dtype=7),
    dict(dq=BQ), dict(dk=BDQ + 64), dict(ws=BDV + 256), dict(dv=BL),
    dict(B=1 << 30, H=1 << 30, N=1 << 20),
])
def test_bwd_invalid_arguments(kw):
    assert callb(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(dtype=fa.FA_FP8_E4M3)])
def test_bwd_unsupported(kw):
    assert callb(**kw) == fa.FA_ERR_UNSUPPORTED


def test_bwd_empty_problem_is_a_no_op():
    assert callb(N=0) == fa.FA_OK
    assert callb(B=0, q=0, dq=0) == fa.FA_OK


# grouped / key-history forward
KQ, KK, KV, KO, KL, KW = (0x300000000 + i * 256 * MB for i in range(6))
KGOOD = dict(q=KQ, k=KK, v=KV, o=KO, lse=KL, B=2, H=8, Hkv=2, Nq=1, Nk=4096, d=128, scale=0.088,
             causal=1, dtype=fa.FA_BF16, splits=4, ws=KW, stream=None)


def callkv(**kw):
    a = dict(KGOOD, **kw)
    return fa.fa_fwd_kv(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"], a["Nq"],
                        a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"], a["splits"], a["ws"],
                        a["stream"])


def test_kv_workspace_size():
    assert fa.fa_fwd_kv_workspace(2, 8, 3, 128, 4) == 4 * 2 * 8 * 3 * 129 * 4
    assert fa.fa_fwd_kv_workspace(2, 8, 3, 128, 1) == 0
    assert fa.fa_fwd_kv_workspace(0, 8, 3, 128, 4) == 0


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(o=0), dict(lse=0), dict(ws=0), dict(ws=KW + 4),
    dict(Hkv=3), dict(Hkv=0), dict(Nk=0), dict(Nq=5000), dict(splits=0), dict(splits=2000),
    dict(scale=0.0), dict(causal=2), dict(dtype=9), dict(B=-1),
    dict(o=KQ), dict(lse=KO), dict(ws=KK + 64), dict(ws=KO),
])
def test_kv_invalid_arguments(kw):
    assert callkv(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(dtype=fa.FA_FP8_E4M3)])
def test_kv_unsupported(kw):
    assert callkv(**kw) == fa.FA_ERR_UNSUPPORTED


def test_kv_empty_and_unsplit_calls_need_no_workspace():
    assert callkv(Nq=0) == fa.FA_OK
    assert callkv(B=0, q=0) == fa.FA_OK


def callkv_noalloc(**kw):
    a = dict(KGOOD, **kw)
    return fa.fa_fwd_kv_noalloc(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["Hkv"],
                                a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], a["dtype"],
                                a["splits"], a["stream"])


def test_noalloc_scratch_limit():
    """The allocation-free entry point rejects, on the host, any call whose
    partials exceed its static scratch; the limit is the header's."""
    assert "FA_NOALLOC_SCRATCH_BYTES" in _header_text()
    assert fa.FA_NOALLOC_SCRATCH_BYTES == 16 << 20
    per = fa.fa_fwd_kv_workspace(2, 8, 8, 128, 1024) // 1024   # one range of these rows
    fit = fa.FA_NOALLOC_SCRATCH_BYTES // per
    assert fit < 1024
    assert callkv_noalloc(Nq=8, splits=fit + 1) == fa.FA_ERR_TOO_LARGE
    assert callkv_noalloc(Nq=64, splits=64) == fa.FA_ERR_TOO_LARGE
    assert "scratch" in fa.strerror(fa.FA_ERR_TOO_LARGE)


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(o=0), dict(lse=0), dict(Hkv=3), dict(Hkv=0), dict(Nk=0),
    dict(Nq=5000), dict(splits=0), dict(splits=2000), dict(scale=0.0), dict(causal=2),
    dict(dtype=9), dict(B=-1), dict(o=KQ), dict(lse=KO),
])
def test_noalloc_invalid_arguments(kw):
    assert callkv_noalloc(**kw) == fa.FA_ERR_INVALID_ARG


def test_noalloc_empty_is_a_no_op():
    assert callkv_noalloc(Nq=0) == fa.FA_OK
    assert callkv_noalloc(B=0, q=0) == fa.FA_OK


# variable-length forward
VQ, VK, VV, VO, VL_, VCQ, VCK, VW = (0x500000000 + i * 256 * MB for i in range(8))
VORD = 0x500000000 + 8 * 256 * MB
VGOOD = dict(q=VQ, k=VK, v=VV, o=VO, lse=VL_, cq=VCQ, ck=VCK, order=None, B=3, H=8, Hkv=2,
             maxq=100, maxk=300, tq=200, tk=500, d=128, scale=0.088, causal=1, dtype=fa.FA_BF16,
             splits=2, ws=VW, stream=None)


def callvl(**kw):
    a = dict(VGOOD, **kw)
    return fa.fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"], a["order"],
                            a["B"], a["H"], a["Hkv"], a["maxq"], a["maxk"], a["tq"], a["tk"],
                            a["d"], a["scale"], a["causal"], a["dtype"], a["splits"], a["ws"],
                            a["stream"])


def test_varlen_workspace_size():
    assert fa.fa_fwd_varlen_workspace(200, 8, 128, 3) == 3 * 200 * 8 * 129 * 4
    assert fa.fa_fwd_varlen_workspace(200, 8, 128, 1) == 0
    assert fa.fa_fwd_varlen_workspace(0, 8, 128, 3) == 0


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(k=0), dict(o=0), dict(lse=0), dict(cq=0), dict(ck=0), dict(ws=0),
    dict(ws=VW + 4), dict(q=VQ + 8), dict(lse=VL_ + 2), dict(cq=VCQ + 2),
    dict(Hkv=3), dict(Hkv=0), dict(H=0), dict(maxq=-1), dict(maxk=-1), dict(tq=-1), dict(tk=-1),
    dict(splits=0), dict(splits=2000), dict(scale=float("nan")), dict(causal=2), dict(dtype=9),
    dict(B=-1), dict(o=VQ), dict(lse=VO), dict(ws=VK + 64), dict(cq=VO + 64), dict(o=VCK),
    dict(order=VORD + 2), dict(order=VO + 64), dict(order=VW + 4), dict(order=VL_),
])
def test_varlen_invalid_arguments(kw):
    assert callvl(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(dtype=fa.FA_FP8_E4M3)])
def test_varlen_unsupported(kw):
    assert callvl(**kw) == fa.FA_ERR_UNSUPPORTED


def test_varlen_empty_batches_are_no_ops():
    assert callvl(B=0) == fa.FA_OK
    assert callvl(tq=0) == fa.FA_OK
    assert callvl(maxq=0) == fa.FA_OK
    assert callvl(B=0, order=VORD) == fa.FA_OK


# longest-first order of a variable-length batch
OGOOD = dict(cq=VCQ, ck=VCK, B=3, maxq=100, maxk=300, tq=200, tk=500, splits=1, order=VORD,
             stream=None)


def callord(**kw):
    a = dict(OGOOD, **kw)
    return fa.fa_varlen_order(a["cq"], a["ck"], a["B"], a["maxq"], a["maxk"], a["tq"], a["tk"],
                              a["splits"], a["order"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(cq=0), dict(ck=0), dict(order=0), dict(cq=VCQ + 2), dict(order=VORD + 1),
    dict(B=-1), dict(maxq=-1), dict(maxk=-1), dict(tq=-1), dict(tk=-1), dict(splits=0),
    dict(splits=1025), dict(B=(1 << 20) + 1), dict(order=VCQ + 4), dict(order=VCK - 8),
])
def test_varlen_order_invalid_arguments(kw):
    assert callord(**kw) == fa.FA_ERR_INVALID_ARG


def test_varlen_order_empty_batch_is_a_no_op():
    assert callord(B=0) == fa.FA_OK
    assert callord(B=0, order=0, cq=0) == fa.FA_OK


# fp8 with block scales, and the quantiser
BQ, BK, BV, BO, BL, BSQ, BSK, BSV = (0x700000000 + i * 256 * MB for i in range(8))
B8GOOD = dict(q=BQ, k=BK, v=BV, o=BO, lse=BL, sq=BSQ, sk=BSK, sv=BSV, B=2, H=4, N=1000, d=128,
             scale=0.088, causal=0, stream=None)


def callb8(**kw):
    a = dict(B8GOOD, **kw)
    return fa.fa_fwd_fp8_block(a["q"], a["k"], a["v"], a["o"], a["lse"], a["sq"], a["sk"],
                               a["sv"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["causal"],
                               a["stream"])


@pytest.mark.parametrize("kw", [
    dict(q=0), dict(o=0), dict(sq=0), dict(sk=0), dict(sv=0), dict(sq=BSQ + 2), dict(q=BQ + 8),
    dict(scale=-1.0), dict(causal=3), dict(B=-1), dict(o=BQ), dict(sk=BO + 64), dict(sv=BL),
])
def test_fp8_block_invalid_arguments(kw):
    assert callb8(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(B=1, H=1, N=131072 + 64)])
def test_fp8_block_unsupported(kw):
    assert callb8(**kw) == fa.FA_ERR_UNSUPPORTED


def test_fp8_block_empty_is_a_no_op():
    assert callb8(N=0) == fa.FA_OK


QX, Q8, QS, QG = (0x900000000 + i * 256 * MB for i in range(4))
QGOOD = dict(x=QX, x8=Q8, s=QS, g=QG, B=2, H=4, N=1000, d=128, rows=64, dtype=fa.FA_BF16,
             stream=None)


def callq(**kw):
    a = dict(QGOOD, **kw)
    return fa.fa_quantize_fp8(a["x"], a["x8"], a["s"], a["g"], a["B"], a["H"], a["N"], a["d"],
                              a["rows"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw", [
    dict(x=0), dict(x8=0), dict(s=0), dict(x=QX + 8), dict(x8=Q8 + 4), dict(s=QS + 2),
    dict(g=QG + 4), dict(B=-1), dict(N=-1), dict(rows=0), dict(dtype=7), dict(x8=QX + 64),
    dict(s=Q8), dict(g=QS), dict(s=QX),
])
def test_quantize_invalid_arguments(kw):
    assert callq(**kw) == fa.FA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(d=96), dict(rows=32), dict(rows=256),
                                dict(dtype=fa.FA_FP8_E4M3)])
def test_quantize_unsupported(kw):
    assert callq(**kw) == fa.FA_ERR_UNSUPPORTED


def test_quantize_empty_is_a_no_op():
    assert callq(N=0) == fa.FA_OK
    assert callq(B=0, x=0) == fa.FA_OK


def test_mfma_probe_library():
    """The matrix-pipe ceiling probe bench.py times beside the forward: it is
    built, exports its two calls, rejects bad arguments on the host and counts
    32x32x16 FLOPs (2 * 32 * 32 * 16 per instruction, 4 chains, 8 waves)."""
    from io_aware_softmax_fa_amd import build as fab
    p = ctypes.CDLL(fab.PROBE_OUT)
    p.fa_probe_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    p.fa_probe_mfma_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    p.fa_probe_mfma_flops.restype = ctypes.c_double
    assert p.fa_probe_mfma(None, 4, 8, None) == -1
    assert p.fa_probe_mfma(ctypes.c_void_p(4096), 0, 8, None) == -1
    assert p.fa_probe_mfma(ctypes.c_void_p(4096), 4, 12, None) == -1   # iters not a multiple of 8
    assert p.fa_probe_mfma_flops(3, 16) == 3 * 8 * 16 * 4 * (2 * 32 * 32 * 16)
