"""The software exp2 of the measurement variant (exp2_fma in fa_fwd.hip, the
FMA-pipe exponential of the FA4 walkthrough, section 3.1.3): its polynomial
is the one csrc/fit_exp2.py fits, and the split + polynomial + exponent
scaling, emulated step by step in float32, stays within the fit's error of
2^x over the whole argument range the softmax produces (masked -inf gives 0)."""
import os
import re

import importlib.util

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "io_aware_softmax_fa_amd", "csrc")
SRC = os.path.join(CSRC, "fa_fwd.hip")
_spec = importlib.util.spec_from_file_location("fit_exp2", os.path.join(CSRC, "fit_exp2.py"))
fit_exp2 = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(fit_exp2)


def kernel_coefficients():
    text = open(SRC).read()
    body = text[text.index("float exp2_fma(float x)"):]
    body = body[:body.index("}")]
    lits = [float(v) for v in re.findall(r"([0-9.]+e[+-][0-9]+)f", body)]
    # fma(c3, f, c2), fma(p, f, c1), fma(p, f, c0)
    c3, c2, c1, c0 = lits
    return np.array([c0, c1, c2, c3], np.float32)


def test_kernel_uses_the_fitted_polynomial():
    c32, e64, e32 = fit_exp2.main(3)
    assert e64 < 1e-4 and e32 < 1e-4
    np.testing.assert_array_equal(kernel_coefficients(), c32)


def exp2_fma_f32(x):
    """exp2_fma's steps in float32 (each FMA rounded once, via float64)."""
    c0, c1, c2, c3 = (np.float64(c) for c in kernel_coefficients())
    x = np.asarray(x, np.float32)
    xc = np.maximum(x, np.float32(-1000.0))
    y = (xc + np.float32(12582912.0)).astype(np.float32)
    r = (y - np.float32(12582912.0)).astype(np.float32)
    f = (xc - r).astype(np.float64)
    p = np.float32(c3 * f + c2).astype(np.float64)
    p = np.float32(p * f + c1).astype(np.float64)
    p = np.float32(p * f + c0)
    n = (y.view(np.uint32).astype(np.int64) - 0x4B400000)
    return np.ldexp(p.astype(np.float64), n).astype(np.float32)


def test_emulated_software_exp2_accuracy():
    x = np.concatenate([np.linspace(-125.0, 8.5, 2_000_001, dtype=np.float32),
                        np.float32(np.arange(-126, 9)) + np.float32(0.5)])   # rounding ties
    got = exp2_fma_f32(x).astype(np.float64)
    want = np.exp2(x.astype(np.float64))
    assert np.max(np.abs(got / want - 1.0)) < 1.0e-4
    assert exp2_fma_f32(np.float32(-np.inf)) == 0.0
    assert exp2_fma_f32(np.float32(-2000.0)) == 0.0
    assert exp2_fma_f32(np.float32(0.0)) == np.float32(kernel_coefficients()[0])
