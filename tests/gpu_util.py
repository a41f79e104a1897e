"""Helpers for the GPU parity tests: upload a seeded case, run it through the C
ABI, and compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import fa_inputs as fi
import oracle

# max |dO| by input dtype and |dLSE| for all, against the fp64 oracle
TOL_O = {fi.F16: 4e-3, fi.BF16: 1.6e-2, fi.FP8_E4M3: 6e-2}
TOL_LSE = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_device(case):
    import torch
    if case.dtype == fi.FP8_E4M3:
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    else:
        tdt = torch.float16 if case.dtype == fi.F16 else torch.bfloat16
        conv = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(tdt).cuda()
    return conv(case.q), conv(case.k), conv(case.v)


def run_gpu(case, poison=True, tensors=None):
    """Run ``case`` through the C ABI on cuda:0; returns (O, LSE) as float64
    numpy arrays. Outputs are pre-filled with NaN so an unwritten element
    cannot pass."""
    import torch
    import io_aware_softmax_fa_amd as fa
    q, k, v = tensors if tensors is not None else to_device(case)
    B, H, N, d = case.B, case.H, case.N, case.d
    odt = torch.bfloat16 if case.dtype in (fi.BF16, fi.FP8_E4M3) else torch.float16
    o = torch.empty((B, H, N, d), dtype=odt, device="cuda")
    lse = torch.empty((B, H, N), dtype=torch.float32, device="cuda")
    if poison:
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
    if case.dtype == fi.FP8_E4M3:
        fa.forward_fp8(q, k, v, case.descale, case.causal, case.scale, out=o, lse=lse)
    else:
        fa.forward(q, k, v, case.causal, case.scale, out=o, lse=lse)
    torch.cuda.synchronize()
    return (o.float().cpu().numpy().astype(np.float64),
            lse.cpu().numpy().astype(np.float64))


def _head_rows(case, b, h, rows_per_head, seed_rows):
    return (np.arange(case.N) if rows_per_head is None
            else fi.sample_rows(seed_rows, b, h, case.N, rows_per_head))


def oracle_heads(case, rows_per_head=None, seed_rows=0, chunk=2048):
    """Yield (b, h, rows, O_ref, LSE_ref) for every head, the oracle evaluated
    on host threads (one head per thread, rows in chunks of ``chunk`` so a
    head at N = 8192 holds at most chunk x N fp64 scores at a time)."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    q, k, v = case.exact("q"), case.exact("k"), case.exact("v")

    def one(bh):
        b, h = bh
        rows = _head_rows(case, b, h, rows_per_head, seed_rows)
        parts = [oracle.attention_rows(q[b, h], k[b, h], v[b, h], rows[i:i + chunk], case.scale,
                                       case.causal) for i in range(0, len(rows), chunk)]
        ro = np.concatenate([p[0] for p in parts]) if parts else np.zeros((0, case.d))
        rl = np.concatenate([p[1] for p in parts]) if parts else np.zeros(0)
        return b, h, rows, ro, rl

    heads = [(b, h) for b in range(case.B) for h in range(case.H)]
    workers = max(1, min(8, len(os.sched_getaffinity(0)), len(heads)))
    if workers == 1 or case.N < 1024:
        yield from map(one, heads)
        return
    with ThreadPoolExecutor(workers) as ex:
        yield from ex.map(one, heads)


def compare(case, o, lse, rows_per_head=None, seed_rows=0):
    """Max |dO|, max |dLSE| and RMSE of O against the oracle, over every row
    (rows_per_head None) or over ``fa_inputs.sample_rows`` of each head."""
    worst_o = worst_l = 0.0
    se = 0.0
    cnt = 0
    for b, h, rows, ro, rl in oracle_heads(case, rows_per_head, seed_rows):
        go, gl = o[b, h][rows], lse[b, h][rows]
        assert np.all(np.isfinite(go)) and np.all(np.isfinite(gl)), "non-finite output"
        worst_o = max(worst_o, float(np.max(np.abs(go - ro))))
        worst_l = max(worst_l, float(np.max(np.abs(gl - rl))))
        se += float(np.sum((go - ro) ** 2))
        cnt += go.size
    return worst_o, worst_l, (se / max(cnt, 1)) ** 0.5


# fp8 cases outside the 6e-2 gate: bound = FP8_K_SIGMA standard deviations of
# the e4m3 rounding noise of P + bf16 rounding of O + FP8_FLOOR (see fp8_bound)
FP8_K_SIGMA = 3.5
FP8_FLOOR = 2.5e-4


def fp8_sigma(w, vv, r=None):
    """Standard deviation of the O error that e4m3 rounding of P causes, per
    element, under the model below; w: normalised weights [rows, N] from the
    oracle's scores, vv: V^2 [N, d]; r: per-key factor P is scaled by before
    rounding (block scales), default 1.

    Rounding p to e4m3 (3 mantissa bits, round to nearest even) moves it by
    at most half a step: relative 2^-4 for normal values, modelled as
    independent and uniform (variance (2^-4)^2/3 of the weight, squared).
    Values under 2^-6 are subnormal in e4m3 with an absolute half step of
    2^-10; in weight units that is at most 2^-10 (the row's reference value
    m never exceeds its row max, so the row sum l >= 1), counted for every
    key whose scaled weight w*r is below 2^-6."""
    if r is None:
        sub = w < 2.0 ** -6
        var = (2.0 ** -4) ** 2 / 3 * ((w ** 2) @ vv) + (2.0 ** -10) ** 2 / 3 * (sub @ vv)
    else:
        sub = (w * r[None, :]) < 2.0 ** -6
        var = (2.0 ** -4) ** 2 / 3 * ((w ** 2) @ vv) + \
            (2.0 ** -10) ** 2 / 3 * ((sub / r[None, :] ** 2) @ vv)
    return np.sqrt(var)


def fp8_bound(case, rows_per_head=None):
    """Per-element bound on |dO| implied by quantising P to e4m3 before GEMM1,
    for fp8 cases outside the B=4 H=16 N=8192 workload the 6e-2 gate is
    stated for (short and causal rows, dominated by a few keys, where e4m3
    rounding of P alone can pass 6e-2): FP8_K_SIGMA = 3.5 standard deviations
    of the rounding noise (fp8_sigma), plus the bf16 rounding of O (half an ulp
    is at most 2^-8 |O|), plus FP8_FLOOR = 2.5e-4 for fp32 accumulation and the
    hardware reciprocal (both ~1e-6 here), which matters only where the noise
    term vanishes (a row on one key, P = 1 exactly).

    The worst case over every fp8 edge case of the per-tensor and block-scale
    kernels measured 0.71-0.72 of this bound: a kernel 1.4x worse fails. With
    six deviations and a 2e-3 floor the same cases used 0.40 of the bound.
    Returns [B][H] arrays of [rows, d]."""
    q, k, v = case.exact("q"), case.exact("k"), case.exact("v")
    out = []
    for b in range(case.B):
        hb = []
        for h in range(case.H):
            rows = (np.arange(case.N) if rows_per_head is None
                    else fi.sample_rows(case.seed, b, h, case.N, rows_per_head))
            s = case.scale * (q[b, h][rows] @ k[b, h].T)
            if case.causal:
                s = np.where(np.arange(case.N)[None, :] > rows[:, None], -np.inf, s)
            w = np.exp(s - s.max(1, keepdims=True))
            w /= w.sum(1, keepdims=True)
            o = w @ v[b, h]
            hb.append(FP8_K_SIGMA * fp8_sigma(w, v[b, h] ** 2) + 2.0 ** -8 * np.abs(o) + FP8_FLOOR)
        out.append(hb)
    return out


def check(case, rows_per_head=None, label="", fp8_derived=False):
    say(f"[gpu] {label} B={case.B} H={case.H} N={case.N} d={case.d} "
        f"dtype={fi.DTYPE_NAMES[case.dtype]} causal={case.causal} seed={case.seed}")
    o, lse = run_gpu(case)
    do, dl, rmse = compare(case, o, lse, rows_per_head, case.seed)
    say(f"      max|dO|={do:.3e} max|dLSE|={dl:.3e} rmse={rmse:.3e}")
    if fp8_derived:
        bound = fp8_bound(case, rows_per_head)
        q, k, v = case.exact("q"), case.exact("k"), case.exact("v")
        worst = 0.0
        for b in range(case.B):
            for h in range(case.H):
                rows = (np.arange(case.N) if rows_per_head is None
                        else fi.sample_rows(case.seed, b, h, case.N, rows_per_head))
                ro, _ = oracle.attention_rows(q[b, h], k[b, h], v[b, h], rows, case.scale,
                                              case.causal)
                worst = max(worst, float(np.max(np.abs(o[b, h][rows] - ro) / bound[b][h])))
        say(f"      fp8 derived bound: worst |dO|/bound = {worst:.3f}")
        assert worst <= 1.0, f"|dO| exceeds the e4m3-derived bound by {worst:.3f}x"
    else:
        assert do <= TOL_O[case.dtype], f"max|dO| {do} > {TOL_O[case.dtype]}"
    assert dl <= TOL_LSE, f"max|dLSE| {dl} > {TOL_LSE}"
    return o, lse
