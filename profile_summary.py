#!/usr/bin/env python3
"""Short text summaries of rocprofv3 runs of ``bench.py``, for ``profiles/``.

Reads rocprofv3's CSV output (``-f csv -d DIR -o run``) and writes a few lines
of figures with the command that made them:

    python profile_summary.py ktrace   --dir D --kernel fa_fwd_kernel --skip W --take K ...
    python profile_summary.py traffic  --fetch-dir D1 --write-dir D2 --kernel fa_fwd_kernel ...
    python profile_summary.py counters --dirs D1 D2 ... --kernel fa_fwd_kernel ...

``--skip`` / ``--take`` select the dispatches of the kernel by launch order, so
a summary covers exactly the launches ``bench.py`` times (its warm-up calls
come first, then the timed steps; the sustained run and the clock sampling
come after them).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
SOURCES = {"fa_fwd": "fa_fwd.hip", "fa_bwd": "fa_bwd.hip", "fa_quant": "fa_quant.hip",
           "bwd_": "fa_bwd.hip"}


def source_of(kernel: str) -> str:
    return next((f for k, f in SOURCES.items() if kernel.startswith(k)), "fa_fwd.hip")


def source_digest(kernel: str) -> str:
    """First 16 hex digits of the SHA-256 of the kernel's source file followed
    by the header every kernel source includes (bench.py reads a traffic
    summary only while this still matches)."""
    h = hashlib.sha256()
    for name in (source_of(kernel), "fa_common.h"):
        with open(os.path.join(ROOT, "io_aware_softmax_fa_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _csv(d: str, suffix: str):
    paths = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not paths:
        sys.exit(f"no *{suffix} under {d}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


def _short(name: str) -> str:
    return name.replace("void ", "").replace("(anonymous namespace)::", "").split("(")[0]


def _select(rows, kernel, skip, take, key="Kernel_Name"):
    """Rows of dispatches of ``kernel`` in launch order, after ``skip``, at most ``take``."""
    mine = [r for r in rows if kernel in r[key]]
    mine.sort(key=lambda r: int(r.get("Dispatch_Id", r.get("Correlation_Id", 0)) or 0))
    mine = mine[skip:]
    return mine[:take] if take else mine


def _bench_line(path):
    if not path:
        return None
    for line in open(path):
        line = line.strip()
        if line.startswith("{"):
            try:
                return json.loads(line)
            except json.JSONDecodeError:
                pass
    return None


def ktrace(a) -> str:
    allrows = _csv(a.dir, "kernel_trace.csv")
    rows = _select(allrows, a.kernel, a.skip, a.take)
    if not rows:
        sys.exit(f"no dispatch of {a.kernel} in {a.dir}")
    ns = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rows]
    out = [f"# {a.title}",
           f"command: {a.command}",
           f"summary: python profile_summary.py ktrace --kernel {a.kernel}"
           + (f" --also {' '.join(a.also)}" if a.also else "")
           + f" --skip {a.skip} --take {a.take} (dispatches of each kernel in launch order"
           + (f"; the first {a.skip} are bench.py's warm-up calls)" if a.skip else ")"),
           f"kernel_source_sha256_16: {source_digest(a.kernel)}  ({source_of(a.kernel)} + fa_common.h)",
           f"kernel: {_short(rows[0]['Kernel_Name'])}",
           f"  dispatches: {len(ns)}  mean_ns: {statistics.mean(ns):.0f}  median_ns: "
           f"{statistics.median(ns):.0f}  min_ns: {min(ns)}  max_ns: {max(ns)}"]
    if a.flops:
        out.append(f"  TFLOP/s at mean: {a.flops / (statistics.mean(ns) * 1e-9) / 1e12:.1f}  "
                   f"at median: {a.flops / (statistics.median(ns) * 1e-9) / 1e12:.1f}  "
                   f"({a.flops:.4e} FLOP per launch)")
    total = statistics.mean(ns)
    for k in a.also or []:
        rk = _select(allrows, k, a.skip, a.take)
        if not rk:
            sys.exit(f"no dispatch of {k} in {a.dir}")
        nk = [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rk]
        total += statistics.mean(nk)
        out += [f"kernel: {_short(rk[0]['Kernel_Name'])}",
                f"  dispatches: {len(nk)}  mean_ns: {statistics.mean(nk):.0f}  median_ns: "
                f"{statistics.median(nk):.0f}  min_ns: {min(nk)}  max_ns: {max(nk)}"]
    if a.also:
        out.append(f"sum of the kernels' mean durations (one step): {total:.0f} ns")
    bj = _bench_line(a.bench_json)
    if bj:
        rf = bj["roofline"]
        out.append(f"bench.py line of the same run: value {bj['value']} {bj['unit']}, ms_per_step "
                   f"{bj['ms_per_step']}, kernel_ms_avg {rf['kernel_ms_avg']} (HIP events), "
                   f"achieved {rf['achieved']} {rf['unit']} = {100 * rf['frac']:.1f}% of "
                   f"{rf['peak']}")
        if bj.get("clock"):
            out.append(f"engine clock while the step repeats: {bj['clock']['sclk_mhz_median']} MHz "
                       f"(median of {bj['clock']['samples']} samples)")
    return "\n".join(out) + "\n"


def traffic(a) -> str:
    res = {}
    for c, d in (("FETCH_SIZE", a.fetch_dir), ("WRITE_SIZE", a.write_dir)):
        rows = _csv(d, "counter_collection.csv")
        copy = [float(r["Counter_Value"]) for r in rows
                if "copyBuffer" in r["Kernel_Name"] and r["Counter_Name"] == c]
        kern = [float(r["Counter_Value"]) for r in
                _select([r for r in rows if r["Counter_Name"] == c], a.kernel, a.skip, a.take)]
        if not copy or not kern:
            sys.exit(f"{c}: no copy or no {a.kernel} dispatch in {d}")
        cp = statistics.mean(copy)
        # the calibration copy moves 1 GiB: 1048576 KiB read and 1048576 KiB written
        res[c] = (statistics.mean(kern), 1048576.0 / cp, len(kern), cp)
    fetch = res["FETCH_SIZE"][0] * 1024 * res["FETCH_SIZE"][1]
    write = res["WRITE_SIZE"][0] * 1024 * res["WRITE_SIZE"][1]
    out = [f"# {a.title}",
           f"command (pass 1): {a.command}",
           f"command (pass 2): the same with --pmc WRITE_SIZE -d <write dir>",
           f"summary: python profile_summary.py traffic --kernel {a.kernel} --skip {a.skip}",
           f"kernel_source_sha256_16: {source_digest(a.kernel)}  ({source_of(a.kernel)} + fa_common.h)",
           "calibration: torch 1 GiB device copy (__amd_rocclr_copyBuffer) in the same process"]
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        k, fac, n, cp = res[c]
        out.append(f"{c}: kernel {k:.1f} KiB/dispatch over {n} dispatches; copy reads {cp:.1f} KiB "
                   f"for 1048576 KiB -> scale {fac:.4f}")
    out += [f"fetch_bytes_per_launch: {fetch:.4e}", f"write_bytes_per_launch: {write:.4e}",
            f"traffic_bytes_per_launch: {fetch + write:.4e}"]
    if a.algorithmic:
        out += [f"algorithmic_bytes_per_launch: {a.algorithmic}  (Q, K, V read once, O and LSE "
                f"written once)", f"traffic / algorithmic: {(fetch + write) / a.algorithmic:.3f}"]
    return "\n".join(out) + "\n"


def counters(a) -> str:
    vals, times = {}, []
    n = 0
    for d in a.dirs:
        rows = _csv(d, "counter_collection.csv")
        byc = {}
        for r in rows:
            byc.setdefault(r["Counter_Name"], []).append(r)
        for c, rs in byc.items():
            sel = _select(rs, a.kernel, a.skip, a.take)
            if sel:
                vals[c] = statistics.mean(float(r["Counter_Value"]) for r in sel)
                n = max(n, len(sel))
        try:
            tr = _select(_csv(d, "kernel_trace.csv"), a.kernel, a.skip, a.take)
            times += [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in tr]
        except SystemExit:
            pass
    out = [f"# {a.title}",
           f"command (pass 1): {a.command}",
           "further passes: the same with the counters listed below, one --pmc group per run",
           f"summary: python profile_summary.py counters --kernel {a.kernel} --skip {a.skip}",
           f"kernel_source_sha256_16: {source_digest(a.kernel)}  ({source_of(a.kernel)} + fa_common.h)",
           f"dispatches averaged per counter: {n}"]
    t = statistics.mean(times) * 1e-9 if times else None
    if t:
        out.append(f"kernel time (trace, all passes): {t * 1e3:.3f} ms")
    g = vals.get("GRBM_GUI_ACTIVE")
    if g and t:
        out.append(f"engine clock = GRBM_GUI_ACTIVE / 8 XCDs / time: {g / 8 / t / 1e9:.3f} GHz")
    if g and "SQ_VALU_MFMA_BUSY_CYCLES" in vals:
        out.append(f"matrix pipe busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 "
                   f"SIMDs): {vals['SQ_VALU_MFMA_BUSY_CYCLES'] / (g / 8 * 1024):.3f}")
    w = vals.get("SQ_WAVES")
    if w:
        per = {c: vals[c] / w for c in ("SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_LDS",
                                         "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU") if c in vals}
        out.append(f"waves: {w:.0f}; per wave: " + ", ".join(f"{c[9:] if c.startswith('SQ_INSTS_') else c} {v:.0f}"
                                                          for c, v in per.items()))
        if per.get("SQ_INSTS_MFMA"):
            m = per["SQ_INSTS_MFMA"]
            parts = []
            if "SQ_INSTS_VALU" in per:
                parts.append(f"VALU excl. MFMA {16 * (per['SQ_INSTS_VALU'] - m) / m:.1f}")
            if "SQ_INSTS_VALU_TRANS_F32" in per:
                parts.append(f"transcendental {16 * per['SQ_INSTS_VALU_TRANS_F32'] / m:.1f}")
            if "SQ_INSTS_LDS" in per:
                parts.append(f"LDS {16 * per['SQ_INSTS_LDS'] / m:.1f}")
            if "SQ_INSTS_SALU" in per:
                parts.append(f"SALU {16 * per['SQ_INSTS_SALU'] / m:.1f}")
            out.append("per 16 MFMA: " + ", ".join(parts))
    if "SQ_LDS_BANK_CONFLICT" in vals and vals.get("SQ_LDS_IDX_ACTIVE"):
        out.append(f"LDS bank conflicts / LDS active cycles: "
                   f"{vals['SQ_LDS_BANK_CONFLICT'] / vals['SQ_LDS_IDX_ACTIVE']:.4f}")
    if "SQ_WAIT_INST_LDS" in vals and vals.get("SQ_WAIT_ANY"):
        out.append(f"SQ_WAIT_INST_LDS / SQ_WAIT_ANY: {vals['SQ_WAIT_INST_LDS'] / vals['SQ_WAIT_ANY']:.3f}")
    if "SQ_ACTIVE_INST_VALU" in vals and g:
        out.append(f"VALU issue-active cycles per SIMD-cycle: "
                   f"{vals['SQ_ACTIVE_INST_VALU'] / (g / 8 * 1024):.3f}")
    if "SQ_INSTS_LDS_LOAD_BANDWIDTH" in vals and g:
        # the counter is in 64-byte units
        out.append(f"LDS read bandwidth = SQ_INSTS_LDS_LOAD_BANDWIDTH x 64 B / (GRBM_GUI_ACTIVE / 8 "
                   f"x 256 CUs): {vals['SQ_INSTS_LDS_LOAD_BANDWIDTH'] * 64 / (g / 8 * 256):.1f} "
                   f"B per clock per CU")
    if "SQ_VALU_MFMA_COEXEC_CYCLES" in vals and g:
        out.append(f"VALU and matrix pipe both busy (SQ_VALU_MFMA_COEXEC_CYCLES per SIMD-cycle): "
                   f"{vals['SQ_VALU_MFMA_COEXEC_CYCLES'] / (g / 8 * 1024):.3f}")
    out.append("raw means: " + ", ".join(f"{c}={v:.4g}" for c, v in sorted(vals.items())))
    return "\n".join(out) + "\n"


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = ap.add_subparsers(dest="what", required=True)
    for name in ("ktrace", "traffic", "counters"):
        p = sub.add_parser(name)
        p.add_argument("--kernel", required=True, help="substring of the kernel name")
        p.add_argument("--skip", type=int, default=0)
        p.add_argument("--take", type=int, default=0)
        p.add_argument("--title", required=True)
        p.add_argument("--command", required=True, help="the profiled command, for the record")
        p.add_argument("-o", "--out", required=True)
        if name == "ktrace":
            p.add_argument("--dir", required=True)
            p.add_argument("--flops", type=float, default=0.0)
            p.add_argument("--bench-json", default=None)
            p.add_argument("--also", nargs="+", default=None,
                           help="further kernels of the same step, each selected like --kernel")
        elif name == "traffic":
            p.add_argument("--fetch-dir", required=True)
            p.add_argument("--write-dir", required=True)
            p.add_argument("--algorithmic", type=int, default=0)
        else:
            p.add_argument("--dirs", nargs="+", required=True)
    a = ap.parse_args(argv)
    text = {"ktrace": ktrace, "traffic": traffic, "counters": counters}[a.what](a)
    with open(a.out, "w") as f:
        f.write(text)
    print(text, end="")


if __name__ == "__main__":
    main()
