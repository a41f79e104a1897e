"""Compile the HIP sources into the in-tree shared library ``libfa_fwd.so``.

Usage: ``python -m io_aware_softmax_fa_amd.build`` (also called by the
repository's ``__graft_entry__.build()``). Cross-compiles for gfx950 with
hipcc; no GPU is needed to build.
"""
from __future__ import annotations

import os
import shlex
import subprocess
import sys

if __package__:
    from . import m0_check
else:  # run as a script
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from io_aware_softmax_fa_amd import m0_check

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRCS = [os.path.join(PKG, "csrc", n) for n in ("fa_fwd.hip", "fa_bwd.hip", "fa_quant.hip")]
OUT = os.path.join(PKG, "libfa_fwd.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed fp32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-instruction results in VGPRs unless registers run out: the
    # backward's score-shaped accumulators are read by VALU instructions
    # (the forward kernels compile to the same code either way)
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-I", os.path.join(ROOT, "include"),
]


def command(out: str = OUT, extra=()) -> list[str]:
    return [HIPCC, *FLAGS, *extra, *SRCS, "-o", out]


def build(verbose: bool = False, extra=(), out: str = OUT) -> str:
    """Compile the library to ``out``; returns its path. Raises on a compiler
    error."""
    tmp = out + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    # hipcc's host pass does not know the packed-fp32 feature (harmless)
    lines = [l for l in r.stderr.splitlines()
             if "is not a recognized feature for this target" not in l]
    # The copy helpers list the reserved register m0 as clobbered, and the
    # compiler warns about each inlined copy. Those warnings are counted and
    # reported in one line below, together with the check (m0_check) that the
    # built code never holds a compiler value in M0; every other warning is
    # printed in full.
    m0_warn = sum("Reserved registers on the clobber list" in l for l in lines)
    m0_ctx = ("contains reserved registers: m0", "Reserved registers on the clobber list",
              "global_load_lds_dwordx4 %0", "buffer_load_dwordx4 %0", "buffer_load_dword %0",
              "In file included from", "      |                ^", "warnings generated",
              "warning generated")
    other = "\n".join(l for l in lines if not any(n in l for n in m0_ctx))
    if other.strip():
        print(other, file=sys.stderr)
    # a host pass that silently drops kernel stubs leaves undefined symbols:
    # load the new library in a separate process before installing it
    chk = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1])", tmp],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        raise RuntimeError(f"built library does not load:\n{chk.stderr.strip()}")
    blocks = m0_check.check_library(tmp)
    print(f"{m0_warn} compiler warnings name the reserved register m0 (clobber lists of the "
          f"inline-asm global->LDS copies); M0 check of the built gfx950 code passed: M0 is "
          f"written only by the {blocks} copy blocks and read only by each block's own load",
          file=sys.stderr)
    os.replace(tmp, out)
    return out


PROBE_SRC = os.path.join(PKG, "csrc", "mfma_probe.hip")
PROBE_OUT = os.path.join(PKG, "libfa_probe.so")


def build_probe(verbose: bool = False) -> str:
    """Compile the matrix-pipe ceiling probe (a measurement tool for bench.py,
    not part of the attention library) to ``libfa_probe.so``."""
    cmd = [HIPCC, *FLAGS, PROBE_SRC, "-o", PROBE_OUT + ".tmp"]
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{r.stderr}")
    os.replace(PROBE_OUT + ".tmp", PROBE_OUT)
    return PROBE_OUT


def variant_path(every: int) -> str:
    """The measurement variant whose f16/bf16 kernels take every ``every``-th
    exponential in software (FA_SWEXP2_EVERY); load it with FA_LIBRARY."""
    return os.path.join(PKG, f"libfa_fwd_swexp2_{every}.so")


if __name__ == "__main__":
    import argparse
    ap = argparse.ArgumentParser(description="build libfa_fwd.so (gfx950)")
    ap.add_argument("--swexp2-every", type=int, default=0,
                    help="build the software-exp2 measurement variant instead "
                         "(every k-th exponential on the FMA pipe) as libfa_fwd_swexp2_<k>.so")
    a = ap.parse_args()
    if a.swexp2_every > 0:
        print(build(verbose=True, extra=(f"-DFA_SWEXP2_EVERY={a.swexp2_every}",),
                    out=variant_path(a.swexp2_every)))
    else:
        print(build(verbose=True))
        print(build_probe(verbose=True))
