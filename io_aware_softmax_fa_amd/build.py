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


def build(verbose: bool = False, extra=()) -> str:
    """Compile the library; returns its path. Raises on a compiler error."""
    tmp = OUT + ".tmp"
    cmd = command(tmp, extra)
    if verbose:
        print(" ".join(shlex.quote(c) for c in cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # known noise: hipcc's host pass does not know the packed-fp32 feature; the
    # copy helper lists m0 (the only code that writes m0) among its clobbers
    noise = ("is not a recognized feature for this target", "contains reserved registers: m0",
             "Reserved registers on the clobber list", "global_load_lds_dwordx4 %0",
             "buffer_load_dwordx4 %0", "buffer_load_dword %0", "In file included from",
             "      |                ^", "warnings generated")
    err = "\n".join(l for l in r.stderr.splitlines() if not any(n in l for n in noise))
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    # a host pass that silently drops kernel stubs leaves undefined symbols:
    # load the new library in a separate process before installing it
    chk = subprocess.run([sys.executable, "-c", "import ctypes, sys; ctypes.CDLL(sys.argv[1])", tmp],
                         capture_output=True, text=True)
    if chk.returncode != 0:
        raise RuntimeError(f"built library does not load:\n{chk.stderr.strip()}")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
