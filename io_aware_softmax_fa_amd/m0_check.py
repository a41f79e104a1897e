"""Build-time check of the M0 register in the library's own gfx950 code.

The global -> LDS copy helpers are inline assembly that set M0 (the LDS base
address of an LDS-DMA load) and list it as clobbered. M0 is a register the
compiler reserves, so it ignores that clobber (and warns): the copies are
correct only if the compiler itself never keeps a value in M0 across them.
This module proves that on the built code object, from the disassembly of the
library's own gfx950 code:

1. every instruction that names M0 is a copy block's ``s_mov_b32 m0, sN``,
   followed by ``s_nop 0`` and the block's LDS-DMA load;
2. every LDS-DMA load (``buffer_load_* ... lds``, ``global_load_lds_*``)
   directly follows such a write, so none relies on an M0 value set elsewhere;
3. no instruction that reads M0 implicitly (relative register moves, GPR
   indexing mode, messages, GWS / ordered-count / append LDS operations,
   trace data) appears at all.

Together these say M0 is written only by the copy blocks and read only by the
load that directly follows each write, so no compiler-generated value lives in
M0 at any point. ``check_library`` raises if the built code breaks this.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

LLVM = "/opt/rocm/llvm/bin"
TARGET = "hipv4-amdgcn-amd-amdhsa--gfx950"

_IMPLICIT = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws|ds_ordered_count|ds_append|"
                       r"ds_consume|s_set_gpr_idx|s_ttracedata|v_interp)")
_DMA = re.compile(r"^(buffer_load_\w+\s.*\blds\b|global_load_lds_\w+)")
_M0_WRITE = re.compile(r"^s_mov_b32\s+m0,\s*s\d+$")
_M0 = re.compile(r"\bm0\b")


def disassemble(so_path: str) -> str:
    """gfx950 disassembly of every device code object inside ``so_path`` (the
    .hip_fatbin section holds one offload bundle per translation unit, one
    after another; each is unbundled and disassembled)."""
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", so_path],
                       check=True, capture_output=True)
        data = open(fat, "rb").read()
        starts = []
        i = data.find(magic)
        while i >= 0:
            starts.append(i)
            i = data.find(magic, i + 1)
        if not starts:
            raise RuntimeError(f"no offload bundle in {so_path}")
        out = []
        for n, (a, b) in enumerate(zip(starts, starts[1:] + [len(data)])):
            part, co = os.path.join(tmp, f"b{n}"), os.path.join(tmp, f"co{n}.elf")
            with open(part, "wb") as f:
                f.write(data[a:b])
            subprocess.run([f"{LLVM}/clang-offload-bundler", "--type=o", f"--targets={TARGET}",
                            f"--input={part}", f"--output={co}", "--unbundle"],
                           check=True, capture_output=True)
            r = subprocess.run([f"{LLVM}/llvm-objdump", "-d", "--mcpu=gfx950", co],
                               check=True, capture_output=True, text=True)
            out.append(r.stdout)
        return "\n".join(out)


def bundle_count(so_path: str) -> int:
    """Number of device code objects (translation units) in ``so_path``."""
    with tempfile.TemporaryDirectory() as tmp:
        fat = os.path.join(tmp, "fatbin")
        subprocess.run([f"{LLVM}/llvm-objcopy", f"--dump-section=.hip_fatbin={fat}", so_path],
                       check=True, capture_output=True)
        return open(fat, "rb").read().count(b"__CLANG_OFFLOAD_BUNDLE__")


def _instructions(text: str):
    """(function, instruction text) pairs in program order; comments, labels
    and blank lines dropped."""
    fn = "?"
    for line in text.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line.strip())
        if m:
            fn = m.group(1)
            continue
        if not line.startswith("\t"):
            continue
        ins = line.split("//")[0].strip()
        if ins:
            yield fn, ins


def violations(text: str) -> list[str]:
    """Instructions that break rules 1-3 above (empty when M0 is safe)."""
    bad = []
    ins = list(_instructions(text))
    for i, (fn, s) in enumerate(ins):
        if _IMPLICIT.match(s):
            bad.append(f"{fn}: implicit M0 reader: {s}")
        elif _M0.search(s):
            ok = (_M0_WRITE.match(s) and i + 2 < len(ins) and ins[i + 1][1] == "s_nop 0"
                  and _DMA.match(ins[i + 2][1]) and ins[i + 1][0] == fn == ins[i + 2][0])
            if not ok:
                bad.append(f"{fn}: M0 outside a copy block: {s}")
        elif _DMA.match(s):
            ok = (i >= 2 and ins[i - 1][1] == "s_nop 0" and _M0_WRITE.match(ins[i - 2][1])
                  and ins[i - 1][0] == fn == ins[i - 2][0])
            if not ok:
                bad.append(f"{fn}: LDS-DMA load without its own M0 write: {s}")
    return bad


def check_library(so_path: str) -> int:
    """Raise RuntimeError if the built library breaks the M0 rules; returns the
    number of copy blocks checked."""
    text = disassemble(so_path)
    bad = violations(text)
    if bad:
        raise RuntimeError("M0 check failed (the compiler uses M0 outside the copy blocks):\n  "
                           + "\n  ".join(bad[:20]))
    return sum(1 for _, s in _instructions(text) if _M0_WRITE.match(s))
