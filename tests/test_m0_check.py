"""The build-time M0 check (io_aware_softmax_fa_amd.m0_check): it passes on
the built library, and it flags each way the compiler could use M0 next to
the inline-asm copies (planted in synthetic disassembly)."""
import os

import pytest

from io_aware_softmax_fa_amd import _lib, m0_check

BLOCK = ["\ts_mov_b32 m0, s35", "\ts_nop 0", "\tbuffer_load_dwordx4 v103, s[8:11], 0 offen nt lds"]
GBLOCK = ["\ts_mov_b32 m0, s2", "\ts_nop 0", "\tglobal_load_lds_dwordx4 v5, s[0:1]"]


def dis(*body):
    return "\n".join(["0000000000001000 <kern>:", *body, "\ts_endpgm"]) + "\n"


@pytest.mark.skipif(not os.path.exists(_lib.LIB_PATH), reason="library not built")
def test_built_library_passes():
    """Every translation unit's code object is checked (one offload bundle per
    HIP source), and the check passes."""
    from io_aware_softmax_fa_amd import build
    assert m0_check.bundle_count(_lib.LIB_PATH) == len(build.SRCS)
    text = m0_check.disassemble(_lib.LIB_PATH)
    for kernel in ("fa_fwd_kernel", "fa_fwd16_kernel", "fa_fwd_fp8_kernel", "bwd_dkdv", "bwd_dq",
                   "fa_quant_kernel"):
        assert kernel in text, kernel
    assert m0_check.check_library(_lib.LIB_PATH) > 0


def test_clean_blocks_pass():
    assert m0_check.violations(dis(*BLOCK, "\tv_add_u32_e32 v2, s15, v98", *GBLOCK)) == []


@pytest.mark.parametrize("body", [
    ["\ts_mov_b32 m0, -1", "\tds_read_b128 v[0:3], v1"],                 # compiler sets M0
    [*BLOCK, "\tv_readlane_b32 s4, v1, m0"],                             # compiler reads M0
    ["\ts_nop 0", "\tbuffer_load_dwordx4 v1, s[8:11], 0 offen lds"],    # DMA on a stale M0
    [*BLOCK[:1], "\tv_mov_b32_e32 v1, 0", *BLOCK[2:]],                   # block split apart
    ["\tv_movrels_b32_e32 v1, v2"],                                       # implicit reader
    ["\ts_set_gpr_idx_on s2, gpr_idx(SRC0)"],                             # GPR indexing mode
    ["\ts_sendmsg sendmsg(MSG_INTERRUPT)"],                               # message
])
def test_planted_m0_uses_are_flagged(body):
    assert m0_check.violations(dis(*body))
