"""The fused attention kernels' device assembly, compiled with the build's
flags, has no read of a matrix-core (MFMA) result fewer wait states after the
MFMA than the hardware needs, including across loop back edges, and no
compiler use of m0 in kernels whose inline assembly sets it for LDS loads
(attention_softmax_amd.isa_check). CPU only: hipcc cross-compiles."""

import os
import shutil

import pytest

from attention_softmax_amd import build, isa_check

pytestmark = pytest.mark.skipif(not os.path.exists(build.hipcc()), reason="hipcc not installed")


def test_checker_finds_a_loop_carried_early_read():
    """A read at a loop head 3 wait states after the MFMA at the loop's end is
    found; the same read behind 8 more wait states, or after a rewrite of the
    register, is not."""
    early = """_Zk:
\tv_mov_b32 v0, 0
.LBB0_1:
\tv_accvgpr_read_b32 v20, a15
\tv_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]
\ts_add_u32 s0, s0, 1
\ts_cmp_lg_u32 s0, s1
\ts_cbranch_scc1 .LBB0_1
\ts_endpgm
.Lfunc_end0:
"""
    found = isa_check.check_text(early)
    assert list(found) == ["_Zk"] and found["_Zk"][0][2] == 3
    padded = early.replace("\ts_cbranch_scc1", "\ts_nop 7\n\ts_cbranch_scc1")
    assert not isa_check.check_text(padded)
    rewritten = early.replace("\ts_cmp_lg_u32", "\tv_mov_b32 v99, 0\n\tv_accvgpr_write_b32 a15, v99\n"
                              "\ts_cmp_lg_u32")
    assert not isa_check.check_text(rewritten)


def test_m0_checker():
    """A compiler write of m0 in a kernel whose inline assembly sets m0 is
    reported; the asm's own write, or m0 in a kernel without such asm, is not."""
    text = """_Zk:
\t;;#ASMSTART
\ts_mov_b32 m0, s4
\tbuffer_load_dwordx4 v1, s[0:3], s5 offen lds
\t;;#ASMEND
\ts_endpgm
.Lfunc_end0:
_Zj:
\ts_mov_b32 m0, s6
\ts_endpgm
"""
    assert not isa_check.m0_outside_asm(text)
    bad = text.replace("\ts_endpgm\n.Lfunc_end0", "\ts_mov_b32 m0, s7\n\ts_endpgm\n.Lfunc_end0")
    assert isa_check.m0_outside_asm(bad) == {"_Zk": ["s_mov_b32 m0, s7"]}


@pytest.mark.parametrize("src", ["attention.hip", "attention_bwd.hip"])
def test_attention_kernels_have_no_early_mfma_reads(src, tmp_path):
    out = build.device_asm(src, str(tmp_path / (src + ".s")))
    with open(out) as fh:
        text = fh.read()
    found = isa_check.check_text(text)
    assert not found, {k: v[:2] for k, v in found.items()}
    m0 = isa_check.m0_outside_asm(text)
    assert not m0, {k: v[:2] for k, v in m0.items()}
    if src == "attention_bwd.hip":  # the inline-assembly LDS loads the m0 check is about
        assert ";;#ASMSTART" in text and " offen lds" in text
    shutil.rmtree(tmp_path, ignore_errors=True)
