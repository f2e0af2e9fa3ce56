"""The build's check that compiler-generated device code leaves m0 alone.

The global/buffer->LDS copies (attention_backward_amd/csrc/common.h) set m0, the LDS destination
of the copy, from inline assembly.  The compiler is told that m0 is clobbered there but may not
keep a value of its own in it across the statement, so the build refuses any kernel whose
compiler-generated code names m0.  These CPU tests check the scanner on small assembly texts and
run it over the device assembly of the current build."""
import glob
import os

import pytest

from attention_backward_amd import build

ASM_OK = """\
_ZN4attn6kernelEv:
\ts_load_dwordx2 s[0:1], s[4:5], 0x0
\t;;#ASMSTART
\ts_mov_b32 m0, s2
\ts_nop 0
\tglobal_load_lds_dwordx4 v[0:1], off
\t;;#ASMEND
\tv_mov_b32 v2, v3 ; m0 in a comment is not a use
\ts_endpgm
"""

ASM_BAD = ASM_OK.replace("\ts_endpgm\n", "\ts_mov_b32 m0, -1\n\tv_movrels_b32 v4, v5\n\ts_endpgm\n")


def test_scanner_accepts_m0_inside_inline_asm(tmp_path):
    p = tmp_path / "ok.s"
    p.write_text(ASM_OK)
    assert build.m0_outside_inline_asm(str(p)) == []


def test_scanner_flags_compiler_m0(tmp_path):
    p = tmp_path / "bad.s"
    p.write_text(ASM_BAD)
    bad = build.m0_outside_inline_asm(str(p))
    assert len(bad) == 1 and "s_mov_b32 m0, -1" in bad[0] and "_ZN4attn6kernelEv" in bad[0]


def test_current_build_has_no_compiler_m0():
    files = sorted(glob.glob(os.path.join(build.BUILD, "*.s")))
    if not files:
        pytest.skip("no device assembly under _build (the library has not been built here)")
    for f in files:
        assert build.m0_outside_inline_asm(f) == [], f
