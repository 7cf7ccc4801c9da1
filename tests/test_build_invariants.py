"""Checks on the gfx950 assembly of the quantizers that build() keeps in
nvfp4_bit_block_amd/_build/quantize.hip.s (CPU only).

The one-instruction cross-lane butterfly is inline assembly (v_fmac_f32_dpp)
preceded by s_nop 1: the two wait states a DPP read needs after a vector
write of its source register.  After a vector-ALU write of EXEC (v_cmpx) it
would need five; the compiler's hazard recognizer does not see inside inline
assembly, so the library must contain no v_cmpx at all.
"""
import os
import re

import pytest

ASM = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "nvfp4_bit_block_amd", "_build",
                   "quantize.hip.s")


@pytest.fixture(scope="module")
def asm():
    if not os.path.exists(ASM):
        pytest.skip("no build: run __graft_entry__.build()")
    return open(ASM).read()


def test_no_vector_exec_writes(asm):
    assert "v_cmpx" not in asm


def test_every_dpp_fmac_block_waits(asm):
    lines = [l.strip() for l in asm.splitlines()]
    starts = 0
    for i, l in enumerate(lines):
        if l.startswith("v_fmac_f32_dpp") and not lines[i - 1].startswith("v_fmac_f32_dpp"):
            starts += 1
            assert re.match(r"s_nop [1-9]", lines[i - 1]), f"DPP block without wait states at line {i}"
    assert starts > 0
