"""Generated-code check of the LM-head kernel (CPU: hipcc cross-compiles).

The kernel's weight loads are inline asm with explicit waits: the compiler
takes an asm output as written at once, so a register copy it placed between
such a load and its wait would copy a value that has not landed.  The block
loop must therefore move no registers at all; this compiles lm_head.hip for
gfx950 and checks that every block of the loop is free of copies.
"""

import os
import re
import shutil
import subprocess

import pytest

from speculative_decoding_sampling_amd import build as B

# register moves, whatever their encoding suffix (_e32, _e64, _dpp, ...)
COPY = re.compile(r"^\s*(v_mov_b32|v_mov_b64|v_accvgpr_mov_b32|v_accvgpr_read_b32|"
                  r"v_accvgpr_write_b32|v_pk_mov_b32)(_\w+)?\s")


def loop_blocks(asm, kernel):
    """Instruction lines of the blocks LLVM marks as part of a loop of ``kernel``."""
    start = asm.index("\n" + kernel + ":")
    body = asm[start:asm.index("s_endpgm", start)]
    lines, in_loop = [], False
    for line in body.splitlines():
        if re.match(r"^(\.LBB\d+_\d+:|; %bb\.\d+:)", line):
            in_loop = "Loop Header" in line or "in Loop:" in line
        elif in_loop and line.startswith("\t") and not line.lstrip().startswith(";"):
            lines.append(line)
    return lines


def test_lm_head_block_loop_copies_no_registers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available")
    out = tmp_path / "lm_head.s"
    subprocess.run([hipcc, *B.FLAGS, "--cuda-device-only", "-S",
                    os.path.join(B.CSRC, "lm_head.hip"), "-o", str(out)],
                   check=True, capture_output=True)
    asm = out.read_text()
    name = re.search(r"^(_ZN5specv14lm_head_kernel\S*):", asm, re.M).group(1)
    loop = loop_blocks(asm, name)
    n_mfma = sum("v_mfma_f32_32x32x16_bf16" in l for l in loop)
    assert n_mfma == 120, n_mfma            # three unrolled k blocks of 40 MFMAs: the block loop
    copies = [l.strip() for l in loop if COPY.match(l)]
    assert not copies, copies[:8]
