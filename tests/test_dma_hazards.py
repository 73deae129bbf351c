"""CPU check of the LDS-DMA kernels' generated code for the scalar-operand hazards.

The DMA instructions are inline assembly, which the compiler's hazard pass
does not inspect.  A vector-ALU write of an SGPR (readfirstlane, a spilled
scalar reloaded with v_readlane) needs 5 wait states before a vector-memory
instruction reads that SGPR, and a write of M0 needs 1 before an LDS DMA.  A
DMA that reads a stale descriptor or offset goes to a wrong global address.
This compiles the MX-fp8 instances (the ones under the highest register
pressure) to gfx950 assembly and requires every `buffer_load ... lds` to sit
right behind an `s_nop` of at least 4."""
import os
import re
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_every_lds_dma_is_behind_five_wait_states(tmp_path):
    asm = str(tmp_path / "inst_mxfp8.s")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
                           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                           "-Wno-pass-failed", "-I", os.path.join(ROOT, "include"),
                           "--cuda-device-only", "-S",
                           os.path.join(ROOT, "block_swizzle_tile_amd", "csrc", "inst_mxfp8.hip"),
                           "-o", asm], stderr=subprocess.DEVNULL)
    lines = [l.split(";")[0].strip() for l in open(asm)]
    lines = [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]
    dmas, bad = 0, []
    for i, l in enumerate(lines):
        if l.startswith("buffer_load") and l.endswith(" lds"):
            dmas += 1
            m = re.match(r"s_nop\s+(\d+)", lines[i - 1])
            if not m or int(m.group(1)) < 4:
                bad.append((lines[i - 1], l))
    assert dmas > 100, "no LDS DMA found in the generated code"
    assert not bad, "%d DMAs without 5 wait states, e.g. %s" % (len(bad), bad[:3])
