"""CPU check of the LDS-DMA kernels' generated code for the scalar-operand hazards.

The DMA instructions are inline assembly, which the compiler's hazard pass
does not inspect.  A vector-ALU write of an SGPR (readfirstlane, a spilled
scalar reloaded with v_readlane) needs 5 wait states before a vector-memory
instruction reads that SGPR, and a write of M0 needs 1 before an LDS DMA.  A
DMA that reads a stale descriptor or offset goes to a wrong global address.
Every translation unit that instantiates the DMA kernels (one per operand
type, each with its matmul-add instances) is checked: every
`buffer_load ... lds` must sit right behind an `s_nop` of at least 4.

The gfx950 code comes from this repository's own build: the device code
object inside each `_build/*.o` (when the object is newer than every source
it depends on), disassembled with llvm-objdump; otherwise the translation
unit is compiled to gfx950 assembly here."""
import os
import re
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_swizzle_tile_amd", "csrc")
OBJ = os.path.join(ROOT, "block_swizzle_tile_amd", "_build")
LLVM = "/opt/rocm/llvm/bin"
TUS = ["inst_f16.hip", "inst_bf16.hip", "inst_i8.hip", "inst_fp8.hip", "inst_mxfp8.hip",
       "inst_slicek.hip"]
DEPS = [os.path.join(CSRC, f) for f in os.listdir(CSRC)] + [os.path.join(ROOT, "include", "bst.h")]


def _fresh(obj):
    return os.path.exists(obj) and all(os.path.getmtime(obj) >= os.path.getmtime(d) for d in DEPS)


def _code_lines(tu, tmp):
    """The gfx950 instructions of one translation unit, comments stripped."""
    obj = os.path.join(OBJ, tu.replace(".hip", ".o"))
    if _fresh(obj):
        work = os.path.join(tmp, tu + ".d")
        os.makedirs(work, exist_ok=True)
        local = os.path.join(work, os.path.basename(obj))
        shutil.copy(obj, local)
        subprocess.check_call([os.path.join(LLVM, "llvm-objdump"), "--offloading", local],
                              cwd=work, stdout=subprocess.DEVNULL)
        co = [f for f in os.listdir(work) if "amdgcn" in f and "gfx950" in f]
        assert len(co) == 1, co
        text = subprocess.check_output([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950",
                                        os.path.join(work, co[0])], text=True)
    else:
        asm = os.path.join(tmp, tu + ".s")
        subprocess.check_call(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O3", "-std=c++17",
                               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                               "-Wno-pass-failed", "-I", os.path.join(ROOT, "include"),
                               "--cuda-device-only", "-S", os.path.join(CSRC, tu), "-o", asm],
                              stderr=subprocess.DEVNULL)
        text = open(asm).read()
    out = []
    for l in text.splitlines():
        l = l.split("//")[0].split(";")[0].strip()
        if not l or l.startswith((".", "<", "Disassembly")) or l.endswith(":"):
            continue
        out.append(l)
    return out


@pytest.fixture(scope="module")
def code(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("dma_hazards"))
    with ThreadPoolExecutor(len(TUS)) as ex:
        return dict(zip(TUS, ex.map(lambda tu: _code_lines(tu, tmp), TUS)))


@pytest.mark.parametrize("tu", TUS)
def test_every_lds_dma_is_behind_five_wait_states(code, tu):
    lines = code[tu]
    dmas, bad = 0, []
    for i, l in enumerate(lines):
        if l.startswith("buffer_load") and l.endswith(" lds"):
            dmas += 1
            m = re.match(r"s_nop\s+(\d+)", lines[i - 1])
            if not m or int(m.group(1)) < 4:
                bad.append((lines[i - 1], l))
    assert dmas > 100, "no LDS DMA found in the generated code of %s" % tu
    assert not bad, "%s: %d DMAs without 5 wait states, e.g. %s" % (tu, len(bad), bad[:3])
