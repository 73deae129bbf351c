"""CPU check of the LDS-DMA kernels' global / LDS addressing.

Builds tests/native/check_dma_bounds.hip host-only (it runs the kernels' own
addressing and scheduler code on the CPU) and requires it to report every
access inside its matrix and every stage fully and exactly covered."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_dma_addressing_in_bounds(tmp_path):
    exe = str(tmp_path / "check_dma_bounds")
    subprocess.check_call(["/opt/rocm/bin/hipcc", "--cuda-host-only", "-std=c++17", "-O2",
                           "-I", os.path.join(ROOT, "include"),
                           "-I", os.path.join(ROOT, "block_swizzle_tile_amd", "csrc"),
                           os.path.join(ROOT, "tests", "native", "check_dma_bounds.hip"),
                           "-o", exe], stderr=subprocess.DEVNULL)
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0 and "ALL OK" in out.stdout, out.stdout[-2000:]
