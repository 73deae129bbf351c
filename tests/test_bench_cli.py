"""CPU checks of bench.py's host-side contract: more than one GPU is refused with a
message, the traffic summary is keyed to the kernel sources, and the measurement modes
are all reachable from the command line."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_traffic_profile_matches_the_kernel_sources():
    """bench.py reports the committed HBM traffic only while the sources hash to the value the
    counters were taken on (skipped, not failed, while they are being retaken)."""
    import pytest

    import bench
    t = json.load(open(os.path.join(ROOT, "profiles", "traffic_fp16_2k.json")))
    assert t["hbm_bytes_per_launch"] == t["fetch_bytes"] + t["write_bytes"]
    if t["kernel_hash"] != bench.kernel_source_hash():
        pytest.skip("the traffic counters predate the current kernel sources (bench reports null)")
    assert t["hbm_bytes_per_launch"] >= 10485760      # at least the algorithmic A + B + C bytes


def test_modes_are_documented_in_help():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                       capture_output=True, text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 0
    for flag in ("--all-configs", "--l2-sweep", "--large", "--clock", "--calib-copy",
                 "--traffic-from", "--shuffle-k", "--mx-shuffle-k"):
        assert flag in r.stdout, flag
