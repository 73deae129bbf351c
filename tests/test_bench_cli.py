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
                 "--traffic-from", "--shuffle-k", "--mx-shuffle-k", "--sweep-configs",
                 "--plan-out", "--summarize", "--phases", "--wg-times"):
        assert flag in r.stdout, flag


def test_summarize_attributes_dispatches_to_settings(tmp_path, capsys):
    """--summarize: the sweep's dispatches (ours only, in dispatch order, n per setting) are
    assigned to the plan's settings, the first launch of each is dropped, and the HBM bytes
    are the counters scaled by the copy calibration."""
    import bench
    plan = {"launches_each": 3, "plan": [
        {"label": "a", "flop": 2e9, "mfma_cycles": 1e6, "alg_bytes": 1e6},
        {"label": "b", "flop": 4e9, "mfma_cycles": 2e6, "alg_bytes": 2e6}]}
    (tmp_path / "plan.json").write_text(json.dumps(plan))
    ours, other = "void bst::gemm_dma_kernel<1, 64, 64>(bst::GemmArgs)", "copy_kernel"
    # kernel trace: durations 9, 2, 2 us for "a" and 9, 4, 4 us for "b", a foreign kernel between
    tr = tmp_path / "trace"
    tr.mkdir()
    lines = ["Dispatch_Id,Kernel_Name,Start_Timestamp,End_Timestamp"]
    durs = [9000, 2000, 2000, 9000, 4000, 4000]
    for i, d in enumerate(durs):
        lines.append('%d,"%s",%d,%d' % (2 * i + 1, ours, 1000 * i, 1000 * i + d))
        lines.append('%d,"%s",0,5' % (2 * i + 2, other))
    (tr / "t_kernel_trace.csv").write_text("\n".join(lines) + "\n")

    def counters(sub, name, vals, kernel=ours):
        dd = tmp_path / sub
        dd.mkdir(exist_ok=True)
        rows = ["Dispatch_Id,Kernel_Name,Counter_Name,Counter_Value"]
        rows += ['%d,"%s",%s,%s' % (i + 1, kernel, name, v) for i, v in enumerate(vals)]
        (dd / ("%s_counter_collection.csv" % name)).write_text("\n".join(rows) + "\n")
    counters("tcc", "TCC_HIT_sum", [0, 3, 3, 0, 1, 1])
    counters("tcc", "TCC_MISS_sum", [9, 1, 1, 9, 1, 1])
    counters("tcc", "TCC_EA0_RDREQ_sum", [0, 2000, 2000, 0, 4000, 4000])
    counters("fetch", "FETCH_SIZE", [0, 500, 500, 0, 1000, 1000])
    counters("write", "WRITE_SIZE", [0, 100, 100, 0, 100, 100])
    counters("sq", "SQ_VALU_MFMA_BUSY_CYCLES", [0, 1e6, 1e6, 0, 2e6, 2e6])
    counters("sq", "SQ_LDS_BANK_CONFLICT", [0, 0, 0, 0, 0, 0])
    counters("calib_fetch", "FETCH_SIZE", [131072, 131072], kernel="copy_kernel")
    counters("calib_write", "WRITE_SIZE", [262144, 262144], kernel="copy_kernel")
    bench.summarize(str(tmp_path))
    out = capsys.readouterr().out
    rows = [l for l in out.splitlines() if l.startswith("| a ") or l.startswith("| b ")]
    a = [x.strip() for x in rows[0].split("|")[1:-1]]
    b = [x.strip() for x in rows[1].split("|")[1:-1]]
    assert a[1] == "2.00" and b[1] == "4.00"                      # median us, cold launch dropped
    assert a[2] == "1000.0" and b[2] == "1000.0"                  # TFLOP/s
    assert a[3] == "75.0" and b[3] == "50.0"                      # L2 hit %
    assert a[4] == "2" and b[4] == "4"                            # fabric read requests / 1000
    # HBM bytes: FETCH scaled by 2 (the copy read 131072 KiB of 256 MiB), WRITE by 1
    assert a[5].startswith("%.1f" % ((500 * 2 + 100) * 1024 / 1e6))
    assert a[7] == "1.000" and b[7] == "1.000"                    # MFMA busy / needed
    assert "FETCH_SIZE scale 2.0000" in out and "WRITE_SIZE scale 1.0000" in out
