"""bench.py's host-side arithmetic, on the CPU: the algorithmic byte and element counts of
each stage on a list small enough to count by hand, the reduction of rocprofv3 CSVs into the
traffic record, and the refusal of more than one GPU."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes_by_hand():
    # numels 5, 8, 3 at Nd = 4: padded 8, 8, 4; shards 2, 2, 1; the 8-element one has no grad
    numels, shards, live, nd = [5, 8, 3], [2, 2, 1], [1, 0, 1], 4
    ab = bench.algorithmic_bytes(numels, shards, live, nd)
    # pack: live grads 5 + 3 = 8 elements read, padded 8 + 4 = 12 written, 2 B each
    assert ab["pack"] == 2 * 8 + 2 * 12
    # live shard elements 2 + 1 = 3: reduce reads 4 rows of 2 B and writes 4 B
    assert ab["shard_live"] == 3 and ab["reduce"] == 3 * (4 * 2 + 4)
    # Adam: g, p, m, v read (16 B), p, m, v, 16-bit param written (14 B)
    assert ab["adam"] == 3 * 30
    # fused: rows in place of g32 (4 x 2 B), p, m, v read, 14 B written
    assert ab["reduce_adam"] == 3 * (4 * 2 + 12 + 14)
    # unpack: every parameter's 16 elements, 2 B read + 2 B written
    assert ab["unpack"] == 16 * 4
    ne = bench.stage_elements(ab)
    assert ne == {"pack": 8, "reduce": 3, "adam": 3, "reduce_adam": 3, "unpack": 16}


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(header)
        wr.writerows(rows)


def test_summarize_profiles_scales_by_copy(tmp_path, monkeypatch):
    """A copy kernel that reads half the known 2 GiB in FETCH_SIZE (the under-count seen on the
    device) sets a fetch factor of 2; the pack kernel's KiB are scaled by it."""
    root = tmp_path / "prof"
    pack = "void zs::pack_kernel<(zs::Dt)0, false>(zs::PackArgs)"
    copy = "elementwise_kernel copy_ 2GiB"
    _write_csv(str(root / "trace" / "x" / "k_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [[pack, 4, 4000, 1000, 60.0, 900, 1100], [copy, 1, 2000, 2000, 40.0, 2000, 2000]])
    kib = 2 * 1024 * 1024
    _write_csv(str(root / "FETCH_SIZE" / "x" / "c_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[copy, "FETCH_SIZE", kib / 2], [pack, "FETCH_SIZE", 100.0], [pack, "FETCH_SIZE", 300.0]])
    _write_csv(str(root / "WRITE_SIZE" / "x" / "c_counter_collection.csv"),
               ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[copy, "WRITE_SIZE", kib], [pack, "WRITE_SIZE", 50.0], [pack, "WRITE_SIZE", 50.0]])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    text = bench.summarize_profiles(str(root), "toy", "rocprofv3 ... -- python3 bench.py")
    assert "| pack | 4 |" in text
    rec = json.loads(out.read_text())["toy"]["pack"]
    # mean FETCH 200 KiB x 2 + mean WRITE 50 KiB x 1
    assert rec["bytes_per_launch"] == int(200 * 1024 * 2.0 + 50 * 1024)
    assert rec["dispatches"] == 2 and rec["source_hash"] == bench.kernel_source_hash()


def test_more_than_one_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
    assert r.stdout == ""


def test_summarize_trace_only(tmp_path, monkeypatch):
    """A directory with only a kernel trace gives the kernel-time table and leaves the traffic
    record untouched."""
    root = tmp_path / "prof"
    _write_csv(str(root / "trace" / "x" / "k_kernel_stats.csv"),
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [["void zs::adam_kernel<1, 8>(zs::DevPlan, zs::AdamArgs, long)", 3, 3_000_000, 1_000_000, 100.0,
                 990_000, 1_010_000]])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    text = bench.summarize_profiles(str(root), "toy", "rocprofv3 --kernel-trace --stats -- python3 bench.py")
    assert "| adam | 3 | 1000.0 |" in text and "HBM traffic" not in text
    assert not out.exists()
