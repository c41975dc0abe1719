"""bench.py host logic on the CPU: the one-GPU guard and the counter
summary that turns rocprofv3 FETCH_SIZE / WRITE_SIZE rows into HBM bytes."""
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BENCH = os.path.join(ROOT, "bench.py")


def test_more_than_one_gpu_is_refused():
    # Every mode (decode, MLP, MLP sweep, router, decode step) measures one GPU.
    for extra in ([], ["--mlp", "opt66b_mlp_bf16"], ["--mlp", "opt66b_mlp_bf16", "--mlp-sweep"],
                  ["--router", "opt66b_f16"], ["--decode-step", "2"]):
        r = subprocess.run([sys.executable, BENCH, "--gpus", "2"] + extra, capture_output=True,
                           text=True, timeout=300)
        assert r.returncode == 2, extra
        assert "one GPU" in r.stderr


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_summarize_traffic_scales_by_the_copy(tmp_path):
    k = "void sha::(anonymous namespace)::sha_decode_mha_kernel<1, 128, 4, 8, 0>(sha::Args)"
    cp = "__amd_rocclr_copyBuffer"
    # decode: 1000 KiB fetched, 10 KiB written per launch; the 1 GiB copy
    # reads as 524288 KiB fetched (half) and 1048576 KiB written.
    _write_counters(tmp_path / "f.csv", [dict(Kernel_Name=k, Grid_Size=360448,
                                              Counter_Name="FETCH_SIZE", Counter_Value=v)
                                         for v in (990, 1010)])
    _write_counters(tmp_path / "w.csv", [dict(Kernel_Name=k, Grid_Size=360448,
                                              Counter_Name="WRITE_SIZE", Counter_Value=10)])
    _write_counters(tmp_path / "cf.csv", [dict(Kernel_Name=cp, Grid_Size=1, Counter_Name="FETCH_SIZE",
                                               Counter_Value=524288)])
    _write_counters(tmp_path / "cw.csv", [dict(Kernel_Name=cp, Grid_Size=1, Counter_Name="WRITE_SIZE",
                                               Counter_Value=1048576)])
    out = tmp_path / "traffic.json"
    r = subprocess.run([sys.executable, BENCH, "--summarize-traffic", "--workload", "opt66b_f16",
                        "--fetch-csv", str(tmp_path / "f.csv"), "--write-csv", str(tmp_path / "w.csv"),
                        "--copy-fetch-csv", str(tmp_path / "cf.csv"),
                        "--copy-write-csv", str(tmp_path / "cw.csv"), "--traffic-out", str(out)],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    rec = json.loads(out.read_text())
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    assert rec["hbm_read_bytes_per_launch"] == 1000 * 1024 * 2
    assert rec["hbm_write_bytes_per_launch"] == 10 * 1024
    assert rec["algorithmic_bytes_per_launch"] == 1408 * 2 * 1920 * 128 * 2
