"""Host-side parts of bench.py (no GPU): the one-GPU rule and the byte-counter arithmetic behind
roofline.traffic."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr


def _counter_csv(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for name, value in rows:
            w.writerow({"Kernel_Name": name, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_summary_scales_each_counter_by_the_copy_kernel(tmp_path):
    """A copy of 1 GiB that FETCH_SIZE counts as 512 MiB and WRITE_SIZE as 1 GiB gives read scale 2
    and write scale 1; the attention kernel's medians are scaled by those and summed."""
    calib_kib = bench.COPY_CALIB_BYTES / 1024
    attn = bench.ATTN_KERNEL + "(pbsa::AttnArgs)"
    fetch = tmp_path / "f.csv"
    write = tmp_path / "w.csv"
    _counter_csv(fetch, "FETCH_SIZE", [(attn, 1000.0), (attn, 1200.0), (attn, 1100.0),
                                       ("__amd_rocclr_copyBuffer", calib_kib / 2), ("__amd_rocclr_copyBuffer", 10.0)])
    _counter_csv(write, "WRITE_SIZE", [(attn, 500.0), (attn, 500.0), ("__amd_rocclr_copyBuffer", calib_kib)])
    out = tmp_path / "traffic.txt"
    assert bench.summarize_pmc(str(fetch), str(write), str(out), "cmd") == 0
    vals = {}
    for line in open(out):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    assert float(vals["fetch_scale"]) == pytest.approx(2.0)
    assert float(vals["write_scale"]) == pytest.approx(1.0)
    # medians 1100 KiB read and 500 KiB written -> (1100 * 2 + 500 * 1) KiB
    assert float(vals["traffic_bytes_per_launch"]) == pytest.approx((1100 * 2 + 500) * 1024, rel=1e-5)
    assert vals["kernel_source_sha256_16"] == bench.kernel_source_hash()


def test_committed_traffic_summary_matches_the_kernel_sources():
    """The committed counter summary was taken on the attention source as it stands (else bench.py
    reports traffic as null)."""
    assert bench.read_traffic() is not None


def test_sq_summary_sums_counters_per_kernel(tmp_path):
    """Counters of two dispatches of one kernel are summed; the ratios are those sums' quotients."""
    path = tmp_path / "sq.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for disp in (1, 2):
            for name, val in (("SQ_INSTS_MFMA", 100.0), ("SQ_INSTS_VALU", 550.0), ("SQ_INSTS_LDS", 150.0),
                              ("SQ_WAIT_INST_ANY", 40.0), ("SQ_WAVE_CYCLES", 100.0)):
                w.writerow({"Dispatch_Id": disp, "Kernel_Name": "void pbsa::k<1>(pbsa::AttnArgs)",
                            "Counter_Name": name, "Counter_Value": val})
    out = tmp_path / "sq.txt"
    assert bench.summarize_sq([("one run", str(path))], str(out), ["cmd a", "cmd b"]) == 0
    text = out.read_text()
    assert "#   cmd a" in text and "## one run" in text
    line = [l for l in text.splitlines() if l.startswith("k<1>")][0].split()
    assert line[1] == "2" and float(line[2]) == 200.0 and float(line[3]) == 1100.0
    assert line[5] == "5.50" and line[6] == "1.50" and line[7] == "40.0%"
