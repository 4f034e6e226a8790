"""Host logic of bench.py (no GPU): the committed rocprofv3 summaries belong to the
current kernel sources, the trace and counter readers do their arithmetic, and
more than one GPU is refused."""
import csv
import glob
import json
import os
import subprocess
import sys

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_committed_profiles_match_the_kernel_sources():
    """Every committed kernel-time and traffic summary was taken on the kernel
    sources in the tree (bench.py drops stale ones from its line, so a stale
    file would silently turn the reported traffic into null)."""
    sha = bench.kernel_source_hash()
    files = sorted(glob.glob(os.path.join(ROOT, "profiles", "kernel_time_*.json")) +
                   glob.glob(os.path.join(ROOT, "profiles", "traffic_*.json")))
    assert files
    for path in files:
        with open(path) as f:
            assert json.load(f)["kernel_source_sha"] == sha, path
    for path in glob.glob(os.path.join(ROOT, "profiles", "*_kernel_*.md")):
        with open(path) as f:
            assert f"Kernel sources hash {sha}" in f.read(), path
    # the default bench workload has both
    assert bench.counted_traffic("long") is not None
    assert bench.profiled_kernel_time("long") is not None


def _write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def _into(tmp_path, monkeypatch):
    """Point bench.py's profile writers at an empty folder."""
    sha = bench.kernel_source_hash()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: sha)
    os.makedirs(tmp_path / "profiles")


def test_kernel_time_adds_the_following_merge_dispatch(tmp_path, monkeypatch):
    """A decode dispatch followed by the split merge's own dispatch counts from the
    decode's start to the merge's end; one with no merge after it counts alone."""
    _into(tmp_path, monkeypatch)
    dec = "void gqa::paged_decode_kernel<128, 16, 16, 0, 8>(int const*)"
    mrg = "void gqa::merge_splits_kernel<128>(float const*)"
    rows = [[dec, 1_000, 11_000], [mrg, 12_000, 14_000],      # 13 us with its merge
            ["void other_kernel()", 15_000, 16_000],
            [dec, 20_000, 30_000],                              # 10 us, no merge after it
            [dec, 40_000, 49_000], [mrg, 50_000, 52_000]]       # 12 us
    _write_csv(str(tmp_path / "trace" / "run_kernel_trace.csv"),
               ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], rows)
    bench.write_kernel_time("verify4", str(tmp_path / "trace"), 35_000_000)
    with open(tmp_path / "profiles" / "kernel_time_verify4.json") as f:
        out = json.load(f)
    assert out["dispatches"] == 3
    assert out["min_us"] == 10.0 and out["max_us"] == 13.0 and out["p50_us"] == 12.0
    assert out["avg_us"] == pytest.approx(35.0 / 3, abs=1e-3)
    assert out["achieved_gbs_avg"] == pytest.approx(35e6 / (out["avg_us"] * 1e-6) / 1e9, abs=0.01)
    assert "merge_splits_kernel" in out["kernel"]


def test_traffic_scales_each_counter_by_the_copy_calibration(tmp_path, monkeypatch):
    """Counters are KiB per dispatch; each is scaled so that the calibration copy
    reads its known byte count, and the merge launch's median is added."""
    _into(tmp_path, monkeypatch)
    dec = "void gqa::paged_decode_kernel<128, 32, 8, 0, 4>(int const*)"
    mrg = "void gqa::merge_splits_kernel<128>(float const*)"
    copy = "void at::native::vectorized_elementwise_kernel<4, add>(int)"
    fill = "void at::native::vectorized_elementwise_kernel<4, FillFunctor<float>>(int)"
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    copy_kib = bench.COPY_BYTES / 1024
    for counter, sub, cal_factor, dec_kib, mrg_kib in (("FETCH_SIZE", "fetch", 0.5, 1000.0, 10.0),
                                                       ("WRITE_SIZE", "write", 1.0, 40.0, 2.0)):
        _write_csv(str(tmp_path / "pmc" / f"copy_{sub}" / "run_counter_collection.csv"), hdr,
                   [[1, fill, counter, 17.0], [2, copy, counter, copy_kib * cal_factor],
                    [3, copy, counter, copy_kib * cal_factor]])
        _write_csv(str(tmp_path / "pmc" / sub / "run_counter_collection.csv"), hdr,
                   [[1, dec, counter, dec_kib], [2, mrg, counter, mrg_kib],
                    [3, dec, counter, dec_kib * 3], [4, mrg, counter, mrg_kib],
                    [5, dec, counter, dec_kib]])
    bench.write_traffic("verify4", str(tmp_path / "pmc"), 4_000_000)
    with open(tmp_path / "profiles" / "traffic_verify4.json") as f:
        out = json.load(f)
    fetch = (1000.0 + 10.0) * 1024 / 0.5            # medians, scaled by 1 / 0.5
    write = (40.0 + 2.0) * 1024 / 1.0
    assert out["FETCH_SIZE"]["scale"] == pytest.approx(2.0)
    assert out["WRITE_SIZE"]["scale"] == pytest.approx(1.0)
    assert out["hbm_bytes_per_call"] == round(fetch + write)
    assert out["traffic_over_algorithmic"] == pytest.approx((fetch + write) / 4_000_000, rel=1e-6)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300,
                       env={**os.environ, "HIP_VISIBLE_DEVICES": ""})
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr
    assert r.stdout == ""
