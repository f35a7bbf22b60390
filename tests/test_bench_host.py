"""Host logic of bench.py that needs no GPU: the one-GPU refusal, the HBM
traffic and counter records made from rocprofv3 CSVs (calibration, clock and
MFMA utilisation arithmetic), and the source hash that keeps a record from
being used once the kernels change."""
import csv
import json
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]


def write_csv(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.DictWriter(fh, fieldnames=FIELDS)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(FIELDS, r)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_kernel_families():
    assert bench.kernel_family("fwd") == "attention"
    assert bench.kernel_family("bwd_dkdv") == "attention"
    assert bench.kernel_family("bwd_dq_f32") == "f32"
    assert bench.kernel_family("decode") == "decode"
    assert bench.kernel_family("packed_ce") == "packed_ce"
    for fam, names in bench.KERNEL_SOURCES.items():
        for n in names:
            assert os.path.exists(os.path.join(ROOT, "long_context_blockwise_attn_amd", "csrc", n)), (fam, n)


def test_traffic_record_scales_by_the_copy(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda w: str(tmp_path / ("traffic_%s.json" % w)))
    fwd = "void bwattn::attn_fwd_kernel<128, 8, 4>(bwattn::FwdArgs)"
    copy = "void at::native::copy_kernel(...)"
    # a 1 MiB copy reads 512 KiB by FETCH_SIZE (factor 2) and writes 1024 KiB
    write_csv(tmp_path / "f.csv", [(1, fwd, "FETCH_SIZE", 1000.0, 0, 1), (2, fwd, "FETCH_SIZE", 3000.0, 0, 1),
                                   (3, copy, "FETCH_SIZE", 512.0, 0, 1)])
    write_csv(tmp_path / "w.csv", [(1, fwd, "WRITE_SIZE", 10.0, 0, 1), (2, fwd, "WRITE_SIZE", 30.0, 0, 1),
                                   (3, copy, "WRITE_SIZE", 1024.0, 0, 1)])
    bench.write_traffic_record("unit", str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), 1, "cmd")
    rec = json.load(open(tmp_path / "traffic_unit.json"))
    k = rec["kernels"]["fwd"]
    assert rec["read_calibration"]["factor"] == pytest.approx(2.0)
    assert rec["write_calibration"]["factor"] == pytest.approx(1.0)
    assert k["dispatches"] == 2
    assert k["read_bytes"] == pytest.approx(2000.0 * 1024 * 2)
    assert k["write_bytes"] == pytest.approx(20.0 * 1024)
    assert k["traffic_bytes"] == pytest.approx(2000.0 * 1024 * 2 + 20.0 * 1024)
    assert k["source_sha256"] == bench.kernel_source_hash("attention")
    # used while the sources hash the same, refused once they do not
    assert bench.load_traffic("unit", "fwd") == pytest.approx(k["traffic_bytes"])
    rec["kernels"]["fwd"]["source_sha256"] = "0" * 64
    json.dump(rec, open(tmp_path / "traffic_unit.json", "w"))
    assert bench.load_traffic("unit", "fwd") is None
    assert bench.load_traffic("missing", "fwd") is None


def test_counter_record_clock_and_utilisation(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "counters_path", lambda w: str(tmp_path / ("counters_%s.json" % w)))
    k = "void bwattn::attn_bwd_dkdv_kernel<128, 8, 2>(bwattn::BwdArgs)"
    ms = 2.0
    clock = 1.9e9
    cycles = clock * ms * 1e-3
    t0, t1 = 1_000_000, 1_000_000 + int(ms * 1e6)
    util = 0.55
    mops = 1.234e9
    write_csv(tmp_path / "p.csv", [
        (7, k, "GRBM_GUI_ACTIVE", 8 * cycles, t0, t1),
        (7, k, "SQ_VALU_MFMA_BUSY_CYCLES", util * 1024 * cycles, t0, t1),
        (7, k, "SQ_INSTS_VALU_MFMA_MOPS_BF16", mops, t0, t1)])
    bench.write_counter_record("unit", [str(tmp_path / "p.csv")], "cmd")
    rec = json.load(open(tmp_path / "counters_unit.json"))["kernels"]["bwd_dkdv"]
    assert rec["clock_ghz"] == pytest.approx(1.9)
    assert rec["mfma_util_at_clock"] == pytest.approx(util)
    out = bench.load_counters("unit", "bwd_dkdv", ms, 2516.6)
    assert out["mfma_flops_per_launch"] == pytest.approx(512 * mops)
    assert out["mfma_tflops"] == pytest.approx(512 * mops / (ms * 1e-3) / 1e12)
    assert out["clock_ghz"] == pytest.approx(1.9)


def test_source_hash_follows_the_sources(tmp_path, monkeypatch):
    pkg = tmp_path / "long_context_blockwise_attn_amd"
    shutil.copytree(os.path.join(ROOT, "long_context_blockwise_attn_amd", "csrc"), pkg / "csrc")
    shutil.copy(os.path.join(ROOT, "long_context_blockwise_attn_amd", "build.py"), pkg / "build.py")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    before = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    with open(pkg / "csrc" / "attn_fwd.hip", "a") as fh:
        fh.write("\n// edited\n")
    after = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    assert after["attention"] != before["attention"]
    assert after["decode"] == before["decode"] and after["packed_ce"] == before["packed_ce"]
    with open(pkg / "csrc" / "tile.hpp", "a") as fh:
        fh.write("\n// edited\n")
    again = {f: bench.kernel_source_hash(f) for f in bench.KERNEL_SOURCES}
    assert again["f32"] != after["f32"] and again["decode"] != after["decode"]
    assert again["packed_ce"] == after["packed_ce"]
