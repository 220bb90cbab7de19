"""Host-side logic of the benchmark and of the rocprofv3 summaries (CPU only): the
one-GPU refusal, the copy-calibrated traffic arithmetic on synthetic counter files,
the source-hash gate on stored traffic, and the workload definitions."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
from rank_gradient_compression_amd import rocprof_summary as rs
from synthetic import CONFIGS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), ([], {"WORLD_SIZE": "4"})])
def test_bench_refuses_more_than_one_gpu(argv, env):
    e = dict(os.environ, **env)
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv], env=e,
                       capture_output=True, text=True, timeout=120)
    assert p.returncode == 2
    assert "one GPU" in p.stderr
    assert p.stdout == ""


def _write_counters(path, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for name, val in rows:
            w.writerow({"Kernel_Name": name, "Grid_Size": 1024, "Counter_Name": "X",
                        "Counter_Value": val})


def test_traffic_is_scaled_by_the_copy_calibration(tmp_path):
    fetch, write = tmp_path / "f", tmp_path / "w"
    fetch.mkdir()
    write.mkdir()
    kern = "void psgd::kern::k_pass1<2, 4, false, true, 0>(psgd::Pass1Args)"
    copy = "__amd_rocclr_copyBuffer"
    # a 2 GiB copy reads as 1 GiB of FETCH_SIZE (factor 2) and 2 GiB of WRITE_SIZE
    # (factor 1); small copies are ignored by the calibration
    _write_counters(fetch / "run_counter_collection.csv",
                    [(kern, 1000.0), (kern, 3000.0), (copy, 1048576.0), (copy, 1048000.0),
                     (copy, 12.0)])
    _write_counters(write / "run_counter_collection.csv",
                    [(kern, 500.0), (kern, 700.0), (copy, 2097152.0), (copy, 5.0)])
    t = rs.traffic(str(fetch), str(write), "pass1_mq")
    f_k, f_n, f_cal, f_cn, _ = t["FETCH_SIZE"]
    assert (f_k, f_n, f_cn) == (2000.0, 2, 2) and f_cal == pytest.approx(1048288.0)
    rep = rs.traffic_report(str(fetch), str(write), "pass1_mq", "w", 2 ** 31, "cf", "cw")
    vals = dict(line.split(": ", 1) for line in rep.splitlines() if ": " in line
                and not line.startswith("#"))
    f_factor = 2 ** 31 / (1048288.0 * 1024)
    w_factor = 2 ** 31 / (2097152.0 * 1024)
    want = 2000.0 * 1024 * f_factor + 600.0 * 1024 * w_factor
    assert abs(float(vals["hbm_bytes_per_launch"]) - want) <= 0.5  # printed in whole bytes
    assert vals["source_hash"] == rs.source_hash()


def test_stored_traffic_is_used_only_for_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    body = "kernel_kind: pass1_mq\nhbm_bytes_per_launch: 12345\n"
    (prof / "traffic_pass1_mq_wl.txt").write_text(f"source_hash: {rs.source_hash()}\n" + body)
    assert bench.load_traffic("pass1_mq", "wl") == 12345.0
    (prof / "traffic_pass1_mq_wl.txt").write_text("source_hash: 0000000000000000\n" + body)
    assert bench.load_traffic("pass1_mq", "wl") is None
    assert bench.load_traffic("pass1_mq", "other") is None


def test_workload_definitions():
    names = [c.name for c in CONFIGS.values()]
    assert len(set(names)) == len(names)
    for c in CONFIGS.values():
        views = c.views()
        off = 0
        for o, shp in views:  # packed back to back in the listed order
            assert o == off
            off += int(np.prod(shp))
        assert off == c.numel
        assert c.wrap in ("", "f16", "bf16")
        assert c.grad_scale > 0 and np.log2(c.grad_scale) == int(np.log2(c.grad_scale))
        assert not (c.wrap and c.dtype != "f32")


def test_mfma_summary_and_its_hash_gate(tmp_path, monkeypatch):
    util, mops = tmp_path / "u", tmp_path / "m"
    util.mkdir()
    mops.mkdir()
    kern = "void psgd::kern::k_pass2_mfma<32, false, true, 2>(psgd::Pass2Args)"

    def write(path, rows):
        with open(path / "run_counter_collection.csv", "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Grid_Size", "Counter_Name",
                                              "Counter_Value"])
            w.writeheader()
            for name, c, v in rows:
                w.writerow({"Kernel_Name": name, "Grid_Size": 1, "Counter_Name": c,
                            "Counter_Value": v})

    write(util, [(kern, "MfmaUtil", 10.0), (kern, "MfmaUtil", 14.0), ("other", "MfmaUtil", 99)])
    write(mops, [(kern, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 1000.0),
                 (kern, "SQ_INSTS_VALU_MFMA_MOPS_F32", 10.0)])
    rep = rs.mfma_report(str(util), str(mops), "pass2_mtp", "wl", 2.0, "cu", "cm")
    vals = {l.split(": ", 1)[0]: l.split(": ", 1)[1].split()[0] for l in rep.splitlines()
            if ": " in l and not l.startswith("#")}
    assert float(vals["mfma_util_percent"]) == 12.0
    assert float(vals["mfma_flops_per_launch"]) == 512.0 * 1010.0
    assert vals["mfma_dtype"] == "BF16"
    assert float(vals["mfma_tflops"]) == pytest.approx(512.0 * 1010.0 / 2e-6 / 1e12, abs=0.01)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "mfma_pass2_mtp_wl.txt").write_text(rep + "\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.load_mfma("pass2_mtp", "wl")
    assert got["dtype"] == "bf16" and got["peak_tflops"] == 2500.0
    assert got["frac"] == pytest.approx(got["tflops"] / 2500.0, abs=1e-4)
    (prof / "mfma_pass2_mtp_wl.txt").write_text(rep.replace(rs.source_hash(), "0" * 16))
    assert bench.load_mfma("pass2_mtp", "wl") is None
