"""Summaries of rocprofv3 CSV output for this library's kernels.

    python -m rank_gradient_compression_amd.rocprof_summary stats DIR
        per-kernel launch count and mean duration from DIR/*kernel_stats.csv
    python -m rank_gradient_compression_amd.rocprof_summary traffic FETCH_DIR WRITE_DIR KIND
        calibrated HBM bytes per launch of one kernel kind from two --pmc runs
        (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch). Each counter is scaled by what
        it reads for the largest device-to-device copies in the same run (the copy
        dispatches whose counter value is within 1% of the largest), whose bytes are
        known: they read and write the same number of bytes.
    python -m rank_gradient_compression_amd.rocprof_summary mean DIR KIND
        mean launch duration (us) of one kernel kind from DIR/*kernel_stats.csv
    python -m rank_gradient_compression_amd.rocprof_summary mfma UTIL_DIR MOPS_DIR KIND
        matrix-core use of one kernel kind from two --pmc runs: the derived MfmaUtil
        (percent of SIMD cycles with the matrix core busy), then the MFMA operation
        counts SQ_INSTS_VALU_MFMA_MOPS_{F32,F16,BF16} (512 flops each).

The traffic summary carries `source_hash`, a digest of the kernel sources, so a
measurement is only used while the kernels it was taken on are unchanged.
"""
from __future__ import annotations

import csv
import glob
import hashlib
import os
import re
import sys

PKG = os.path.dirname(os.path.abspath(__file__))

# library kernel kind -> kernel symbol patterns (vector and matrix-core variants)
KIND_PATTERNS = {
    "pass1_mq": r"k_pass1(_mfma)?<",
    "pass2_mtp": r"k_pass2(_mfma)?<",
    "pass3_decompress_error": r"k_pass3(_mfma)?<",
    "orthogonalize": r"k_orth<",
    "pass2_reduce": r"k_pass2_reduce<",
    "gram": r"k_gram<",
}
COPY_PATTERN = r"copyBuffer"
# this library's kernels (and the calibration copy) in the statistics table
OWN_PATTERN = r"psgd::kern::k_|copyBuffer"


def source_hash() -> str:
    h = hashlib.sha256()
    for name in ("kernels.hip", "internal.h", "host.cpp"):
        with open(os.path.join(PKG, "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    m = re.search(r"(k_\w+<[^>]*>|k_\w+|\w*copyBuffer\w*)", name)
    return m.group(1) if m else name[:60]


def stats(directory: str) -> str:
    path = glob.glob(os.path.join(directory, "*kernel_stats.csv"))[0]
    lines = [f"{'kernel':44s} {'calls':>7s} {'mean_us':>10s} {'min_us':>9s} {'max_us':>9s}"]
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if not re.search(OWN_PATTERN, r["Name"]):
                continue
            rows.append((float(r["TotalDurationNs"]), short_name(r["Name"]), int(r["Calls"]),
                         float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                         float(r["MaxNs"]) / 1e3))
    for _, n, c, avg, mn, mx in sorted(rows, reverse=True):
        lines.append(f"{n:44s} {c:7d} {avg:10.2f} {mn:9.2f} {mx:9.2f}")
    return "\n".join(lines)


def mean_us(directory: str, kind: str) -> float:
    """Mean duration (us) of one kernel kind's launches in DIR/*kernel_stats.csv."""
    path = glob.glob(os.path.join(directory, "*kernel_stats.csv"))[0]
    total = calls = 0.0
    with open(path) as f:
        for r in csv.DictReader(f):
            if re.search(KIND_PATTERNS[kind], r["Name"]):
                total += float(r["TotalDurationNs"])
                calls += int(r["Calls"])
    return total / calls / 1e3 if calls else 0.0


def _counter_rows(directory: str):
    path = glob.glob(os.path.join(directory, "*counter_collection.csv"))[0]
    with open(path) as f:
        for r in csv.DictReader(f):
            yield r["Kernel_Name"], int(r["Grid_Size"]), float(r["Counter_Value"])


def _per_dispatch(directory: str, pattern: str):
    vals = [(g, v) for n, g, v in _counter_rows(directory) if re.search(pattern, n)]
    return vals


def traffic(fetch_dir: str, write_dir: str, kind: str) -> str:
    pat = KIND_PATTERNS[kind]
    out = {}
    for label, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        kern = [v for _, v in _per_dispatch(d, pat)]
        copies = [v for _, v in _per_dispatch(d, COPY_PATTERN)]
        vmax = max(copies)
        cal = [v for v in copies if v >= 0.99 * vmax]
        out[label] = (sum(kern) / len(kern), len(kern), sum(cal) / len(cal), len(cal), vmax)
    return out


def traffic_report(fetch_dir: str, write_dir: str, kind: str, workload: str,
                   copy_bytes: int, command_fetch: str, command_write: str) -> str:
    t = traffic(fetch_dir, write_dir, kind)
    f_k, f_n, f_cal, f_cn, _ = t["FETCH_SIZE"]
    w_k, w_n, w_cal, w_cn, _ = t["WRITE_SIZE"]
    f_factor = copy_bytes / (f_cal * 1024.0)
    w_factor = copy_bytes / (w_cal * 1024.0)
    hbm = f_k * 1024.0 * f_factor + w_k * 1024.0 * w_factor
    return "\n".join([
        f"# HBM traffic per launch of {kind} on the {workload} workload",
        f"# fetch command: {command_fetch}",
        f"# write command: {command_write}",
        f"kernel_kind: {kind}",
        f"workload: {workload}",
        f"source_hash: {source_hash()}",
        f"fetch_kib_per_launch: {f_k:.1f}  (mean of {f_n} dispatches)",
        f"write_kib_per_launch: {w_k:.1f}  (mean of {w_n} dispatches)",
        f"copy_calibration_bytes_each_way: {copy_bytes}",
        f"copy_fetch_kib: {f_cal:.1f}  (mean of {f_cn} dispatches) -> factor {f_factor:.4f}",
        f"copy_write_kib: {w_cal:.1f}  (mean of {w_cn} dispatches) -> factor {w_factor:.4f}",
        f"hbm_bytes_per_launch: {hbm:.0f}",
    ])


def _counter_by_name(directory: str, pattern: str):
    path = glob.glob(os.path.join(directory, "*counter_collection.csv"))[0]
    out = {}
    with open(path) as f:
        for r in csv.DictReader(f):
            if re.search(pattern, r["Kernel_Name"]):
                out.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in out.items()}, {k: len(v) for k, v in out.items()}


def mfma_report(util_dir: str, mops_dir: str, kind: str, workload: str, mean_us: float,
                command_util: str, command_mops: str) -> str:
    pat = KIND_PATTERNS[kind]
    util, n_u = _counter_by_name(util_dir, pat)
    mops, n_m = _counter_by_name(mops_dir, pat)
    flops = 512.0 * sum(v for k, v in mops.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    lines = [
        f"# matrix-core use per launch of {kind} on the {workload} workload",
        f"# utilisation command: {command_util}",
        f"# operations command: {command_mops}",
        f"kernel_kind: {kind}",
        f"workload: {workload}",
        f"source_hash: {source_hash()}",
        f"mfma_util_percent: {util.get('MfmaUtil', float('nan')):.2f}  "
        f"(mean of {n_u.get('MfmaUtil', 0)} dispatches)",
    ]
    for k in sorted(mops):
        lines.append(f"{k.lower()}_per_launch: {mops[k]:.0f}")
    kinds = {k.rsplit("_", 1)[1]: v for k, v in mops.items()
             if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_")}
    if kinds:
        lines.append(f"mfma_dtype: {max(kinds, key=kinds.get)}")
    lines.append(f"mfma_flops_per_launch: {flops:.0f}")
    if mean_us > 0:
        lines.append(f"mean_launch_us: {mean_us:.2f}  (kernel statistics of the same workload)")
        lines.append(f"mfma_tflops: {flops / (mean_us * 1e-6) / 1e12:.2f}")
    return "\n".join(lines)


if __name__ == "__main__":
    if sys.argv[1] == "stats":
        print(stats(sys.argv[2]))
    elif sys.argv[1] == "traffic":
        print(traffic_report(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5],
                             int(sys.argv[6]), sys.argv[7], sys.argv[8]))
    elif sys.argv[1] == "mfma":
        print(mfma_report(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5],
                          float(sys.argv[6]), sys.argv[7], sys.argv[8]))
    elif sys.argv[1] == "mean":
        print(f"{mean_us(sys.argv[2], sys.argv[3]):.3f}")
    elif sys.argv[1] == "hash":
        print(source_hash())
