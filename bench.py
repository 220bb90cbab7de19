"""Benchmark of PowerSGD bucket compression on one MI355X.

One step = one powersgd_compress_bucket call on a fresh synthetic gradient bucket
(every pass of the method: error-feedback add, P = M'Q, Gram-Schmidt, Q = M'^T P,
decompress + error update). Buckets are generated on the GPU before timing, one per
step, so inputs are resident in HBM when the timed region starts.

value = whole-job gradient throughput: bucket bytes per step / time per step.
roofline = the dominant kernel's algorithmic bytes per launch / its mean launch
duration (HIP events recorded by the library on the launch stream during the
timed region), against the 8 TB/s HBM peak.
cpu_baseline = the fp64 oracle timed on the host on a bounded sample of the same
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 1]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "gradient GB/s compressed per PowerSGD step + % of HBM roofline, 1 GPU"
HBM_PEAK_GBS = 8000.0
DEFAULT_CONFIG = 1


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def load_traffic(kernel: str, workload: str):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/), if the
    measurement was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    from rank_gradient_compression_amd.rocprof_summary import source_hash
    if vals.get("source_hash") != source_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# dense matrix-core peaks of MI355X, TFLOP/s
MFMA_PEAK_TFLOPS = {"F32": 157.3, "F16": 2500.0, "BF16": 2500.0}


def load_mfma(kernel: str, workload: str):
    """Matrix-core use of a kernel measured with rocprofv3 counters (profiles/), if the
    measurement was taken on the current kernel sources."""
    path = os.path.join(ROOT, "profiles", f"mfma_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.split()[0] if v.split() else ""
    from rank_gradient_compression_amd.rocprof_summary import source_hash
    if vals.get("source_hash") != source_hash():
        return None
    try:
        tflops = float(vals["mfma_tflops"])
        dt = vals.get("mfma_dtype", "F32")
        peak = MFMA_PEAK_TFLOPS.get(dt, MFMA_PEAK_TFLOPS["F32"])
        return {"util_percent": float(vals["mfma_util_percent"]), "tflops": tflops,
                "dtype": dt.lower(), "peak_tflops": peak, "frac": round(tflops / peak, 4)}
    except (KeyError, ValueError):
        return None


def copy_bandwidth(torch, nbytes: int = 1 << 31, reps: int = 10) -> float:
    """GB/s of a plain device-to-device copy (bytes read + bytes written)."""
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for _ in range(reps):
        dst.copy_(src)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * nbytes / (ms * 1e-3) / 1e9


def cpu_baseline(cfg, budget_s: float = 20.0):
    """The oracle, as it stands, on whole steps of the same workload for ~budget_s."""
    import numpy as np
    from threadpoolctl import threadpool_info

    import oracle
    from synthetic import BucketGenerator

    gen = BucketGenerator(cfg, "cpu")
    hp = oracle.HParams(**{k: v for k, v in cfg.hparams.items()
                           if k in oracle.HParams.__dataclass_fields__})
    st = oracle.OracleState(hp)
    views = cfg.views()
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    times = []
    t_start = time.perf_counter()
    step = 0
    while True:
        bucket = gen.bucket(step)
        arr = bucket.numpy()
        scale = cfg.loss_scale if cfg.dtype == "f16" else 1.0
        t0 = time.perf_counter()
        if cfg.batched:
            st.compress_bucket_batched(arr, inv_loss_scale=1.0 / scale)
        elif cfg.wrap:
            st.compress_bucket_wrapped(arr, views, cfg.wrap)
        else:
            st.compress_bucket(arr, views, inv_loss_scale=1.0 / scale)
        times.append(time.perf_counter() - t0)
        step += 1
        if time.perf_counter() - t_start > budget_s:  # whole steps until the budget is spent
            break
    per_step = float(np.median(times))
    gbs = cfg.numel * cfg.element_bytes / per_step / 1e9
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} whole steps of the {cfg.name} bucket "
                      f"({cfg.numel} elements), median {per_step:.3f} s/step, fp64 numpy "
                      f"with {threads} BLAS threads"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the per-kernel event timing (no roofline object)")
    ap.add_argument("--snapshot", action="store_true",
                    help="also time one state export and import after the run (stderr)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        eprint("bench.py measures one GPU only: the compression step runs on one rank and "
               "the library issues no collectives; run with --gpus 1.")
        return 2

    import torch

    from rank_gradient_compression_amd import PowerSGDState, powersgd_batched_side
    from synthetic import CONFIGS, BucketGenerator

    cfg = CONFIGS[args.config]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    copy_gbs = copy_bandwidth(torch)
    eprint(f"[bench] device-to-device copy: {copy_gbs:.0f} GB/s (read + write)")
    bucket_bytes = cfg.numel * cfg.element_bytes
    total = 2 * args.steps + args.warmup
    gen = BucketGenerator(cfg, "cuda")

    # One distinct bucket per step while it fits in a third of free HBM; beyond that
    # the pool is reused (the kernels' work does not depend on the values).
    free, _ = torch.cuda.mem_get_info()
    pool_n = max(1, min(total, int(free * 0.33) // bucket_bytes))
    eprint(f"[bench] {cfg.name}: {cfg.numel} elements, {bucket_bytes / 1e6:.1f} MB per bucket, "
           f"{pool_n} distinct buckets for {total} steps")
    # Benchmark steps carry the workload's random inf draws only (the forced inf step
    # belongs to the correctness runs).
    pool = [gen.bucket(i, forced=False) for i in range(pool_n)]
    side = powersgd_batched_side(cfg.numel) if cfg.batched else 0
    if cfg.batched:
        # the batched variant works in a buffer that holds the padded square matrix
        padded = []
        for b in pool:
            buf = torch.zeros(side * side, dtype=b.dtype, device=dev)
            buf[:cfg.numel].copy_(b)
            padded.append(buf)
        pool = padded
    views = cfg.views()
    hp = dict(cfg.hparams)
    hp["compression_stats_logging_frequency"] = 0
    st = PowerSGDState(device=0, **hp)
    stream = torch.cuda.current_stream()
    found = torch.zeros(1, dtype=torch.int32, device=dev)
    inv = 1.0 / cfg.loss_scale if cfg.dtype == "f16" else 1.0

    def run(i):
        if cfg.dtype == "f16":
            found.zero_()      # a new iteration: GradScaler starts from "no inf found"
        if cfg.batched:
            st.compress_bucket_batched(pool[i % pool_n], numel=cfg.numel, inv_loss_scale=inv,
                                       found_inf=found if cfg.dtype == "f16" else None,
                                       stream=stream)
        elif cfg.wrap:
            st.compress_bucket_wrapped(pool[i % pool_n], views, cfg.wrap, stream=stream)
        else:
            st.compress_bucket(pool[i % pool_n], views, inv_loss_scale=inv,
                               found_inf=found if cfg.dtype == "f16" else None, stream=stream)

    for i in range(args.warmup):
        run(i)
    torch.cuda.synchronize()
    eprint("[bench] warmup done")

    # Timed region: K steps back to back, no per-kernel events.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        run(args.warmup + i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    value = bucket_bytes / (ms_per_step * 1e-3) / 1e9

    # Second timed region over the same K steps with HIP events recorded by the
    # library around every kernel on the launch stream (events between kernels add
    # host and queue work, so they are kept out of the region `value` comes from).
    if not args.no_kernel_timing:
        st.set_timing(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            run(args.warmup + args.steps + i)
        torch.cuda.synchronize()
        ev_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        eprint(f"[bench] {ms_per_step * 1e3:.1f} us/step; with per-kernel events "
               f"{ev_ms * 1e3:.1f} us/step")
    roofline = None
    if not args.no_kernel_timing:
        kt = st.kernel_times()
        for name, ms, n, by in kt:
            if n:
                eprint(f"[bench] kernel {name:24s} launches {n:6d}  mean {ms / n * 1e3:9.2f} us"
                       f"  algorithmic {by / n / 1e6:9.2f} MB/launch"
                       + (f"  {by / (ms * 1e-3) / 1e9:8.1f} GB/s" if by > 0 else ""))
        streaming = [(ms, name, n, by) for name, ms, n, by in kt if by > 0 and n > 0]
        ms, name, n, by = max(streaming)
        avg_s = ms * 1e-3 / n
        achieved = by / n / avg_s / 1e9
        sum_ms = sum(x[1] for x in kt)
        eprint(f"[bench] kernels total {sum_ms / args.steps * 1e3:.1f} us/step")
        traffic = load_traffic(name, cfg.name)
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": traffic, "kernel": name,
                    "mean_launch_us": round(avg_s * 1e6, 3),
                    "algorithmic_bytes_per_launch": by / n}
        if cfg.hparams["matrix_approximation_rank"] >= 16:
            # the matrix-core passes: utilisation from rocprofv3 counters
            mfma = {k: load_mfma(k, cfg.name)
                    for k in ("pass1_mq", "pass2_mtp", "pass3_decompress_error")}
            roofline["mfma"] = {k: v for k, v in mfma.items() if v is not None} or None
    if args.snapshot:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        blob = st.export_state()
        t_exp = time.perf_counter() - t0
        t0 = time.perf_counter()
        st.import_state(blob)
        t_imp = time.perf_counter() - t0
        eprint(f"[bench] snapshot {len(blob) / 1e6:.1f} MB: export {t_exp * 1e3:.1f} ms "
               f"({len(blob) / t_exp / 1e9:.2f} GB/s), import {t_imp * 1e3:.1f} ms "
               f"({len(blob) / t_imp / 1e9:.2f} GB/s), host side a Python bytearray")
        del blob
    st.close()
    del pool
    torch.cuda.empty_cache()

    from rank_gradient_compression_amd import powersgd as api
    hp_c = api.powersgd_hparams_init()
    hp_c.matrix_approximation_rank = cfg.hparams["matrix_approximation_rank"]
    hp_c.min_compression_rate = cfg.hparams["min_compression_rate"]
    comp_elems = 0
    if cfg.batched:
        comp_elems = side * side  # one padded square matrix
    else:
        for _, shp in views:
            comp, n, m, _r = api.powersgd_classify_view(hp_c, shp)
            comp_elems += n * m if comp else 0
    ef = bool(cfg.hparams.get("use_error_feedback", True))
    if cfg.wrap:
        # fp32 bucket, 16-bit M' and E: 8 + 2 + 8 per compressed element (6 + 2 + 4
        # without error feedback); the cast of the other views reads and writes fp32
        algo_bytes = comp_elems * (18 if ef else 12) + (cfg.numel - comp_elems) * 8
    else:
        # fp32: 12 + 4 + 12 (4 + 4 + 4 without error feedback); fp16: 6 + 6 + 12 (2 + 2 + 2)
        per_elt = (28 if ef else 12) if cfg.dtype == "f32" else (24 if ef else 6)
        algo_bytes = comp_elems * per_elt + (0 if cfg.dtype == "f32" or cfg.batched else
                                             (cfg.numel - comp_elems) * 6)
    step_frac = algo_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.wrap or "f32",
        "data": "synthetic (seeded low-rank + noise gradients, model-shaped views)",
        "config": {"workload": cfg.name, "bucket_bytes": bucket_bytes,
                   "views": len(views), "compressed_elements": comp_elems,
                   "variant": ("batched: one %d x %d padded matrix" % (side, side)
                               if cfg.batched else
                               "%s_compress_wrapper(powerSGD_hook), fp32 bucket" % cfg.wrap
                               if cfg.wrap else "per-layer"),
                   "matrix_approximation_rank": cfg.hparams["matrix_approximation_rank"],
                   "step_hbm_roofline_frac": round(step_frac, 4),
                   "measured_copy_GBps": round(copy_gbs, 1),
                   "step_algorithmic_bytes": algo_bytes},
        "roofline": roofline,
    }
    if not args.no_cpu_baseline:
        eprint("[bench] timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
