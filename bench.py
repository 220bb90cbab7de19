"""Benchmark of PowerSGD bucket compression on one MI355X.

One step = one powersgd_compress_bucket call on a fresh synthetic gradient bucket
(every pass of the method: error-feedback add, P = M'Q, Gram-Schmidt, Q = M'^T P,
decompress + error update). Buckets are generated on the GPU before timing, so
inputs are resident in HBM when the timed region starts.

value = whole-job gradient throughput: bucket bytes per step / median step time,
over all steady-state steps of three fresh-state repeats (each step timed with
events on the launch stream).
roofline = the dominant kernel's algorithmic bytes per launch / its mean launch
duration (HIP events recorded by the library on the launch stream during the
timed region), against the 8 TB/s HBM peak.
cpu_baseline = the fp64 oracle timed on the host on a bounded sample of the same
workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--repeats 3] [--config 3]

The default workload is the GPT-style bucket (8 layers of 4096 x 4096, 4096 x 16384
and 16384 x 4096 matrices, 5.9 GB, rank 32 on the matrix cores): the largest
configuration, which no cache holds. The ResNet-50-shaped bucket (warm and cold) and
the BERT-large one are reported on stderr and in "secondary".
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
DEFAULT_CONFIG = 3


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


def _oracle_hparams(cfg):
    import oracle
    return oracle.HParams(**{k: v for k, v in cfg.hparams.items()
                             if k in oracle.HParams.__dataclass_fields__})


def _oracle_steps(cfg, budget_s: float, min_steps: int = 2):
    """Whole oracle steps of `cfg` (each on its own seeded bucket) until budget_s of
    host time is spent (at least min_steps, at most cfg.steps); per-step seconds."""
    import oracle
    from synthetic import BucketGenerator

    gen = BucketGenerator(cfg, "cpu")
    st = oracle.OracleState(_oracle_hparams(cfg))
    views = cfg.views()
    scale = cfg.loss_scale if cfg.dtype == "f16" else 1.0
    times = []
    t_start = time.perf_counter()
    for step in range(cfg.steps):
        arr = gen.bucket(step).numpy()
        t0 = time.perf_counter()
        if cfg.batched:
            st.compress_bucket_batched(arr, inv_loss_scale=1.0 / scale)
        elif cfg.wrap:
            st.compress_bucket_wrapped(arr, views, cfg.wrap)
        else:
            st.compress_bucket(arr, views, inv_loss_scale=1.0 / scale)
        times.append(time.perf_counter() - t0)
        if len(times) >= min_steps and time.perf_counter() - t_start > budget_s:
            break
    return times


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, budget_s: float = 20.0):
    """The oracle, as it stands, timed on the host. Workloads whose fp64 state would
    not fit comfortably in host memory (above 2^28 elements) are sampled: their first
    layer's views form a bucket of their own (same shapes, generator and
    hyperparameters). Besides the figure with all BLAS threads, one-thread figures
    are given for the single 256 x 512 matrix and the ResNet-50-shaped bucket."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    from synthetic import CONFIGS, shrink_config

    sample = cfg
    what = f"whole steps of the {cfg.name} bucket ({cfg.numel} elements)"
    if cfg.numel > (1 << 28) and not cfg.batched:
        per_layer = 5 if cfg.name.startswith("gpt") else 16
        sample = shrink_config(cfg, cfg.shapes[:per_layer], name=cfg.name + "-first-layer")
        what = (f"whole steps of the {cfg.name} bucket's first layer ({len(sample.shapes)} views, "
                f"{sample.numel} of {cfg.numel} elements), a bucket of its own")
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    times = _oracle_steps(sample, budget_s)
    steady = times[1:] if len(times) > 1 else times
    per_step = float(np.median(steady))
    gbs = sample.numel * sample.element_bytes / per_step / 1e9
    one = {}
    with threadpool_limits(1):
        for c in (CONFIGS[0], CONFIGS[1]):
            t = _oracle_steps(c, 5.0)
            st = t[1:] if len(t) > 1 else t
            med = float(np.median(st))
            one[c.name] = {"value": round(c.numel * c.element_bytes / med / 1e9, 4),
                           "unit": "GB/s", "s_per_step": round(med, 4), "steps": len(t)}
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{len(times)} {what}; median of steps 2.. {per_step:.3f} s/step; fp64 "
                      f"numpy (Gram-Schmidt in double-double) with {threads} BLAS threads",
            "nproc": os.cpu_count(), "cpu_model": cpu_model(), "one_thread": one}


class Workload:
    """A pool of GPU-resident buckets of one workload and the call that compresses one."""

    def __init__(self, torch, cfg, steps_needed: int, share: float = 0.33):
        from rank_gradient_compression_amd import powersgd_batched_side
        from synthetic import BucketGenerator

        self.torch = torch
        self.cfg = cfg
        self.bucket_bytes = cfg.numel * cfg.element_bytes
        gen = BucketGenerator(cfg, "cuda")
        free, _ = torch.cuda.mem_get_info()
        # one distinct bucket per step while the pool fits in a share of free HBM; beyond
        # that buckets are reused (the kernels' work does not depend on the values)
        self.pool_n = max(1, min(steps_needed, int(free * share) // (3 * self.bucket_bytes)))
        # benchmark steps carry the workload's random inf draws only (the forced inf
        # step belongs to the correctness runs)
        pool = [gen.bucket(i, forced=False) for i in range(self.pool_n)]
        self.side = powersgd_batched_side(cfg.numel) if cfg.batched else 0
        if cfg.batched:
            padded = []
            for b in pool:
                buf = torch.zeros(self.side * self.side, dtype=b.dtype, device="cuda")
                buf[:cfg.numel].copy_(b)
                padded.append(buf)
            pool = padded
        self.pool = pool
        self.views = cfg.views()
        self.hp = dict(cfg.hparams)
        self.hp["compression_stats_logging_frequency"] = 0
        self.found = torch.zeros(1, dtype=torch.int32, device="cuda")
        self.inv = 1.0 / cfg.loss_scale if cfg.dtype == "f16" else 1.0
        self.st = None

    def fresh_state(self):
        from rank_gradient_compression_amd import PowerSGDState
        if self.st is not None:
            self.st.close()
        self.st = PowerSGDState(device=0, **self.hp)
        return self.st

    def run(self, i: int) -> None:
        cfg, st = self.cfg, self.st
        stream = self.torch.cuda.current_stream()
        bucket = self.pool[i % self.pool_n]
        fi = self.found if cfg.dtype == "f16" else None
        if fi is not None:
            fi.zero_()  # a new iteration: GradScaler starts from "no inf found"
        if cfg.batched:
            st.compress_bucket_batched(bucket, numel=cfg.numel, inv_loss_scale=self.inv,
                                       found_inf=fi, stream=stream)
        elif cfg.wrap:
            st.compress_bucket_wrapped(bucket, self.views, cfg.wrap, stream=stream)
        else:
            st.compress_bucket(bucket, self.views, inv_loss_scale=self.inv, found_inf=fi,
                               stream=stream)

    def timed_steps(self, first: int, k: int, flush=None, flush_read: bool = False):
        """Per-step milliseconds of steps first..first+k-1 from events on the launch
        stream, each step timed alone; `flush` (a device tensor) is overwritten, or with
        `flush_read` read, before every step, outside its events, so each step starts
        with a cold last-level cache (holding the flush buffer's dirty lines, or clean
        ones). The K steps are bracketed by synchronizations."""
        torch = self.torch
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(k)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for j in range(k):
            if flush is not None:
                if flush_read:
                    flush.sum()
                else:
                    flush.fill_(float(j))
            ev[j][0].record()
            self.run(first + j)
            ev[j][1].record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return [a.elapsed_time(b) for a, b in ev], wall

    def close(self):
        if self.st is not None:
            self.st.close()
            self.st = None
        self.pool = []
        self.torch.cuda.empty_cache()


def measure(torch, cfg, steps: int, warmup: int, repeats: int, flush=None,
            flush_read: bool = False):
    """`repeats` fresh states, each: `warmup` untimed steps (the first allocates), then
    `steps` timed steps. Returns the per-step times of every repeat, the walls of the
    timed regions, and the workload (its last state still open)."""
    wl = Workload(torch, cfg, warmup + steps)
    per_rep, walls = [], []
    for rep in range(repeats):
        wl.fresh_state()
        for i in range(warmup):
            wl.run(i)
        torch.cuda.synchronize()
        t, wall = wl.timed_steps(warmup, steps, flush, flush_read)
        per_rep.append(t)
        walls.append(wall)
    return per_rep, walls, wl


def algorithmic_bytes(cfg, comp_elems: int, per_elt_f32: float = 28.0):
    """Bytes the three passes must move per step (error feedback: 12 + 4 + 12 per
    compressed fp32 element; fp16: 6 + 6 + 12; without error feedback 4 + 4 + 4 and
    2 + 2 + 2; the wrapped hook 8 + 2 + 8 with 16-bit M' and E), plus the pass-through
    work on uncompressed views (fp16 unscale 2 + 4; the wrapper's cast 4 + 4)."""
    ef = bool(cfg.hparams.get("use_error_feedback", True))
    if cfg.wrap:
        return comp_elems * (18 if ef else 12) + (cfg.numel - comp_elems) * 8
    if cfg.dtype == "f32":
        return comp_elems * (per_elt_f32 if ef else 12)
    return comp_elems * (24 if ef else 6) + (0 if cfg.batched else (cfg.numel - comp_elems) * 6)


def moved_bytes(cfg, comp_elems: int):
    """Bytes the library actually moves per step: with error feedback the error memory's
    place keeps M' and the error is rebuilt from it, so pass 3 only writes M_hat. fp32
    buckets: 12 + 4 + 4 per compressed element; fp16 buckets (M' in two alternating
    places, the inf check inside pass 1): 10 + 4 + 2, and the check and unscale of the
    uncompressed views (2 + 2 + 2); the wrapped hook (16-bit M'): 8 + 2 + 4 and the cast
    of the uncompressed views (4 + 4). Without error feedback: the algorithmic bytes."""
    ef = bool(cfg.hparams.get("use_error_feedback", True))
    if cfg.wrap and ef:
        return comp_elems * 14 + (cfg.numel - comp_elems) * 8
    if ef:
        if cfg.dtype == "f32":
            return comp_elems * 20
        unc = 0 if cfg.batched else cfg.numel - comp_elems
        return comp_elems * 16 + unc * 6
    return algorithmic_bytes(cfg, comp_elems)


def compressed_elements(cfg, side: int) -> int:
    from rank_gradient_compression_amd import powersgd as api
    if cfg.batched:
        return side * side
    hp_c = api.powersgd_hparams_init()
    hp_c.matrix_approximation_rank = cfg.hparams["matrix_approximation_rank"]
    hp_c.min_compression_rate = cfg.hparams["min_compression_rate"]
    total = 0
    for _, shp in cfg.views():
        comp, n, m, _r = api.powersgd_classify_view(hp_c, shp)
        total += n * m if comp else 0
    return total


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--repeats", type=int, default=3,
                    help="fresh-state repeats; the headline is the median step over all")
    ap.add_argument("--config", type=int, default=DEFAULT_CONFIG)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true",
                    help="skip the per-kernel event timing (no roofline object)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="skip the other workloads reported on stderr")
    ap.add_argument("--snapshot", action="store_true",
                    help="also time one state export and import after the run (stderr)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        eprint("bench.py measures one GPU only: the compression step runs on one rank and "
               "the library issues no collectives; run with --gpus 1.")
        return 2

    import numpy as np
    import torch

    from synthetic import CONFIGS

    cfg = CONFIGS[args.config]
    torch.cuda.set_device(0)
    copy_gbs = copy_bandwidth(torch)
    eprint(f"[bench] device-to-device copy: {copy_gbs:.0f} GB/s (read + write)")

    per_rep, walls, wl = measure(torch, cfg, args.steps, args.warmup, args.repeats)
    bucket_bytes = wl.bucket_bytes
    steps_all = [t for rep in per_rep for t in rep]
    ms_per_step = float(np.median(steps_all))
    value = bucket_bytes / (ms_per_step * 1e-3) / 1e9
    eprint(f"[bench] {cfg.name}: {cfg.numel} elements, {bucket_bytes / 1e6:.1f} MB per bucket, "
           f"{wl.pool_n} distinct buckets")
    for rep, (t, w) in enumerate(zip(per_rep, walls)):
        eprint(f"[bench] repeat {rep}: median {np.median(t) * 1e3:.1f} us/step, mean "
               f"{np.mean(t) * 1e3:.1f}, min {min(t) * 1e3:.1f}, max {max(t) * 1e3:.1f}; "
               f"timed region {w * 1e3 / len(t) * 1e3:.1f} us/step by the host clock")

    # Per-kernel event timing on the launch stream, over K more steps of the last state
    # (the events add host and queue work, so they stay out of the headline's region).
    roofline = None
    if not args.no_kernel_timing:
        wl.st.set_timing(True)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        for i in range(args.steps):
            wl.run(args.warmup + args.steps + i)
        torch.cuda.synchronize()
        ev_ms = (time.perf_counter() - t1) * 1e3 / args.steps
        eprint(f"[bench] with per-kernel events {ev_ms * 1e3:.1f} us/step")
        kt = wl.st.kernel_times()
        for name, ms, n, by in kt:
            if n:
                eprint(f"[bench] kernel {name:24s} launches {n:6d}  mean {ms / n * 1e3:9.2f} us"
                       f"  algorithmic {by / n / 1e6:9.2f} MB/launch"
                       + (f"  {by / (ms * 1e-3) / 1e9:8.1f} GB/s" if by > 0 else ""))
        streaming = [(ms, name, n, by) for name, ms, n, by in kt if by > 0 and n > 0]
        ms, name, n, by = max(streaming)
        avg_s = ms * 1e-3 / n
        achieved = by / n / avg_s / 1e9
        eprint(f"[bench] kernels total {sum(x[1] for x in kt) / args.steps * 1e3:.1f} us/step")
        roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                    "traffic": load_traffic(name, cfg.name), "kernel": name,
                    "mean_launch_us": round(avg_s * 1e6, 3),
                    "algorithmic_bytes_per_launch": by / n}
        if cfg.hparams["matrix_approximation_rank"] >= 16:
            mfma = {k: load_mfma(k, cfg.name)
                    for k in ("pass1_mq", "pass2_mtp", "pass3_decompress_error")}
            roofline["mfma"] = {k: v for k, v in mfma.items() if v is not None} or None
    if args.snapshot:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        blob = wl.st.export_state()
        t_exp = time.perf_counter() - t0
        t0 = time.perf_counter()
        wl.st.import_state(blob)
        t_imp = time.perf_counter() - t0
        eprint(f"[bench] snapshot {len(blob) / 1e6:.1f} MB: export {t_exp * 1e3:.1f} ms "
               f"({len(blob) / t_exp / 1e9:.2f} GB/s), import {t_imp * 1e3:.1f} ms "
               f"({len(blob) / t_imp / 1e9:.2f} GB/s), host side a Python bytearray")
        del blob
    side = wl.side
    views = wl.views
    wl.close()

    comp_elems = compressed_elements(cfg, side)
    algo_bytes = algorithmic_bytes(cfg, comp_elems)
    step_frac = algo_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS
    moved = moved_bytes(cfg, comp_elems)
    moved_frac = moved / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS

    # Other workloads, for context (stderr and a summary object): the ResNet-50-shaped
    # bucket warm (its 74 MB bucket and E stay in the 256 MB last-level cache between
    # steps) and cold (a 1 GiB buffer written before every step, which leaves the cache
    # full of dirty lines the step then writes back; or read, which leaves clean ones),
    # and BERT-large.
    secondary = {}
    if not args.no_secondary:
        flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(0.0)
        for key, c, fl, rd in (("resnet50-bucket-r2 warm", CONFIGS[1], None, False),
                               ("resnet50-bucket-r2 cold", CONFIGS[1], flush, False),
                               ("resnet50-bucket-r2 cold, clean cache", CONFIGS[1], flush, True),
                               ("bert-large-bucket-r4-batched", CONFIGS[2], None, False)):
            pr, _, w2 = measure(torch, c, args.steps, args.warmup, 1, fl, rd)
            med = float(np.median(pr[0]))
            ce = compressed_elements(c, w2.side)
            w2.close()
            gbs = c.numel * c.element_bytes / (med * 1e-3) / 1e9
            frac = algorithmic_bytes(c, ce) / (med * 1e-3) / 1e9 / HBM_PEAK_GBS
            mfrac = moved_bytes(c, ce) / (med * 1e-3) / 1e9 / HBM_PEAK_GBS
            secondary[key] = {"ms_per_step": round(med, 5), "GBps": round(gbs, 1),
                              "step_hbm_roofline_frac": round(frac, 4),
                              "step_moved_frac": round(mfrac, 4)}
            eprint(f"[bench] {key}: median {med * 1e3:.1f} us/step, {gbs:.0f} GB/s gradient, "
                   f"{frac * 100:.1f}% of 8 TB/s on the three-pass byte count, "
                   f"{mfrac * 100:.1f}% on the bytes moved")
        del flush
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC, "value": round(value, 3), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": cfg.wrap or cfg.dtype,
        "data": "synthetic (seeded low-rank + noise gradients, model-shaped views)",
        "config": {"workload": cfg.name, "bucket_bytes": bucket_bytes,
                   "views": len(views), "compressed_elements": comp_elems,
                   "variant": ("batched: one %d x %d padded matrix" % (side, side)
                               if cfg.batched else
                               "%s_compress_wrapper(powerSGD_hook), fp32 bucket" % cfg.wrap
                               if cfg.wrap else "per-layer"),
                   "matrix_approximation_rank": cfg.hparams["matrix_approximation_rank"],
                   "timing": f"median step of {args.repeats} fresh-state repeats x "
                             f"{args.steps} steps after {args.warmup} warmup steps each",
                   "step_hbm_roofline_frac": round(step_frac, 4),
                   "step_algorithmic_bytes": algo_bytes,
                   "step_moved_bytes": moved,
                   "step_moved_frac": round(moved_frac, 4),
                   "measured_copy_GBps": round(copy_gbs, 1)},
        "roofline": roofline,
        "secondary": secondary or None,
    }
    if not args.no_cpu_baseline:
        eprint("[bench] timing the oracle on the host")
        out["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
