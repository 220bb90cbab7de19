"""Side-by-side runs of the HIP library and the fp64 oracle on identical inputs.

Comparison rules (per compressed view, per quantity, per step):
  relative Frobenius error ||X_gpu - X_oracle|| / ||X_oracle|| <= tol, with
  tol = 1e-4 for fp32 buckets and 2e-3 for fp16 buckets; for E, when
  ||E_oracle|| < 1e-3 ||M'_oracle|| (near-exact recovery) the denominator is
  ||M'_oracle||. Decisions and found_inf are compared bit-exactly; uncompressed
  fp32 views must be bit-identical to the input, uncompressed fp16 views
  bit-identical to the oracle's round-to-nearest-even output.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

import oracle
from oracle import HParams, OracleState
from rank_gradient_compression_amd import PowerSGDState

TOL = {"f32": 1e-4, "f16": 2e-3}

_hip = None


def device_to_tensor(ptr: int, shape, dtype) -> torch.Tensor:
    """A torch copy of `shape` elements of `dtype` at device address `ptr` (memory the
    library owns), made with hipMemcpy after the device has finished its queued work."""
    global _hip
    if _hip is None:
        import ctypes
        _hip = ctypes.CDLL("libamdhip64.so")
        _hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                   ctypes.c_int]
        _hip.hipMemcpy.restype = ctypes.c_int
    out = torch.empty(shape, dtype=dtype, device="cuda")
    torch.cuda.synchronize()
    if out.numel():
        rc = _hip.hipMemcpy(out.data_ptr(), ptr, out.numel() * out.element_size(),
                            3)  # hipMemcpyDeviceToDevice
        assert rc == 0, f"hipMemcpy failed with {rc}"
    return out


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def rel_fro(a: np.ndarray, b: np.ndarray, denom: Optional[float] = None) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    d = np.linalg.norm(b) if denom is None else denom
    diff = np.linalg.norm(a - b)
    if d == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return float(diff / d)


def numel(shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


@dataclass
class StepReport:
    step: int
    worst: Dict[str, float] = field(default_factory=dict)
    found_inf: bool = False

    def update(self, name: str, value: float) -> None:
        self.worst[name] = max(self.worst.get(name, 0.0), value)


def oracle_hparams(hp: dict) -> HParams:
    keys = HParams.__dataclass_fields__.keys()
    return HParams(**{k: v for k, v in hp.items() if k in keys})


class BucketParity:
    """Runs the library and the oracle on the same bucket, step after step, and
    compares every view (whole-bucket oracle: for oracle-sized buckets)."""

    def __init__(self, hp: dict, views, dtype: str = "f32", bucket_index: int = 0,
                 quantities=("P", "Q", "Mhat", "E")):
        self.quantities = tuple(quantities)
        self.hp = dict(hp)
        self.views = [(int(o), tuple(int(d) for d in s)) for o, s in views]
        self.dtype = dtype
        self.bucket_index = bucket_index
        self.gpu = PowerSGDState(**self.hp)
        self.oracle = OracleState(oracle_hparams(self.hp))
        self.tol = TOL[dtype]

    def step(self, host_bucket: torch.Tensor, step: int, is_last: bool = True,
             inv_loss_scale: float = 1.0, check: bool = True) -> StepReport:
        dev = host_bucket.to("cuda")
        found = torch.zeros(1, dtype=torch.int32, device="cuda")
        prev_state = None
        if self.dtype == "f16" and check:
            prev_state = self._snapshot()
        self.gpu.compress_bucket(dev, self.views, bucket_index=self.bucket_index,
                                 is_last=is_last, inv_loss_scale=inv_loss_scale,
                                 found_inf=found if self.dtype == "f16" else None)
        res = self.oracle.compress_bucket(host_bucket.numpy(), self.views,
                                          bucket_index=self.bucket_index, is_last=is_last,
                                          inv_loss_scale=inv_loss_scale)
        torch.cuda.synchronize()
        rep = StepReport(step=step, found_inf=res.found_inf)
        if not check:
            return rep
        gpu_out = dev.cpu()
        if self.dtype == "f16":
            assert bool(found.item()) == res.found_inf, (step, "found_inf")
        if res.skipped:
            assert torch.equal(gpu_out.view(torch.int16), host_bucket.view(torch.int16))
            if prev_state is not None:
                after = self._snapshot()
                for k in prev_state:
                    assert torch.equal(prev_state[k], after[k]), (step, k, "state changed")
            return rep
        if res.passthrough:
            self._check_uncompressed_all(gpu_out, res, host_bucket)
            return rep
        dec = self.gpu.decisions(self.bucket_index, len(self.views))
        assert dec == [int(v.compressed) for v in res.views], (step, "decisions")
        for vi, ((off, shp), vr) in enumerate(zip(self.views, res.views)):
            size = numel(shp)
            if not vr.compressed:
                self._check_uncompressed(gpu_out[off:off + size], res.output[off:off + size],
                                         host_bucket[off:off + size], vi, step)
                continue
            self._compare_view(rep, vi, vr, gpu_out[off:off + size])
        return rep

    def _snapshot(self):
        snap = {}
        try:
            dec = self.gpu.decisions(self.bucket_index, len(self.views))
        except Exception:
            return snap
        for vi, d in enumerate(dec):
            if d:
                p, q = self.gpu.factors(self.bucket_index, vi)
                snap[f"Q{vi}"] = q.cpu()
                if self.hp.get("use_error_feedback", True):
                    snap[f"E{vi}"] = self.gpu.error(self.bucket_index, vi).cpu()
        torch.cuda.synchronize()
        return snap

    def _check_uncompressed(self, gpu_vals, oracle_vals, inp, vi, step):
        if self.dtype == "f32":
            assert torch.equal(gpu_vals.view(torch.int32), inp.view(torch.int32)), (step, vi)
        else:
            exp = torch.from_numpy(np.ascontiguousarray(oracle_vals))
            assert torch.equal(gpu_vals.view(torch.int16), exp.view(torch.int16)), (step, vi)

    def _check_uncompressed_all(self, gpu_out, res, inp):
        for vi, (off, shp) in enumerate(self.views):
            size = numel(shp)
            self._check_uncompressed(gpu_out[off:off + size], res.output[off:off + size],
                                     inp[off:off + size], vi, -1)

    def _compare_view(self, rep: StepReport, vi: int, vr, gpu_mhat_flat) -> None:
        n, m, r = self.gpu.view_info(self.bucket_index, vi)
        assert (n, m, r) == (vr.n, vr.m, vr.rank), (vi, "shape")
        p, q = self.gpu.factors(self.bucket_index, vi)
        p = p.cpu().double().numpy()
        q = q.cpu().double().numpy()
        mhat = gpu_mhat_flat.double().numpy().reshape(n, m)
        errs = {"P": rel_fro(p, vr.p), "Q": rel_fro(q, vr.q), "Mhat": rel_fro(mhat, vr.m_hat)}
        if vr.error is not None:
            e = self.gpu.error(self.bucket_index, vi).cpu().double().numpy()
            ne = np.linalg.norm(vr.error)
            nm = np.linalg.norm(vr.m_prime)
            errs["E"] = rel_fro(e, vr.error, denom=nm if ne < 1e-3 * nm else None)
        for k, v in errs.items():
            if k not in self.quantities:
                continue
            rep.update(k, v)
            assert v <= self.tol, (rep.step, vi, k, v, (n, m, r))


class TensorTrack:
    """The oracle's per-matrix state for one sampled view of a large bucket: the
    oracle's own functions, fed the view's slice of the same input bucket."""

    def __init__(self, hp: dict, view_index: int, n: int, m: int, rank: int,
                 bucket_index: int = 0):
        self.hp = oracle_hparams(hp)
        self.view = view_index
        self.n, self.m, self.rank = n, m, rank
        self.bucket_index = bucket_index
        self.e = None
        self.q = None

    def step(self, g: np.ndarray, iteration: int):
        hp = self.hp
        eps = float(hp.orthogonalization_epsilon)
        if hp.warm_start and self.q is not None:
            q = self.q
        else:
            epoch = 0 if hp.warm_start else iteration
            q = oracle.gram_schmidt(oracle.standard_normal_q0(
                self.m, self.rank, hp.random_seed, self.bucket_index, self.view, epoch), eps)
        vr = oracle.compress_matrix_step(g.reshape(self.n, self.m), self.e, q, eps,
                                         hp.use_error_feedback)
        if hp.use_error_feedback:
            self.e = vr.error
        if hp.warm_start:
            self.q = vr.q
        return vr


def compare_sampled(gpu: PowerSGDState, bucket_index: int, vi: int, vr, gpu_bucket_slice,
                    tol: float, rep: StepReport) -> None:
    n, m, r = gpu.view_info(bucket_index, vi)
    assert (n, m, r) == (vr.n, vr.m, vr.rank)
    p, q = gpu.factors(bucket_index, vi)
    errs = {"P": rel_fro(p.cpu().double().numpy(), vr.p),
            "Q": rel_fro(q.cpu().double().numpy(), vr.q),
            "Mhat": rel_fro(gpu_bucket_slice.cpu().double().numpy().reshape(n, m), vr.m_hat)}
    if vr.error is not None:
        e = gpu.error(bucket_index, vi).cpu().double().numpy()
        ne, nm = np.linalg.norm(vr.error), np.linalg.norm(vr.m_prime)
        errs["E"] = rel_fro(e, vr.error, denom=nm if ne < 1e-3 * nm else None)
    for k, v in errs.items():
        rep.update(k, v)
        assert v <= tol, (rep.step, vi, k, v, (n, m, r))


# ---------------------------------------------------- the wrapped hook (16-bit state)

# 4 units of 16-bit rounding (u = 2^-11 binary16, 2^-8 bfloat16): both sides round every
# materialized tensor; only the accumulation before each rounding differs.
TOL_WRAPPED = {"f16": 4 * 2.0 ** -11, "bf16": 4 * 2.0 ** -8}


class TensorTrackWrapped(TensorTrack):
    """TensorTrack for the wrapped hook: the view's slice is cast to 16 bits and the
    oracle's 16-bit matrix step follows it."""

    def __init__(self, hp: dict, view_index: int, n: int, m: int, rank: int, dt: str,
                 bucket_index: int = 0):
        super().__init__(hp, view_index, n, m, rank, bucket_index)
        self.rnd = oracle.round_f16 if dt == "f16" else oracle.round_bf16

    def step(self, g: np.ndarray, iteration: int):
        hp, rnd = self.hp, self.rnd
        eps = float(hp.orthogonalization_epsilon)
        if hp.warm_start and self.q is not None:
            q = self.q
        else:
            epoch = 0 if hp.warm_start else iteration
            q = rnd(oracle.gram_schmidt(rnd(oracle.standard_normal_q0(
                self.m, self.rank, hp.random_seed, self.bucket_index, self.view, epoch)), eps))
        mp, p, qn, mh, err = oracle.compress_matrix_step_lowp(
            rnd(g.reshape(self.n, self.m)), self.e, q, eps, hp.use_error_feedback, rnd)
        if hp.use_error_feedback:
            self.e = err
        if hp.warm_start:
            self.q = qn
        return oracle.ViewResult(compressed=True, n=self.n, m=self.m, rank=self.rank,
                                 m_prime=mp, p=p, q=qn, m_hat=mh, error=err)


# Steps over which a 16-bit trajectory is held to the oracle: two correct 16-bit
# trajectories that differ only in how sums are accumulated separate geometrically
# (the ResNet-50 bucket in bfloat16: about 1u by step 4, 3u by step 10, 13u by step 13
# between fp64- and fp32-accumulated oracle runs), so the bound applies to the first
# steps and later steps are checked through properties that hold on any trajectory.
WRAPPED_ORACLE_STEPS = 5


def check_wrapped_properties(gpu: PowerSGDState, bucket_index: int, vi: int, dt: str,
                             g_in: np.ndarray, e_prev, out_view: np.ndarray):
    """The GPU's own results of one compressed view, at any step: M_hat is 16-bit, and
    E = M' - M_hat rounded once, with M' = rnd(rnd(G) + E_prev). Returns E."""
    rnd = oracle.round_f16 if dt == "f16" else oracle.round_bf16
    u = 2.0 ** -11 if dt == "f16" else 2.0 ** -8
    n, m, _ = gpu.view_info(bucket_index, vi)
    mh = out_view.astype(np.float64).reshape(n, m)
    assert np.all(rnd(mh) == mh), (vi, "M_hat is not 16-bit")
    g16 = rnd(g_in.astype(np.float64)).reshape(n, m)
    mp = rnd(g16 + e_prev) if e_prev is not None else g16
    e = gpu.error(bucket_index, vi).cpu().double().numpy()
    assert np.all(np.abs(e - (mp - mh)) <= u * np.abs(e) + 1e-30), (vi, "E != rnd(M' - M_hat)")
    return e
