"""Seeded generation of synthetic gradient buckets with torch's generators.

A matrix view (ndim >= 2, seen as shape[0] x prod(shape[1:])) holds
    G = U diag(s) V^T + noise_std * N,   s_j = j ** -spectrum_power, j = 1..k,
with U (n x k) and V (m x k) drawn N(0, 1) once per view and N drawn N(0, 1)
afresh every step, so the low-rank part is the same at every step (error
feedback and warm start see a persistent gradient direction) and the noise is
new. A vector view holds N(0, 1) values drawn afresh every step.

fp16 workloads store RNE(G * amp_prescale * loss_scale) and may receive one
injected +inf at a seeded position on selected steps; fp32 workloads store
G * grad_scale (1 unless a workload sets it).

Values depend on (workload seed, view, role, step) and on the device type
(torch's CPU and GPU generators produce different streams); a given test or
benchmark always draws both sides' inputs from one device.
"""
from __future__ import annotations

from typing import Optional

import torch

from .workloads import WorkloadConfig

_ROLE_U, _ROLE_V, _ROLE_NOISE, _ROLE_VEC, _ROLE_INF = 1, 2, 3, 4, 5


def _seed(cfg_seed: int, view: int, role: int, step: int) -> int:
    # A simple injective packing into 63 bits (views < 2**20, steps < 2**24).
    return ((cfg_seed & 0xFFFF) << 47) | ((view & 0xFFFFF) << 27) | ((role & 0x7) << 24) \
        | (step & 0xFFFFFF)


class BucketGenerator:
    def __init__(self, cfg: WorkloadConfig, device: str = "cpu"):
        self.cfg = cfg
        self.device = torch.device(device)
        self.views = cfg.views()
        self._factors = {}

    def _gen(self, view: int, role: int, step: int) -> torch.Generator:
        g = torch.Generator(device=self.device)
        g.manual_seed(_seed(self.cfg.seed, view, role, step))
        return g

    def _low_rank(self, vi: int, n: int, m: int) -> torch.Tensor:
        key = vi
        if key not in self._factors:
            k = self.cfg.spectrum_rank
            u = torch.randn(n, k, generator=self._gen(vi, _ROLE_U, 0), device=self.device)
            v = torch.randn(m, k, generator=self._gen(vi, _ROLE_V, 0), device=self.device)
            s = torch.arange(1, k + 1, device=self.device, dtype=torch.float64)
            s = s.pow(-self.cfg.spectrum_power).to(torch.float32)
            self._factors[key] = (u * s, v)
        us, v = self._factors[key]
        return us @ v.t()

    def gradient(self, step: int, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        """The fp32 gradient bucket of `step` (before any loss scaling)."""
        cfg = self.cfg
        if out is None:
            out = torch.empty(cfg.numel, dtype=torch.float32, device=self.device)
        for vi, (off, shape) in enumerate(self.views):
            size = 1
            for d in shape:
                size *= d
            dst = out[off:off + size]
            if len(shape) >= 2:
                n, m = shape[0], size // shape[0]
                noise = torch.randn(n, m, generator=self._gen(vi, _ROLE_NOISE, step),
                                    device=self.device)
                dst.copy_((self._low_rank(vi, n, m) + cfg.noise_std * noise).reshape(-1))
            else:
                dst.copy_(torch.randn(size, generator=self._gen(vi, _ROLE_VEC, step),
                                      device=self.device))
        return out

    def inf_injected(self, step: int, forced: bool = True) -> bool:
        """Whether `step` carries an injected inf: the workload's Bernoulli draw, plus
        the forced steps of the correctness runs when `forced`."""
        cfg = self.cfg
        if cfg.dtype != "f16":
            return False
        if forced and step in cfg.forced_inf_steps:
            return True
        if cfg.inf_probability <= 0.0:
            return False
        g = torch.Generator().manual_seed(_seed(cfg.seed, 0, _ROLE_INF, step))
        return bool(torch.rand(1, generator=g).item() < cfg.inf_probability)

    def bucket(self, step: int, loss_scale: Optional[float] = None,
               inject_inf: Optional[bool] = None, forced: bool = True) -> torch.Tensor:
        """The stored bucket of `step`: fp32 gradients, or loss-scaled fp16 ones."""
        cfg = self.cfg
        g = self.gradient(step)
        if cfg.dtype == "f32":
            return g * cfg.grad_scale if cfg.grad_scale != 1.0 else g
        scale = cfg.loss_scale if loss_scale is None else loss_scale
        h = (g * (cfg.amp_prescale * scale)).to(torch.float16)
        if inject_inf is None:
            inject_inf = self.inf_injected(step, forced)
        if inject_inf:
            gen = torch.Generator().manual_seed(_seed(cfg.seed, 1, _ROLE_INF, step))
            pos = int(torch.randint(0, cfg.numel, (1,), generator=gen).item())
            h[pos] = float("inf")
        return h
