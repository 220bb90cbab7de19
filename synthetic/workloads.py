"""The benchmark workloads as bucket layouts plus generator parameters.

Each workload is a flat gradient bucket of parameter-shaped views packed
back to back with no padding, in the order listed, the way a data-parallel
gradient bucket flattens per-parameter tensors. Shapes follow the models the
workloads are named after; values are synthetic (low rank plus noise), so no
dataset or trained weight is involved.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Tuple

Shape = Tuple[int, ...]


@dataclass
class WorkloadConfig:
    name: str
    shapes: List[Shape]
    # hyperparameters passed to the compressor (names as PowerSGDState names them)
    hparams: Dict[str, object]
    steps: int
    spectrum_rank: int            # k: true rank of the low-rank part
    spectrum_power: float         # singular-value weights s_j = j ** -power, j = 1..k
    noise_std: float = 0.01
    dtype: str = "f32"            # "f32" or "f16" (loss-scaled gradients)
    amp_prescale: float = 1.0     # f16 only: gradient multiplier before the loss scale
    loss_scale: float = 1.0       # f16 only: initial loss scale
    inf_probability: float = 0.0  # f16 only: per-step chance of an injected inf
    forced_inf_steps: Tuple[int, ...] = ()
    seed: int = 0
    notes: str = ""
    batched: bool = False         # the whole bucket as one zero-padded square matrix
    wrap: str = ""                # "f16" / "bf16": the hook under fp16/bf16_compress_wrapper
    grad_scale: float = 1.0       # f32 only: gradient multiplier (a power of two: exact)

    def views(self):
        return packed_views(self.shapes)

    @property
    def numel(self) -> int:
        return sum(_numel(s) for s in self.shapes)

    @property
    def element_bytes(self) -> int:
        return 2 if self.dtype == "f16" else 4


def _numel(shape: Shape) -> int:
    n = 1
    for d in shape:
        n *= int(d)
    return n


def packed_views(shapes: List[Shape]):
    """[(offset, shape)] for shapes packed contiguously from offset 0."""
    out = []
    off = 0
    for s in shapes:
        out.append((off, tuple(int(d) for d in s)))
        off += _numel(s)
    return out


def _resnet50_shapes() -> List[Shape]:
    conv = ([(64, 3, 7, 7)] + [(64, 64, 3, 3)] * 6 + [(256, 64, 1, 1)] * 7
            + [(128, 128, 3, 3)] * 4 + [(512, 128, 1, 1)] * 4 + [(256, 256, 3, 3)] * 6
            + [(1024, 256, 1, 1)] * 6 + [(512, 512, 3, 3)] * 3 + [(2048, 512, 1, 1)] * 3
            + [(1000, 2048)])
    cycle = (64, 128, 256, 512, 1024, 2048)
    vectors = [(cycle[i % len(cycle)],) for i in range(53)]
    return conv + vectors


def _bert_large_shapes() -> List[Shape]:
    layer = ([(1024, 1024)] * 4 + [(4096, 1024), (1024, 4096)]
             + [(1024,)] * 4 + [(4096,), (1024,)] + [(1024,)] * 4)
    return layer * 24


def _gpt_shapes() -> List[Shape]:
    layer = [(4096, 4096)] * 3 + [(4096, 16384), (16384, 4096)]
    return layer * 8


_BASE = dict(start_powerSGD_iter=0, min_compression_rate=2.0, use_error_feedback=True,
             warm_start=True, orthogonalization_epsilon=0.0, random_seed=0,
             batch_tensors_with_same_shape=False)


def _hp(**kw):
    d = dict(_BASE)
    d.update(kw)
    return d


CONFIGS: Dict[int, WorkloadConfig] = {
    0: WorkloadConfig(
        name="single-256x512-r1", shapes=[(256, 512)],
        hparams=_hp(matrix_approximation_rank=1), steps=3,
        spectrum_rank=8, spectrum_power=1.0, seed=1000),
    1: WorkloadConfig(
        name="resnet50-bucket-r2", shapes=_resnet50_shapes(),
        hparams=_hp(matrix_approximation_rank=2), steps=10,
        spectrum_rank=8, spectrum_power=1.0, seed=1001),
    2: WorkloadConfig(
        name="bert-large-bucket-r4-batched", shapes=_bert_large_shapes(),
        hparams=_hp(matrix_approximation_rank=4, batch_tensors_with_same_shape=True),
        steps=20, spectrum_rank=64, spectrum_power=1.0, seed=1002),
    3: WorkloadConfig(
        name="gpt-bucket-r32", shapes=_gpt_shapes(),
        hparams=_hp(matrix_approximation_rank=32, orthogonalization_epsilon=1e-8),
        steps=10, spectrum_rank=128, spectrum_power=0.5, seed=1003),
    4: WorkloadConfig(
        name="bert-large-bucket-r4-amp-fp16", shapes=_bert_large_shapes(),
        hparams=_hp(matrix_approximation_rank=4, batch_tensors_with_same_shape=True),
        steps=20, spectrum_rank=64, spectrum_power=1.0, dtype="f16",
        amp_prescale=2.0 ** -10, loss_scale=65536.0, inf_probability=0.001,
        forced_inf_steps=(10,), seed=1004,
        notes="fp16 value = RNE(G * 2^-10 * S); the 2^-10 keeps |value| below the fp16 "
              "maximum at S = 65536"),
    5: WorkloadConfig(
        name="resnet50-bucket-batched-r1", shapes=_resnet50_shapes(),
        hparams=_hp(matrix_approximation_rank=1), steps=10,
        spectrum_rank=8, spectrum_power=1.0, seed=1001, batched=True,
        notes="the ResNet-50 bucket (same values as the per-layer workload) viewed as one "
              "4315 x 4315 matrix, 4313 padded zeros; rank 1 as the pages recommend for "
              "this variant"),
    6: WorkloadConfig(
        name="resnet50-bucket-r2-bf16-wrapper", shapes=_resnet50_shapes(),
        hparams=_hp(matrix_approximation_rank=2), steps=10,
        spectrum_rank=8, spectrum_power=1.0, seed=1001, wrap="bf16",
        notes="the ResNet-50 fp32 bucket under bf16_compress_wrapper(powerSGD_hook)"),
    7: WorkloadConfig(
        name="bert-large-bucket-r4-fp16-wrapper", shapes=_bert_large_shapes(),
        hparams=_hp(matrix_approximation_rank=4, batch_tensors_with_same_shape=True),
        steps=20, spectrum_rank=64, spectrum_power=1.0, seed=1002, wrap="f16",
        grad_scale=2.0 ** -10,
        notes="the BERT-large fp32 bucket, gradients x 2^-10, under "
              "fp16_compress_wrapper(powerSGD_hook); unscaled, the warm-started P = M'Q "
              "(about sigma^2, 1e6 here) would overflow binary16"),
    8: WorkloadConfig(
        name="gpt-bucket-r32-bf16-wrapper", shapes=_gpt_shapes(),
        hparams=_hp(matrix_approximation_rank=32, orthogonalization_epsilon=1e-8),
        steps=10, spectrum_rank=128, spectrum_power=0.5, seed=1003, wrap="bf16",
        notes="the GPT-style fp32 bucket under bf16_compress_wrapper(powerSGD_hook), "
              "rank 32 on the matrix cores"),
}


def shrink_config(cfg: WorkloadConfig, shapes: List[Shape], steps: int = None,
                  name: str = None) -> WorkloadConfig:
    """A copy of `cfg` with other view shapes (for oracle-sized parity cases)."""
    return WorkloadConfig(
        name=name or (cfg.name + "-small"), shapes=list(shapes), hparams=dict(cfg.hparams),
        steps=cfg.steps if steps is None else steps, spectrum_rank=cfg.spectrum_rank,
        spectrum_power=cfg.spectrum_power, noise_std=cfg.noise_std, dtype=cfg.dtype,
        amp_prescale=cfg.amp_prescale, loss_scale=cfg.loss_scale,
        inf_probability=cfg.inf_probability, forced_inf_steps=cfg.forced_inf_steps,
        seed=cfg.seed, notes=cfg.notes, batched=cfg.batched, wrap=cfg.wrap,
        grad_scale=cfg.grad_scale)
