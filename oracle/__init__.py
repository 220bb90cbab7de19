"""fp64 CPU oracle for PowerSGD bucket compression.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg, never by the product path. It shares no code with
the HIP library and imports nothing from it.

Parity status per function (what pins each one is listed in the tests):
  rng.philox4x64_10, rng.mulhilo64 .... pinned (numpy.random.Philox, Python ints)
  rng.box_muller ...................... pinned (closed-form points, distribution)
  rng.standard_normal_q0 .............. pinned (layout/key invariants, distribution)
  powersgd.should_compress ............ pinned (brute-force integer arithmetic)
  powersgd.gram_schmidt ............... pinned (QR uniqueness, Householder QR,
                                        closed forms for epsilon > 0, a 200-bit
                                        mpmath run at condition number 1e14, the
                                        rank-deficient trajectory's E = 0)
  ddarith (double-double steps) ....... pinned (exact rationals for TwoSum,
                                        TwoProduct, sums and dot products)
  OracleState.compress_bucket ......... pinned (rational projection, hand-worked
                                        example, invariants, Eckart-Young limit)
  powersgd.batched_side ............... pinned (brute force over integers)
  OracleState.compress_bucket_batched . pinned (hand-worked two-step example,
                                        exact rank-1 recovery, error-feedback
                                        identity over the padding, fp16 cases)
  OracleState.export_state/import_state  pinned (fields written out by hand, closed-
                                        form length, round trip, rejections)
  lowp.round_f16, lowp.round_bf16 ..... pinned (hand-worked ties and overflow,
                                        torch's binary32 -> bfloat16 conversion,
                                        nearest-value brute force on bit patterns)
  lowp.compress_matrix_step_lowp,
  OracleState.compress_bucket_wrapped . pinned (exact single-row recovery, 16-bit
                                        fixed points, error-feedback identity, the
                                        fp64 hook within 16u, the wrapper's casts)
"""
from .powersgd import (HParams, LayoutChanged, OracleState, StepResult, ViewResult,
                       any_nonfinite, batched_side, compress_matrix_step,
                       effective_rank, gram_schmidt, matrix_view, should_compress)
from .lowp import compress_matrix_step_lowp, round_bf16, round_f16
from .rng import box_muller, mulhilo64, philox4x64_10, standard_normal_q0

__all__ = [
    "HParams", "LayoutChanged", "OracleState", "StepResult", "ViewResult",
    "any_nonfinite", "batched_side", "compress_matrix_step",
    "effective_rank", "gram_schmidt", "matrix_view", "should_compress",
    "box_muller", "mulhilo64", "philox4x64_10", "standard_normal_q0",
    "compress_matrix_step_lowp", "round_bf16", "round_f16",
]
