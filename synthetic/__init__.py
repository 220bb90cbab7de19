"""Seeded synthetic gradient buckets, shared by the tests, the benchmark and the
oracle-side checks. This package holds workload shapes and random inputs only:
none of the compression method's arithmetic lives here."""
from .workloads import CONFIGS, WorkloadConfig, packed_views, shrink_config
from .generate import BucketGenerator

__all__ = ["CONFIGS", "WorkloadConfig", "packed_views", "shrink_config", "BucketGenerator"]
