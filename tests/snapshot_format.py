"""Reader of the version-1 state snapshot for the tests (independent of the library's
and the oracle's own readers): header fields, bucket records with their views, and the
E and Q arrays of every compressed view. The compressed views and their ranks are
decided by `classify(shape) -> None | (n, m, k)` for per-layer buckets; a batched
bucket's one s x s view has rank min(r, s). The record's variant word keeps the
batched flag in bit 0 and a 16-bit state's precision in bits 8-9."""
from __future__ import annotations

import struct
from typing import Callable, Optional, Tuple

import numpy as np

HEADER = struct.Struct("<8sIIiIdQqqqqq")
HEADER_FIELDS = ("magic", "version", "flags", "rank", "reserved", "min_compression_rate",
                 "random_seed", "iteration", "numel_in", "numel_comm", "next_log_iteration",
                 "nbuckets")
BUCKET = struct.Struct("<qqIIq")


def parse(blob: bytes, classify: Callable[[Tuple[int, ...]], Optional[Tuple[int, int, int]]]):
    blob = bytes(blob)
    head = dict(zip(HEADER_FIELDS, HEADER.unpack_from(blob, 0)))
    pos = HEADER.size
    ef = bool(head["flags"] & 1)
    buckets = []
    for _ in range(head["nbuckets"]):
        idx, numel, variant, has_q, nviews = BUCKET.unpack_from(blob, pos)
        batched = variant & 1
        pos += BUCKET.size
        views = []
        for _ in range(nviews):
            off, ndim = struct.unpack_from("<qq", blob, pos)
            pos += 16
            shp = struct.unpack_from(f"<{ndim}q", blob, pos)
            pos += 8 * ndim
            views.append((off, tuple(shp)))
        rec = {"index": idx, "numel": numel, "variant": variant, "has_q": has_q,
               "views": views, "E": {}, "Q": {}}
        for vi, (_, shp) in enumerate(views):
            if batched:
                n = m = shp[0]
                k = min(head["rank"], n)
            else:
                c = classify(shp)
                if c is None:
                    continue
                n, m, k = c
            if ef:
                rec["E"][vi] = np.frombuffer(blob, "<f4", n * m, pos).reshape(n, m)
                pos += 4 * n * m
            if has_q:
                rec["Q"][vi] = np.frombuffer(blob, "<f4", m * k, pos).reshape(m, k)
                pos += 4 * m * k
        buckets.append(rec)
    assert pos == len(blob), (pos, len(blob))
    return head, buckets
