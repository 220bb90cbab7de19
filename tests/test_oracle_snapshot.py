"""Pins of the oracle's state snapshot (export_state / import_state) and of its call
bookkeeping (statistics on skipped fp16 calls, the logging schedule).

The snapshot format is the library's documented version-1 layout; the pages give no
checkpoint format. The fixture tests/golden/snapshot_v1_fields.json lists its fields
by hand, so a wrong field order, width or count in the oracle fails here."""
import json
import os
import struct

import numpy as np
import pytest

import oracle
from oracle.powersgd import _BucketMemory

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "snapshot_v1_fields.json")
PACK = {"char8": "8s", "u32": "<I", "i32": "<i", "u64": "<Q", "i64": "<q", "f64": "<d"}


def _fixture():
    with open(GOLDEN) as f:
        return json.load(f)


def _pack_fields(fields):
    out = b""
    for kind, value, _ in fields:
        if kind == "f32":
            out += struct.pack(f"<{len(value)}f", *value)
        elif kind == "char8":
            out += struct.pack("8s", value.encode())
        else:
            out += struct.pack(PACK[kind], value)
    return out


def _fixture_state(fx):
    st = oracle.OracleState(oracle.HParams(**fx["hparams"]))
    s = fx["state"]
    st.iteration, st.numel_in = s["iteration"], s["numel_in"]
    st.numel_comm, st.next_log_iteration = s["numel_comm"], s["next_log_iteration"]
    for b in s["buckets"]:
        layout = (("batched", b["numel"]) if b["batched"]
                  else tuple((off, tuple(shp)) for off, shp in b["views"]))
        mem = _BucketMemory(layout=layout, numel=b["numel"])
        for v, eq in b["compressed"].items():
            mem.error[int(v)] = np.array(eq["E"], dtype=np.float64)
            mem.q[int(v)] = np.array(eq["Q"], dtype=np.float64)
        st.buckets[b["index"]] = mem
    return st


def test_export_writes_the_documented_fields():
    fx = _fixture()
    want = _pack_fields(fx["fields"])
    assert len(want) == fx["total_bytes"]
    assert _fixture_state(fx).export_state() == want


def test_import_reads_the_documented_fields():
    fx = _fixture()
    st = oracle.OracleState(oracle.HParams(**fx["hparams"]))
    st.import_state(_pack_fields(fx["fields"]))
    s = fx["state"]
    assert (st.iteration, st.numel_in, st.numel_comm, st.next_log_iteration) == (
        s["iteration"], s["numel_in"], s["numel_comm"], s["next_log_iteration"])
    assert sorted(st.buckets) == [b["index"] for b in s["buckets"]]
    for b in s["buckets"]:
        mem = st.buckets[b["index"]]
        assert mem.numel == b["numel"]
        if b["batched"]:
            assert mem.layout == ("batched", b["numel"])
        else:
            assert mem.layout == tuple((off, tuple(shp)) for off, shp in b["views"])
        for v, eq in b["compressed"].items():
            np.testing.assert_array_equal(mem.error[int(v)], np.array(eq["E"]))
            np.testing.assert_array_equal(mem.q[int(v)], np.array(eq["Q"]))


def _views():
    # a compressed conv-like view, a vector, a matrix the rate test keeps whole, and a
    # second compressed matrix
    return [(0, (16, 3, 3, 3)), (432, (16,)), (448, (4, 4)), (464, (24, 20))]


def _bucket(step, numel=944, seed=3):
    rng = np.random.default_rng(seed * 100 + step)
    return rng.standard_normal(numel).astype(np.float32)


def _hp(**kw):
    base = dict(matrix_approximation_rank=2, start_powerSGD_iter=0,
                compression_stats_logging_frequency=0, random_seed=5)
    base.update(kw)
    return oracle.HParams(**base)


@pytest.mark.parametrize("ef,warm", [(True, True), (True, False), (False, True)])
def test_round_trip_and_continuation(ef, warm):
    hp = _hp(use_error_feedback=ef, warm_start=warm)
    a = oracle.OracleState(hp)
    for t in range(3):
        a.compress_bucket(_bucket(t), _views(), bucket_index=1)
        a.compress_bucket_batched(_bucket(t, 50), bucket_index=4)
    blob = a.export_state()
    b = oracle.OracleState(hp)
    b.import_state(blob)
    assert b.export_state() == blob
    # the snapshot rounds E and Q to binary32: continuing from it stays within that
    # rounding of continuing from the fp64 state
    for t in range(3, 5):
        ra = a.compress_bucket(_bucket(t), _views(), bucket_index=1)
        rb = b.compress_bucket(_bucket(t), _views(), bucket_index=1)
        d = np.linalg.norm(ra.output64 - rb.output64) / np.linalg.norm(ra.output64)
        assert d < 1e-5, d
        ra = a.compress_bucket_batched(_bucket(t, 50), bucket_index=4)
        rb = b.compress_bucket_batched(_bucket(t, 50), bucket_index=4)
        d = np.linalg.norm(ra.output64 - rb.output64) / np.linalg.norm(ra.output64)
        assert d < 1e-5, d
    assert (a.iteration, a.numel_in, a.numel_comm) == (b.iteration, b.numel_in, b.numel_comm)


def test_snapshot_length_closed_form():
    hp = _hp()
    a = oracle.OracleState(hp)
    a.compress_bucket(_bucket(0), _views(), bucket_index=1)
    a.compress_bucket_batched(_bucket(0, 50), bucket_index=4)
    views_bytes = sum(16 + 8 * len(shp) for _, shp in _views())
    # compressed: 16 x 27 and 24 x 20 at rank 2; the batched bucket: 8 x 8 at rank 2
    per_layer = 32 + views_bytes + 4 * (16 * 27 + 27 * 2) + 4 * (24 * 20 + 20 * 2)
    batched = 32 + 32 + 4 * (8 * 8 + 8 * 2)
    assert len(a.export_state()) == 80 + per_layer + batched


def _corrupt(blob, pos, fmt, value):
    b = bytearray(blob)
    struct.pack_into(fmt, b, pos, value)
    return bytes(b)


def test_import_rejects_malformed_snapshots_and_keeps_the_state():
    hp = _hp()
    a = oracle.OracleState(hp)
    a.compress_bucket(_bucket(0), _views(), bucket_index=1)
    a.compress_bucket_batched(_bucket(0, 50), bucket_index=4)
    blob = a.export_state()
    b = oracle.OracleState(hp)
    b.compress_bucket(_bucket(9), _views(), bucket_index=2)
    before = b.export_state()
    bad = [
        b"XSGDSNAP" + blob[8:],                      # magic
        _corrupt(blob, 8, "<I", 2),                  # version
        _corrupt(blob, 12, "<I", 1),                 # flags (warm start missing)
        _corrupt(blob, 16, "<i", 3),                 # rank
        _corrupt(blob, 20, "<I", 1),                 # reserved
        _corrupt(blob, 24, "<d", 2.5),               # min_compression_rate
        _corrupt(blob, 32, "<Q", 6),                 # random_seed
        _corrupt(blob, 40, "<q", -1),                # iteration
        _corrupt(blob, 72, "<q", 3),                 # bucket count past the end
        _corrupt(blob, 80 + 8, "<q", 10),            # numel: views leave the bucket
        _corrupt(blob, 80 + 16, "<I", 2),            # batched flag out of range
        blob[:-1],                                   # truncated
        blob + b"\0",                                # trailing byte
    ]
    for data in bad:
        with pytest.raises(ValueError):
            b.import_state(data)
        assert b.export_state() == before
    # bucket indices must ascend: swap the two records
    first_len = len(blob) - 80 - (32 + 32 + 4 * (8 * 8 + 8 * 2))
    recs = blob[80:80 + first_len], blob[80 + first_len:]
    with pytest.raises(ValueError):
        b.import_state(blob[:80] + recs[1] + recs[0])
    # a warm-start Q in a snapshot for a state without warm start
    c = oracle.OracleState(_hp(warm_start=False))
    with pytest.raises(ValueError):
        c.import_state(_corrupt(blob, 12, "<I", 1))


def test_skipped_fp16_calls_count_in_the_statistics():
    hp = _hp(start_powerSGD_iter=1)
    st = oracle.OracleState(hp)
    views = _views()
    good = _bucket(0).astype(np.float16)
    bad = good.copy()
    bad[500] = np.inf
    st.compress_bucket(bad, views)           # before the start iteration: not counted
    assert (st.iteration, st.numel_in, st.numel_comm) == (1, 0, 0)
    st.compress_bucket(bad, views)           # skipped, but counted
    numel = 944
    comm = (16 + 27) * 2 + 16 + 16 + (24 + 20) * 2
    assert (st.iteration, st.numel_in, st.numel_comm) == (2, numel, comm)
    assert not st.buckets                    # nothing memorized
    st.compress_bucket(good, views)
    assert (st.iteration, st.numel_in, st.numel_comm) == (3, 2 * numel, 2 * comm)
    # the batched variant: numel in, 2 s r out
    bb = _bucket(1, 50).astype(np.float16)
    bb[3] = np.nan
    st.compress_bucket_batched(bb, bucket_index=7)
    assert (st.numel_in, st.numel_comm) == (2 * numel + 50, 2 * comm + 2 * 8 * 2)


def test_logging_schedule():
    # start 2, every 3 iterations: lines due at iterations 2, 5, 8
    st = oracle.OracleState(_hp(start_powerSGD_iter=2, compression_stats_logging_frequency=3))
    seen = []
    for t in range(9):
        st.compress_bucket(_bucket(t), _views())
        seen.append(st.next_log_iteration)
    assert seen == [2, 2, 5, 5, 5, 8, 8, 8, 11]
    # a bucket that is not the last of its iteration moves nothing
    st.compress_bucket(_bucket(9), _views(), bucket_index=3, is_last=False)
    assert (st.iteration, st.next_log_iteration) == (9, 11)


@pytest.mark.parametrize("dt,code", [("f16", 1), ("bf16", 2)])
def test_wrapped_buckets_record_their_precision(dt, code):
    hp = _hp()
    a = oracle.OracleState(hp)
    for t in range(2):
        a.compress_bucket_wrapped(_bucket(t), _views(), dt, bucket_index=6)
    blob = a.export_state()
    # the one bucket record follows the header: index, numel, then the variant word
    idx, numel, variant = struct.unpack_from("<qqI", blob, 80)
    assert (idx, numel, variant) == (6, 944, code << 8)
    b = oracle.OracleState(hp)
    b.import_state(blob)
    assert b.export_state() == blob
    assert b.buckets[6].layout == ("wrapped", dt, tuple(_views()))
    ra = a.compress_bucket_wrapped(_bucket(2), _views(), dt, bucket_index=6)
    rb = b.compress_bucket_wrapped(_bucket(2), _views(), dt, bucket_index=6)
    np.testing.assert_array_equal(ra.output, rb.output)   # 16-bit state: nothing lost
    # a value that is not 16-bit is rounded into the 16-bit state on import
    first_e = 80 + 32 + sum(16 + 8 * len(shp) for _, shp in _views())
    x = bytearray(blob)
    struct.pack_into("<f", x, first_e, 1.0 + 2.0 ** -20)
    b.import_state(bytes(x))
    assert b.buckets[6].error[0][0, 0] == 1.0
    # precision code 3 and other bits do not exist
    for bad in (3 << 8, code << 10, 1 << 4):
        with pytest.raises(ValueError):
            b.import_state(_corrupt(blob, 96, "<I", bad))


@pytest.mark.parametrize("dt,code", [("f16", 1), ("bf16", 2)])
def test_batched_wrapped_buckets_record_batched_and_precision(dt, code):
    hp = _hp()
    a = oracle.OracleState(hp)
    for t in range(2):
        a.compress_bucket_batched_wrapped(_bucket(t, 50), dt, bucket_index=9)
    blob = a.export_state()
    idx, numel, variant = struct.unpack_from("<qqI", blob, 80)
    assert (idx, numel, variant) == (9, 50, 1 | (code << 8))
    b = oracle.OracleState(hp)
    b.import_state(blob)
    assert b.export_state() == blob and b.buckets[9].layout == ("batched", 50, dt)
    ra = a.compress_bucket_batched_wrapped(_bucket(2, 50), dt, bucket_index=9)
    rb = b.compress_bucket_batched_wrapped(_bucket(2, 50), dt, bucket_index=9)
    np.testing.assert_array_equal(ra.output, rb.output)
