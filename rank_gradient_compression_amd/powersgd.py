"""ctypes binding of libpowersgd.so (include/powersgd.h), argument marshalling only.

The module-level functions carry the C names and forward to the library; every
step of the compression runs in the HIP kernels. `PowerSGDState` is a small
convenience wrapper over them that accepts torch tensors for device memory and
torch streams. There is no CPU fallback: if the library is missing, loading fails.
"""
from __future__ import annotations

import array
import ctypes
import os
from typing import Iterable, List, Optional, Sequence, Tuple

from . import build as _build

POWERSGD_OK = 0
POWERSGD_ERR_INVALID_ARG = -1
POWERSGD_ERR_LAYOUT_CHANGED = -2
POWERSGD_ERR_OOM = -3
POWERSGD_ERR_HIP = -4
POWERSGD_ERR_UNSUPPORTED = -5
POWERSGD_ERR_NOT_FOUND = -6
POWERSGD_F32 = 0
POWERSGD_F16 = 1
POWERSGD_BF16 = 2
POWERSGD_MAX_NDIM = 8
POWERSGD_MAX_RANK = 32
POWERSGD_NUM_KERNELS = 8

# Every function the header declares, for load checks.
EXPORTED = (
    "powersgd_hparams_init", "powersgd_state_create", "powersgd_state_destroy",
    "powersgd_compress_bucket", "powersgd_status_string", "powersgd_last_error",
    "powersgd_get_decisions", "powersgd_get_view_info", "powersgd_copy_factors",
    "powersgd_copy_error", "powersgd_get_stats", "powersgd_set_timing",
    "powersgd_get_kernel_times", "powersgd_kernel_name", "powersgd_classify_view",
    "powersgd_batched_side", "powersgd_compress_bucket_batched",
    "powersgd_state_export", "powersgd_state_import", "powersgd_compress_bucket_wrapped",
    "powersgd_compress_bucket_batched_wrapped", "powersgd_get_factors", "powersgd_get_error",
    "powersgd_draw_q0", "powersgd_compress_matrix_noalloc",
)


class powersgd_hparams(ctypes.Structure):
    _fields_ = [
        ("matrix_approximation_rank", ctypes.c_int32),
        ("start_powerSGD_iter", ctypes.c_int64),
        ("min_compression_rate", ctypes.c_double),
        ("use_error_feedback", ctypes.c_int32),
        ("warm_start", ctypes.c_int32),
        ("orthogonalization_epsilon", ctypes.c_double),
        ("random_seed", ctypes.c_uint64),
        ("compression_stats_logging_frequency", ctypes.c_int64),
        ("batch_tensors_with_same_shape", ctypes.c_int32),
    ]


class powersgd_view(ctypes.Structure):
    _fields_ = [
        ("offset", ctypes.c_int64),
        ("ndim", ctypes.c_int32),
        ("shape", ctypes.c_int64 * POWERSGD_MAX_NDIM),
    ]


class PowerSGDError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_string(status)} ({status}): {detail}")


_lib: Optional[ctypes.CDLL] = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Loads the built library (raises if it has not been built). The environment
    variable RGC_POWERSGD_LIBRARY may name another build of it."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    path = path or os.environ.get("RGC_POWERSGD_LIBRARY") or _build.library_path()
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it first (python -m rank_gradient_compression_amd.build)")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    i32, i64, f32, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double
    sigs = {
        "powersgd_hparams_init": (None, [ctypes.POINTER(powersgd_hparams)]),
        "powersgd_state_create": (i32, [ctypes.POINTER(powersgd_hparams), i32,
                                        ctypes.POINTER(P)]),
        "powersgd_state_destroy": (None, [P]),
        "powersgd_compress_bucket": (i32, [P, i64, i32, P, i32, i64,
                                           ctypes.POINTER(powersgd_view), i32, f32, P, P]),
        "powersgd_batched_side": (i64, [i64]),
        "powersgd_compress_bucket_wrapped": (i32, [P, i64, i32, P, i32, i64,
                                                   ctypes.POINTER(powersgd_view), i32, P]),
        "powersgd_compress_bucket_batched_wrapped": (i32, [P, i64, i32, P, i32, i64, i64, P]),
        "powersgd_compress_bucket_batched": (i32, [P, i64, i32, P, i32, i64, i64, f32, P, P]),
        "powersgd_status_string": (ctypes.c_char_p, [i32]),
        "powersgd_last_error": (ctypes.c_char_p, []),
        "powersgd_get_decisions": (i32, [P, i64, ctypes.POINTER(ctypes.c_uint8), i32]),
        "powersgd_get_view_info": (i32, [P, i64, i32, ctypes.POINTER(i64),
                                         ctypes.POINTER(i64), ctypes.POINTER(i32)]),
        "powersgd_copy_factors": (i32, [P, i64, i32, P, P, P]),
        "powersgd_copy_error": (i32, [P, i64, i32, P, P]),
        "powersgd_get_factors": (i32, [P, i64, i32, ctypes.POINTER(P), ctypes.POINTER(P),
                                       ctypes.POINTER(i64), ctypes.POINTER(i64),
                                       ctypes.POINTER(i32)]),
        "powersgd_get_error": (i32, [P, i64, ctypes.POINTER(P)]),
        "powersgd_draw_q0": (i32, [ctypes.c_uint64, i64, i32, ctypes.c_uint64, i64, i32, P, P,
                                   P]),
        "powersgd_compress_matrix_noalloc": (i32, [ctypes.POINTER(powersgd_hparams), i64, i32,
                                                   ctypes.c_uint64, P, i64, i64, P, P, i32, P,
                                                   P]),
        "powersgd_get_stats": (i32, [P, ctypes.POINTER(i64), ctypes.POINTER(i64),
                                     ctypes.POINTER(i64)]),
        "powersgd_set_timing": (i32, [P, i32]),
        "powersgd_get_kernel_times": (i32, [P, ctypes.POINTER(f64), ctypes.POINTER(i64),
                                            ctypes.POINTER(f64)]),
        "powersgd_kernel_name": (ctypes.c_char_p, [i32]),
        "powersgd_state_export": (i32, [P, P, i64, ctypes.POINTER(i64), P]),
        "powersgd_state_import": (i32, [P, P, i64, P]),
        "powersgd_classify_view": (i32, [ctypes.POINTER(powersgd_hparams),
                                         ctypes.POINTER(powersgd_view), ctypes.POINTER(i32),
                                         ctypes.POINTER(i64), ctypes.POINTER(i64),
                                         ctypes.POINTER(i32)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != POWERSGD_OK:
        raise PowerSGDError(status, powersgd_last_error())


# ------------------------------------------------------- C functions, same names

def powersgd_hparams_init() -> powersgd_hparams:
    hp = powersgd_hparams()
    load_library().powersgd_hparams_init(ctypes.byref(hp))
    return hp


def powersgd_state_create(hp: powersgd_hparams, device: int = 0) -> ctypes.c_void_p:
    out = ctypes.c_void_p()
    _check(load_library().powersgd_state_create(ctypes.byref(hp), device, ctypes.byref(out)))
    return out


def powersgd_state_destroy(state) -> None:
    load_library().powersgd_state_destroy(state)


def status_string(status: int) -> str:
    return load_library().powersgd_status_string(status).decode()


powersgd_status_string = status_string


def powersgd_last_error() -> str:
    return load_library().powersgd_last_error().decode()


# offset, ndim, shape[POWERSGD_MAX_NDIM] as 64-bit words: ndim is an int32 followed by
# four bytes of alignment padding, so on this little-endian target the word holding it
# carries its value in the low half and zero in the padding
_VIEW_WORDS = 2 + POWERSGD_MAX_NDIM


class PreparedViews:
    """A views list marshalled once into the C array the library reads. Every function
    that takes `views` also takes one of these, which spares a per-call conversion
    when the same layout is compressed every step (as a DDP hook does per bucket)."""

    __slots__ = ("array", "count")

    def __init__(self, views: Sequence[Tuple[int, Sequence[int]]]):
        self.array = _marshal_views(views)
        self.count = len(views)

    def __len__(self) -> int:
        return self.count


def _marshal_views(views) -> ctypes.Array:
    n = len(views)
    flat = [0] * (_VIEW_WORDS * max(1, n))
    for i, (off, shape) in enumerate(views):
        nd = len(shape)
        if nd > POWERSGD_MAX_NDIM:
            raise ValueError(f"view {i}: more than {POWERSGD_MAX_NDIM} dimensions")
        b = i * _VIEW_WORDS
        flat[b] = off
        flat[b + 1] = nd
        flat[b + 2:b + 2 + nd] = shape
    # integers only (a float offset or dimension raises TypeError); the ctypes array
    # keeps the buffer alive
    return (powersgd_view * max(1, n)).from_buffer(array.array("q", flat))


def _views_arg(views):
    return views if isinstance(views, PreparedViews) else list(views)


def make_views(views):
    """The C array of powersgd_view for `views` ((offset, shape) pairs, or PreparedViews)."""
    if isinstance(views, PreparedViews):
        return views.array
    return _marshal_views(views)


def powersgd_compress_bucket(state, bucket_index: int, is_last: bool, bucket_ptr: int,
                             dtype: int, numel: int, views, inv_loss_scale: float,
                             found_inf_ptr: Optional[int], stream: Optional[int]) -> None:
    arr = make_views(views)
    _check(load_library().powersgd_compress_bucket(
        state, int(bucket_index), int(bool(is_last)), ctypes.c_void_p(bucket_ptr), int(dtype),
        int(numel), arr, len(views), float(inv_loss_scale),
        ctypes.c_void_p(found_inf_ptr) if found_inf_ptr else None,
        ctypes.c_void_p(stream) if stream else None))


def powersgd_compress_bucket_wrapped(state, bucket_index: int, is_last: bool,
                                     bucket_ptr: int, compute_dtype: int, numel: int, views,
                                     stream: Optional[int]) -> None:
    arr = make_views(views)
    _check(load_library().powersgd_compress_bucket_wrapped(
        state, int(bucket_index), int(bool(is_last)), ctypes.c_void_p(bucket_ptr),
        int(compute_dtype), int(numel), arr, len(views),
        ctypes.c_void_p(stream) if stream else None))


def powersgd_compress_bucket_batched_wrapped(state, bucket_index: int, is_last: bool,
                                             bucket_ptr: int, compute_dtype: int, numel: int,
                                             capacity: int, stream: Optional[int]) -> None:
    _check(load_library().powersgd_compress_bucket_batched_wrapped(
        state, int(bucket_index), int(bool(is_last)), ctypes.c_void_p(bucket_ptr),
        int(compute_dtype), int(numel), int(capacity),
        ctypes.c_void_p(stream) if stream else None))


def powersgd_batched_side(numel: int) -> int:
    return int(load_library().powersgd_batched_side(int(numel)))


def powersgd_compress_bucket_batched(state, bucket_index: int, is_last: bool, bucket_ptr: int,
                                     dtype: int, numel: int, capacity: int,
                                     inv_loss_scale: float, found_inf_ptr: Optional[int],
                                     stream: Optional[int]) -> None:
    _check(load_library().powersgd_compress_bucket_batched(
        state, int(bucket_index), int(bool(is_last)), ctypes.c_void_p(bucket_ptr), int(dtype),
        int(numel), int(capacity), float(inv_loss_scale),
        ctypes.c_void_p(found_inf_ptr) if found_inf_ptr else None,
        ctypes.c_void_p(stream) if stream else None))


def powersgd_get_decisions(state, bucket_index: int, nviews: int) -> List[int]:
    out = (ctypes.c_uint8 * max(1, nviews))()
    _check(load_library().powersgd_get_decisions(state, bucket_index, out, nviews))
    return [int(out[i]) for i in range(nviews)]


def powersgd_get_view_info(state, bucket_index: int, view: int) -> Tuple[int, int, int]:
    n, m, r = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(load_library().powersgd_get_view_info(state, bucket_index, view, ctypes.byref(n),
                                                 ctypes.byref(m), ctypes.byref(r)))
    return n.value, m.value, r.value


def powersgd_copy_factors(state, bucket_index: int, view: int, p_ptr: Optional[int],
                          q_ptr: Optional[int], stream: Optional[int]) -> None:
    _check(load_library().powersgd_copy_factors(
        state, bucket_index, view, ctypes.c_void_p(p_ptr) if p_ptr else None,
        ctypes.c_void_p(q_ptr) if q_ptr else None, ctypes.c_void_p(stream) if stream else None))


def powersgd_copy_error(state, bucket_index: int, view: int, e_ptr: int,
                        stream: Optional[int]) -> None:
    _check(load_library().powersgd_copy_error(
        state, bucket_index, view, ctypes.c_void_p(e_ptr),
        ctypes.c_void_p(stream) if stream else None))


def powersgd_get_factors(state, bucket_index: int, view: int) -> Tuple[int, int, int, int, int]:
    """(P pointer, Q pointer, n, m, r): state-owned device copies of the view's factors,
    enqueued on the stream of the bucket's latest call."""
    p, q = ctypes.c_void_p(), ctypes.c_void_p()
    n, m, r = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    _check(load_library().powersgd_get_factors(state, bucket_index, view, ctypes.byref(p),
                                               ctypes.byref(q), ctypes.byref(n),
                                               ctypes.byref(m), ctypes.byref(r)))
    return p.value or 0, q.value or 0, n.value, m.value, r.value


def powersgd_get_error(state, bucket_index: int) -> int:
    """Device pointer to the state-owned, bucket-shaped fp32 error memory."""
    e = ctypes.c_void_p()
    _check(load_library().powersgd_get_error(state, bucket_index, ctypes.byref(e)))
    return e.value or 0


def powersgd_draw_q0(random_seed: int, bucket_index: int, view: int, epoch: int, m: int,
                     rank: int, out_ptr: int, words_ptr: Optional[int],
                     stream: Optional[int]) -> None:
    _check(load_library().powersgd_draw_q0(
        int(random_seed) & 0xFFFFFFFFFFFFFFFF, int(bucket_index), int(view),
        int(epoch) & 0xFFFFFFFFFFFFFFFF, int(m), int(rank), ctypes.c_void_p(out_ptr),
        ctypes.c_void_p(words_ptr) if words_ptr else None,
        ctypes.c_void_p(stream) if stream else None))


def powersgd_compress_matrix_noalloc(hp: powersgd_hparams, bucket_index: int, view: int,
                                     epoch: int, m_ptr: int, n: int, m: int,
                                     e_ptr: Optional[int], q_ptr: int, q_valid: bool,
                                     p_ptr: Optional[int], stream: Optional[int]) -> None:
    _check(load_library().powersgd_compress_matrix_noalloc(
        ctypes.byref(hp), int(bucket_index), int(view), int(epoch) & 0xFFFFFFFFFFFFFFFF,
        ctypes.c_void_p(m_ptr), int(n), int(m), ctypes.c_void_p(e_ptr) if e_ptr else None,
        ctypes.c_void_p(q_ptr), int(bool(q_valid)), ctypes.c_void_p(p_ptr) if p_ptr else None,
        ctypes.c_void_p(stream) if stream else None))


def powersgd_get_stats(state) -> Tuple[int, int, int]:
    it, a, b = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().powersgd_get_stats(state, ctypes.byref(it), ctypes.byref(a),
                                             ctypes.byref(b)))
    return it.value, a.value, b.value


def powersgd_state_export(state, stream: Optional[int]) -> bytearray:
    lib = load_library()
    size = ctypes.c_int64()
    _check(lib.powersgd_state_export(state, None, 0, ctypes.byref(size), None))
    out = bytearray(size.value)
    view = (ctypes.c_char * max(size.value, 1)).from_buffer(out if size.value else bytearray(1))
    _check(lib.powersgd_state_export(state, view, size.value, ctypes.byref(size),
                                     ctypes.c_void_p(stream) if stream else None))
    return out


def powersgd_state_import(state, snapshot, stream: Optional[int]) -> None:
    if isinstance(snapshot, bytes):
        data, n = snapshot, len(snapshot)
    else:
        buf = bytearray(snapshot) if not isinstance(snapshot, bytearray) else snapshot
        n = len(buf)
        data = (ctypes.c_char * max(n, 1)).from_buffer(buf if n else bytearray(1))
    _check(load_library().powersgd_state_import(state, data, n,
                                                ctypes.c_void_p(stream) if stream else None))


def powersgd_set_timing(state, enable: bool) -> None:
    _check(load_library().powersgd_set_timing(state, int(bool(enable))))


def powersgd_get_kernel_times(state):
    ms = (ctypes.c_double * POWERSGD_NUM_KERNELS)()
    cnt = (ctypes.c_int64 * POWERSGD_NUM_KERNELS)()
    by = (ctypes.c_double * POWERSGD_NUM_KERNELS)()
    _check(load_library().powersgd_get_kernel_times(state, ms, cnt, by))
    return [(powersgd_kernel_name(k), ms[k], cnt[k], by[k]) for k in range(POWERSGD_NUM_KERNELS)]


def powersgd_classify_view(hp: powersgd_hparams, shape: Sequence[int]):
    """(compress, n, m, rank) for a view of this shape under hp (host only)."""
    view = make_views([(0, shape)])
    c, r = ctypes.c_int32(), ctypes.c_int32()
    n, m = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().powersgd_classify_view(ctypes.byref(hp), view, ctypes.byref(c),
                                                 ctypes.byref(n), ctypes.byref(m),
                                                 ctypes.byref(r)))
    return bool(c.value), n.value, m.value, r.value


def powersgd_kernel_name(kind: int) -> str:
    return load_library().powersgd_kernel_name(kind).decode()


# ----------------------------------------------------------- convenience wrapper

_HP_NAMES = [f[0] for f in powersgd_hparams._fields_]


class PowerSGDState:
    """Owns one library state; buckets are torch tensors on the state's device."""

    def __init__(self, device: int = 0, **hparams):
        hp = powersgd_hparams_init()
        for k, v in hparams.items():
            if k not in _HP_NAMES:
                raise TypeError(f"unknown hyperparameter {k!r}")
            setattr(hp, k, type(getattr(hp, k))(v) if not isinstance(v, bool) else int(v))
        self.hparams = hp
        self.device = device
        self._state = powersgd_state_create(hp, device)

    def close(self) -> None:
        if self._state:
            powersgd_state_destroy(self._state)
            self._state = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @staticmethod
    def _stream_handle(stream) -> Optional[int]:
        import torch
        if stream is None:
            stream = torch.cuda.current_stream()
        return int(stream.cuda_stream)

    @staticmethod
    def _bucket_args(bucket, found_inf):
        import torch
        if not bucket.is_cuda or not bucket.is_contiguous() or bucket.dim() != 1:
            raise ValueError("bucket must be a contiguous 1-D device tensor")
        if bucket.dtype == torch.float32:
            dtype = POWERSGD_F32
        elif bucket.dtype == torch.float16:
            dtype = POWERSGD_F16
        else:
            raise TypeError("bucket must be float32 or float16")
        fi = None
        if found_inf is not None:
            if found_inf.dtype != torch.int32 or not found_inf.is_cuda:
                raise TypeError("found_inf must be a device int32 tensor")
            fi = found_inf.data_ptr()
        return dtype, fi

    def compress_bucket(self, bucket, views: Sequence[Tuple[int, Sequence[int]]],
                        bucket_index: int = 0, is_last: bool = True,
                        inv_loss_scale: float = 1.0, found_inf=None, stream=None) -> None:
        dtype, fi = self._bucket_args(bucket, found_inf)
        powersgd_compress_bucket(self._state, bucket_index, is_last, bucket.data_ptr(), dtype,
                                 bucket.numel(), _views_arg(views), inv_loss_scale, fi,
                                 self._stream_handle(stream))

    def compress_bucket_wrapped(self, bucket, views: Sequence[Tuple[int, Sequence[int]]],
                                compute_dtype: str = "f16", bucket_index: int = 0,
                                is_last: bool = True, stream=None) -> None:
        """powerSGD_hook under fp16_compress_wrapper ("f16") or bf16_compress_wrapper
        ("bf16") on a float32 bucket, in place."""
        import torch
        if not bucket.is_cuda or not bucket.is_contiguous() or bucket.dim() != 1:
            raise ValueError("bucket must be a contiguous 1-D device tensor")
        if bucket.dtype != torch.float32:
            raise TypeError("the wrapped hook takes a float32 bucket")
        dt = {"f16": POWERSGD_F16, "bf16": POWERSGD_BF16}[compute_dtype]
        powersgd_compress_bucket_wrapped(self._state, bucket_index, is_last, bucket.data_ptr(),
                                         dt, bucket.numel(), _views_arg(views),
                                         self._stream_handle(stream))

    def compress_bucket_batched_wrapped(self, buffer, compute_dtype: str = "f16",
                                        numel: Optional[int] = None, bucket_index: int = 0,
                                        is_last: bool = True, stream=None) -> None:
        """batched_powerSGD_hook under fp16_compress_wrapper ("f16") or
        bf16_compress_wrapper ("bf16") on the first `numel` elements of a float32
        `buffer` holding at least powersgd_batched_side(numel) ** 2 elements."""
        import torch
        if not buffer.is_cuda or not buffer.is_contiguous() or buffer.dim() != 1:
            raise ValueError("buffer must be a contiguous 1-D device tensor")
        if buffer.dtype != torch.float32:
            raise TypeError("the wrapped hook takes a float32 buffer")
        dt = {"f16": POWERSGD_F16, "bf16": POWERSGD_BF16}[compute_dtype]
        n = buffer.numel() if numel is None else int(numel)
        powersgd_compress_bucket_batched_wrapped(self._state, bucket_index, is_last,
                                                 buffer.data_ptr(), dt, n, buffer.numel(),
                                                 self._stream_handle(stream))

    def compress_bucket_batched(self, buffer, numel: Optional[int] = None,
                                bucket_index: int = 0, is_last: bool = True,
                                inv_loss_scale: float = 1.0, found_inf=None,
                                stream=None) -> None:
        """batched_powerSGD_hook on the first `numel` elements of `buffer` (default: all
        of it), which must hold at least powersgd_batched_side(numel) ** 2 elements:
        the buffer is the zero-padded square matrix, and its first numel elements are
        the result."""
        dtype, fi = self._bucket_args(buffer, found_inf)
        n = buffer.numel() if numel is None else int(numel)
        powersgd_compress_bucket_batched(self._state, bucket_index, is_last, buffer.data_ptr(),
                                         dtype, n, buffer.numel(), inv_loss_scale, fi,
                                         self._stream_handle(stream))

    def decisions(self, bucket_index: int, nviews: int) -> List[int]:
        return powersgd_get_decisions(self._state, bucket_index, nviews)

    def view_info(self, bucket_index: int, view: int) -> Tuple[int, int, int]:
        return powersgd_get_view_info(self._state, bucket_index, view)

    def factors(self, bucket_index: int, view: int, stream=None):
        import torch
        n, m, r = self.view_info(bucket_index, view)
        dev = torch.device("cuda", self.device)
        p = torch.empty((n, r), dtype=torch.float32, device=dev)
        q = torch.empty((m, r), dtype=torch.float32, device=dev)
        powersgd_copy_factors(self._state, bucket_index, view, p.data_ptr(), q.data_ptr(),
                              self._stream_handle(stream))
        return p, q

    def error(self, bucket_index: int, view: int, stream=None):
        import torch
        n, m, _ = self.view_info(bucket_index, view)
        e = torch.empty((n, m), dtype=torch.float32, device=torch.device("cuda", self.device))
        powersgd_copy_error(self._state, bucket_index, view, e.data_ptr(),
                            self._stream_handle(stream))
        return e

    def stats(self) -> Tuple[int, int, int]:
        return powersgd_get_stats(self._state)

    def export_state(self, stream=None) -> bytearray:
        """The state's snapshot (format in include/powersgd.h), after the work already
        enqueued on `stream`."""
        return powersgd_state_export(self._state, self._stream_handle(stream))

    def import_state(self, snapshot, stream=None) -> None:
        """Replaces the state with a snapshot taken under the same hyperparameters."""
        powersgd_state_import(self._state, snapshot, self._stream_handle(stream))

    def set_timing(self, enable: bool) -> None:
        powersgd_set_timing(self._state, enable)

    def kernel_times(self):
        return powersgd_get_kernel_times(self._state)
