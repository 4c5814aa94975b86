"""ctypes binding of libeffort (include/effort.h): same names, argument marshalling only.

Arguments that are device buffers accept a torch tensor (its data_ptr is
passed) or a raw integer address; host buffers accept numpy arrays.  `stream`
defaults to torch's current stream when torch has a GPU, else the null stream.
Every non-zero status raises EffortError.  There is no fallback: if the
library is missing, importing this module fails.
"""
from __future__ import annotations

import ctypes
import os
import re

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libeffort.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "effort.h")

EFFORT_OK, EFFORT_EINVAL, EFFORT_ENOSPACE, EFFORT_EHIP, EFFORT_EUNSUPPORTED, EFFORT_ECORRUPT = range(6)
EFFORT_MAX_BATCH = 16
EFFORT_MAX_GROUP_WIDTH = 8192


class EffortError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        msg = "%s: %s (status %d)" % (where, effort_strerror(code), code)
        if code == EFFORT_EHIP:
            msg += ": " + effort_last_hip_error()
        super().__init__(msg)


EFFORT_ENTRY_U32, EFFORT_ENTRY_R12, EFFORT_ENTRY_Q8 = 0, 1, 2


class effort_prepare_opts(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int32), ("entry_format", ctypes.c_int32),
                ("crop_segments", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class effort_desc(ctypes.Structure):
    _fields_ = [
        ("magic", ctypes.c_uint32), ("version", ctypes.c_uint32),
        ("in_dim", ctypes.c_int64), ("out_dim", ctypes.c_int64),
        ("probes_per_row", ctypes.c_int32), ("groups", ctypes.c_int32),
        ("group_width", ctypes.c_int32), ("index_bytes", ctypes.c_int32),
        ("row_stride", ctypes.c_int64), ("group_stride", ctypes.c_int64),
        ("entry_format", ctypes.c_int32), ("crop_segments", ctypes.c_int32),
        ("off_probes", ctypes.c_uint64), ("off_counts", ctypes.c_uint64),
        ("off_entries", ctypes.c_uint64), ("off_rowmax", ctypes.c_uint64),
        ("off_floor", ctypes.c_uint64), ("total_bytes", ctypes.c_uint64),
        ("checksum", ctypes.c_uint64), ("desc_check", ctypes.c_uint64),
    ]

    def copy(self) -> "effort_desc":
        d = effort_desc()
        ctypes.memmove(ctypes.byref(d), ctypes.byref(self), ctypes.sizeof(self))
        return d


if not os.path.exists(LIB_PATH):
    raise ImportError("libeffort.so is not built (python dynamic_sparsity_approximate_amd/build.py)")
# One HIP runtime per process: torch ships its own libamdhip64 (soname
# libamdhip64.so.7, loaded by the file name libamdhip64.so).  Loading torch first
# lets libeffort's dependency on libamdhip64.so.7 resolve to that same copy;
# loading libeffort first would bring in a second runtime that sees no device.
try:
    import torch  # noqa: F401
except ImportError:  # C-only use: the system runtime is the only one
    pass
_lib = ctypes.CDLL(LIB_PATH)

_p, _i32, _i64, _u64, _f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint64, ctypes.c_float
_D = ctypes.POINTER(effort_desc)
_PROTOS = {
    "effort_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "effort_last_hip_error": ([], ctypes.c_char_p),
    "effort_default_groups": ([_i64], _i32),
    "effort_layout_bytes": ([_i64, _i64, _i32, ctypes.POINTER(_u64)], ctypes.c_int),
    "effort_layout_bytes_ex": ([_i64, _i64, _i32, _i32, ctypes.POINTER(_u64)], ctypes.c_int),
    "effort_workspace_bytes": ([_D, _i32, ctypes.POINTER(_u64)], ctypes.c_int),
    "effort_workspace_init": ([_p, _u64, _p], ctypes.c_int),
    "effort_prepare_host": ([_p, _i64, _i64, _i32, _p, _u64, _D], ctypes.c_int),
    "effort_prepare_host_ex": ([_p, _i64, _i64, _i32, _i32, _p, _u64, _D], ctypes.c_int),
    "effort_prepare": ([_p, _i64, _i64, _i32, _p, _u64, _D, _p], ctypes.c_int),
    "effort_layout_bytes_opts": ([_p, _i64, _i64, _i32, _p, ctypes.POINTER(_u64)], ctypes.c_int),
    "effort_prepare_host_opts": ([_p, _i64, _i64, _i32, _p, _p, _u64, _D], ctypes.c_int),
    "effort_layout_check": ([_D, _p], ctypes.c_int),
    "effort_matvec": ([_D, _p, _p, _f32, _p, _p, _u64, _p], ctypes.c_int),
    "effort_matvec_batched": ([_D, _p, _p, _i32, _f32, _p, _p, _u64, _p], ctypes.c_int),
    "effort_matvec_noalloc": ([_D, _p, _p, _f32, _p, _p], ctypes.c_int),
    "effort_workspace_bytes_multi": ([_D, _i32, ctypes.POINTER(_u64)], ctypes.c_int),
    "effort_matvec_multi": ([_D, ctypes.POINTER(_p), _i32, ctypes.POINTER(_p),
                             ctypes.POINTER(_f32), ctypes.POINTER(_p), _p, _u64, _p], ctypes.c_int),
    "effort_matvec_debug": ([_D, _p, _p, _f32, _p, _p, _u64, _p, _p, _p, _p, _p, _p, _p], ctypes.c_int),
    "effort_matvec_batched_debug": ([_D, _p, _p, _i32, _f32, _p, _p, _u64, _p, _p, _p, _p, _p, _p],
                                    ctypes.c_int),
    "effort_matvec_multi_debug": ([_D, ctypes.POINTER(_p), _i32, ctypes.POINTER(_p),
                                   ctypes.POINTER(_f32), ctypes.POINTER(_p), _p, _u64, _p, _p,
                                   ctypes.POINTER(_p), _p, _p], ctypes.c_int),
    "effort_matvec_timed": ([_D, _p, _p, _f32, _p, _p, _u64, _p, _p], ctypes.c_int),
    "dense_gemv": ([_p, _p, _i64, _i64, _p, _p], ctypes.c_int),
    "dense_gemm_small": ([_p, _p, _i32, _i64, _i64, _p, _p], ctypes.c_int),
    "effort_silu_mul": ([_p, _p, _i64, _p, _p], ctypes.c_int),
    "effort_axpby": ([_p, _f32, _p, _f32, _i64, _p, _p], ctypes.c_int),
    "effort_event_create": ([ctypes.POINTER(_p)], ctypes.c_int),
    "effort_event_record": ([_p, _p], ctypes.c_int),
    "effort_event_elapsed_ms": ([_p, _p, ctypes.POINTER(_f32)], ctypes.c_int),
    "effort_event_destroy": ([_p], ctypes.c_int),
    "effort_stream_synchronize": ([_p], ctypes.c_int),
}
for _name, (_args, _res) in _PROTOS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = _res


def lib():
    return _lib


def header_functions() -> list:
    """Names of the functions include/effort.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w]*\s*\**\s*([A-Za-z_]\w*)\s*\(", text, flags=re.M)


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError("cannot pass %r as a pointer" % type(x))


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    try:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
    except Exception:  # pragma: no cover - torch absent
        pass
    return None


def _check(rc: int, where: str):
    if rc != EFFORT_OK:
        raise EffortError(rc, where)


def _check_ws(rc: int, where: str, ws, ws_bytes: int, stream):
    """As _check; after EFFORT_EHIP the workspace is zero-filled again (a call
    that failed part-way may leave set the words every call expects to find
    zero) before the error is raised."""
    if rc == EFFORT_EHIP and ws is not None:
        _lib.effort_workspace_init(_ptr(ws), ws_bytes, _stream(stream))
    _check(rc, where)


def effort_strerror(status: int) -> str:
    return _lib.effort_strerror(status).decode()


def effort_last_hip_error() -> str:
    return _lib.effort_last_hip_error().decode()


def effort_default_groups(out_dim: int) -> int:
    return int(_lib.effort_default_groups(out_dim))


def effort_layout_bytes(in_dim: int, out_dim: int, P: int) -> int:
    b = _u64()
    _check(_lib.effort_layout_bytes(in_dim, out_dim, P, ctypes.byref(b)), "effort_layout_bytes")
    return int(b.value)


def effort_layout_bytes_ex(in_dim: int, out_dim: int, P: int, groups: int) -> int:
    b = _u64()
    _check(_lib.effort_layout_bytes_ex(in_dim, out_dim, P, groups, ctypes.byref(b)),
           "effort_layout_bytes_ex")
    return int(b.value)


def effort_workspace_bytes(desc: effort_desc, batch: int = 1) -> int:
    b = _u64()
    _check(_lib.effort_workspace_bytes(ctypes.byref(desc), batch, ctypes.byref(b)),
           "effort_workspace_bytes")
    return int(b.value)


def effort_workspace_init(ws, ws_bytes: int, stream=None):
    _check(_lib.effort_workspace_init(_ptr(ws), ws_bytes, _stream(stream)), "effort_workspace_init")


def _host_w(w_fp16):
    w = np.ascontiguousarray(w_fp16)
    if w.dtype == np.float16:
        w = w.view(np.uint16)
    if w.dtype != np.uint16 or w.ndim != 2:
        raise TypeError("w_fp16 must be a 2-D uint16/float16 array")
    return w


def effort_layout_bytes_opts(w_fp16, P: int, groups: int = 0, entry_format: int = EFFORT_ENTRY_U32,
                             crop: int = 0) -> int:
    w = _host_w(w_fp16)
    m, n = w.shape
    o = effort_prepare_opts(groups, entry_format, crop, 0)
    b = _u64()
    _check(_lib.effort_layout_bytes_opts(w.ctypes.data, m, n, P, ctypes.byref(o), ctypes.byref(b)),
           "effort_layout_bytes_opts")
    return int(b.value)


def effort_prepare_host(w_fp16, P: int, groups: int = 0, entry_format: int = EFFORT_ENTRY_U32,
                        crop: int = 0):
    """Host fp16 bits [in][out] -> (desc, layout blob as a uint8 numpy array).
    `entry_format` and `crop` (stored segments, 0 = all) select the layout
    options of effort_prepare_host_opts."""
    w = _host_w(w_fp16)
    m, n = w.shape
    desc = effort_desc()
    if entry_format == EFFORT_ENTRY_U32 and crop in (0, P):
        nbytes = effort_layout_bytes_ex(m, n, P, groups)
        blob = np.empty(nbytes // 8, dtype=np.uint64).view(np.uint8)  # 8-byte aligned
        _check(_lib.effort_prepare_host_ex(w.ctypes.data, m, n, P, groups, blob.ctypes.data, nbytes,
                                           ctypes.byref(desc)), "effort_prepare_host")
        return desc, blob
    o = effort_prepare_opts(groups, entry_format, crop, 0)
    nbytes = effort_layout_bytes_opts(w, P, groups, entry_format, crop)
    blob = np.empty(nbytes // 8, dtype=np.uint64).view(np.uint8)
    _check(_lib.effort_prepare_host_opts(w.ctypes.data, m, n, P, ctypes.byref(o), blob.ctypes.data,
                                         nbytes, ctypes.byref(desc)), "effort_prepare_host_opts")
    return desc, blob


def effort_prepare(w_fp16, P: int, layout_dev, layout_bytes: int, stream=None) -> effort_desc:
    w = np.ascontiguousarray(w_fp16)
    if w.dtype == np.float16:
        w = w.view(np.uint16)
    m, n = w.shape
    desc = effort_desc()
    _check(_lib.effort_prepare(w.ctypes.data, m, n, P, _ptr(layout_dev), layout_bytes,
                               ctypes.byref(desc), _stream(stream)), "effort_prepare")
    return desc


def effort_layout_check(desc: effort_desc, blob) -> None:
    _check(_lib.effort_layout_check(ctypes.byref(desc), _ptr(blob)), "effort_layout_check")


def effort_matvec(desc, layout, v, effort: float, y, ws, ws_bytes: int, stream=None):
    _check_ws(_lib.effort_matvec(ctypes.byref(desc), _ptr(layout), _ptr(v), effort, _ptr(y),
                                 _ptr(ws), ws_bytes, _stream(stream)), "effort_matvec", ws, ws_bytes,
              stream)


EFFORT_NOALLOC_WORKSPACE_BYTES = 8 << 20


def effort_matvec_noalloc(desc, layout, v, effort: float, y, stream=None):
    _check(_lib.effort_matvec_noalloc(ctypes.byref(desc), _ptr(layout), _ptr(v), effort, _ptr(y),
                                      _stream(stream)), "effort_matvec_noalloc")


def effort_matvec_batched(desc, layout, v, batch: int, effort: float, y, ws, ws_bytes: int,
                          stream=None):
    _check_ws(_lib.effort_matvec_batched(ctypes.byref(desc), _ptr(layout), _ptr(v), batch, effort,
                                         _ptr(y), _ptr(ws), ws_bytes, _stream(stream)),
              "effort_matvec_batched", ws, ws_bytes, stream)


def effort_matvec_batched_debug(desc, layout, v, batch: int, effort: float, y, ws, ws_bytes: int,
                                cutoff=None, K=None, row_kept=None, fingerprint=None,
                                kept_mask=None, stream=None):
    _check_ws(_lib.effort_matvec_batched_debug(ctypes.byref(desc), _ptr(layout), _ptr(v), batch,
                                               effort, _ptr(y), _ptr(ws), ws_bytes, _ptr(cutoff),
                                               _ptr(K), _ptr(row_kept), _ptr(fingerprint),
                                               _ptr(kept_mask), _stream(stream)),
              "effort_matvec_batched_debug", ws, ws_bytes, stream)


def _desc_array(descs):
    arr = (effort_desc * len(descs))()
    for j, d in enumerate(descs):
        arr[j] = d
    return arr


def effort_workspace_bytes_multi(descs) -> int:
    b = _u64()
    _check(_lib.effort_workspace_bytes_multi(_desc_array(descs), len(descs), ctypes.byref(b)),
           "effort_workspace_bytes_multi")
    return int(b.value)


def effort_matvec_multi(descs, layouts, vs, efforts, ys, ws, ws_bytes: int, stream=None):
    """ys[j] = approximate vs[j] . W_j at efforts[j].  `vs` may be one vector
    (shared by all matrices) and `efforts` one float (for all)."""
    n = len(descs)
    if not isinstance(vs, (list, tuple)):
        vs = [vs] * n
    if isinstance(efforts, (int, float)):
        efforts = [float(efforts)] * n
    if not (len(layouts) == len(vs) == len(ys) == len(efforts) == n):
        raise ValueError("descs, layouts, vs, efforts and ys must have one entry per matrix")
    _check_ws(_lib.effort_matvec_multi(_desc_array(descs), (_p * n)(*[_ptr(x) for x in layouts]),
                                       n, (_p * n)(*[_ptr(v) for v in vs]), (_f32 * n)(*efforts),
                                       (_p * n)(*[_ptr(y) for y in ys]), _ptr(ws), ws_bytes,
                                       _stream(stream)), "effort_matvec_multi", ws, ws_bytes, stream)


def effort_matvec_multi_debug(descs, layouts, vs, efforts, ys, ws, ws_bytes: int, cutoff=None,
                              K=None, row_kept=None, fingerprint=None, stream=None):
    """effort_matvec_multi with parity outputs: cutoff [count], K [count][2],
    fingerprint [count] (device buffers), row_kept a list of count device
    buffers (or None)."""
    n = len(descs)
    if not isinstance(vs, (list, tuple)):
        vs = [vs] * n
    if isinstance(efforts, (int, float)):
        efforts = [float(efforts)] * n
    if not (len(layouts) == len(vs) == len(ys) == len(efforts) == n):
        raise ValueError("descs, layouts, vs, efforts and ys must have one entry per matrix")
    rk = None if row_kept is None else (_p * n)(*[_ptr(r) for r in row_kept])
    _check_ws(_lib.effort_matvec_multi_debug(_desc_array(descs),
                                             (_p * n)(*[_ptr(x) for x in layouts]), n,
                                             (_p * n)(*[_ptr(v) for v in vs]), (_f32 * n)(*efforts),
                                             (_p * n)(*[_ptr(y) for y in ys]), _ptr(ws), ws_bytes,
                                             _ptr(cutoff), _ptr(K), rk, _ptr(fingerprint),
                                             _stream(stream)),
              "effort_matvec_multi_debug", ws, ws_bytes, stream)


def effort_matvec_debug(desc, layout, v, effort: float, y, ws, ws_bytes: int, cutoff=None, K=None,
                        row_kept=None, fingerprint=None, kept_mask=None, status=None, stream=None):
    _check_ws(_lib.effort_matvec_debug(ctypes.byref(desc), _ptr(layout), _ptr(v), effort, _ptr(y),
                                       _ptr(ws), ws_bytes, _ptr(cutoff), _ptr(K), _ptr(row_kept),
                                       _ptr(fingerprint), _ptr(kept_mask), _ptr(status),
                                       _stream(stream)),
              "effort_matvec_debug", ws, ws_bytes, stream)


def effort_matvec_timed(desc, layout, v, effort: float, y, ws, ws_bytes: int, events, stream=None):
    if len(events) != 6:
        raise ValueError("events: six handles, (start, stop) for select, dispatch, bucketMul")
    arr = (_p * 6)(*[e if e else None for e in events])
    _check_ws(_lib.effort_matvec_timed(ctypes.byref(desc), _ptr(layout), _ptr(v), effort, _ptr(y),
                                       _ptr(ws), ws_bytes, _stream(stream), arr),
              "effort_matvec_timed", ws, ws_bytes, stream)


def dense_gemv(w, v, in_dim: int, out_dim: int, y, stream=None):
    _check(_lib.dense_gemv(_ptr(w), _ptr(v), in_dim, out_dim, _ptr(y), _stream(stream)), "dense_gemv")


def dense_gemm_small(w, v, batch: int, in_dim: int, out_dim: int, y, stream=None):
    _check(_lib.dense_gemm_small(_ptr(w), _ptr(v), batch, in_dim, out_dim, _ptr(y), _stream(stream)),
           "dense_gemm_small")


def effort_silu_mul(h1, h3, n: int, out, stream=None):
    _check(_lib.effort_silu_mul(_ptr(h1), _ptr(h3), n, _ptr(out), _stream(stream)), "effort_silu_mul")


def effort_axpby(a, ga: float, b, gb: float, n: int, out, stream=None):
    _check(_lib.effort_axpby(_ptr(a), ga, _ptr(b), gb, n, _ptr(out), _stream(stream)), "effort_axpby")


def effort_event_create() -> int:
    e = _p()
    _check(_lib.effort_event_create(ctypes.byref(e)), "effort_event_create")
    return int(e.value)


def effort_event_record(event: int, stream=None):
    _check(_lib.effort_event_record(event, _stream(stream)), "effort_event_record")


def effort_event_elapsed_ms(start: int, end: int) -> float:
    ms = _f32()
    _check(_lib.effort_event_elapsed_ms(start, end, ctypes.byref(ms)), "effort_event_elapsed_ms")
    return float(ms.value)


def effort_event_destroy(event: int):
    _check(_lib.effort_event_destroy(event), "effort_event_destroy")


def effort_stream_synchronize(stream=None):
    _check(_lib.effort_stream_synchronize(_stream(stream)), "effort_stream_synchronize")
