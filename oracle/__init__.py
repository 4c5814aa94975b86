"""Oracle of the "Effort" approximate vector-matrix multiply -- TEST INFRASTRUCTURE.

Only tests/, ``__graft_entry__.smoke()`` and the CPU-baseline leg of bench.py
may import this package.  It wraps ``oracle.c`` (plain single-threaded C, built
with gcc, -O2 -ffp-contract=off, no fast-math) through ctypes and shares no
code with the GPU library.

Parity status of each function (pins live in tests/test_oracle_pins.py):
  f16_to_f64   pinned: all 65536 patterns against numpy's float16
  pair_hash    pinned: splitmix64 reference output of the generator module
  probes       pinned: order statistics from numpy sort; P = n gives all magnitudes
  chart        pinned: exact fp32 products (double product rounded once)
  cutoff       pinned: full numpy sort; rank identities
  keep_sum     pinned: effort = 1 equals the dense product; brute-force top-K
               products with P = n; nesting, scaling, sign and permutation
               invariants; dropped-mass bound
  run          composition of the above
  dense        pinned: numpy float64 matmul
  stored_mask  pinned: numpy lexsort of (|w| desc, column asc) per row; crop = P stores all
  run_cropped  pinned: crop = P equals run(); effort 1 keeps exactly the stored pairs; a
               call whose kept set lies in the stored part equals run(); numpy sums
  quantize_q8  pinned: levels by brute force from the definition (numpy), nearest level per
               weight, probes unchanged, lo maps to itself, signs kept, error bound
  silu_mul     pinned: silu(x) - silu(-x) = x, silu(0) = 0, silu(ln 3) = (3/4) ln 3,
               silu(x) -> x for large x, linear in the second operand
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_pair_hash.argtypes = [ctypes.c_uint64]
    lib.oracle_pair_hash.restype = ctypes.c_uint64
    lib.oracle_probes.argtypes = [p, i64, i64, i32, p]
    lib.oracle_chart.argtypes = [p, p, i64, i32, p]
    lib.oracle_cutoff.argtypes = [p, i64, f32, p, p, p]
    lib.oracle_keep_sum.argtypes = [p, i64, i64, p, f32, p, p, p, p, p]
    lib.oracle_run.argtypes = [p, i64, i64, p, i32, p, f32, p, p, p, p, p, p, p, p, p]
    lib.oracle_dense.argtypes = [p, i64, i64, p, p]
    lib.oracle_stored_mask.argtypes = [p, i64, i64, i32, i32, p]
    lib.oracle_quantize_q8.argtypes = [p, i64, i64, i32, p]
    lib.oracle_quantize_q8.restype = ctypes.c_int
    lib.oracle_run_cropped.argtypes = [p, i64, i64, p, i32, i32, p, f32, p, p, p, p, p, p, p, p, p]
    for f in (lib.oracle_probes, lib.oracle_chart, lib.oracle_cutoff, lib.oracle_keep_sum,
              lib.oracle_run, lib.oracle_dense, lib.oracle_stored_mask, lib.oracle_run_cropped):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _w(W):
    W = np.ascontiguousarray(W)
    if W.dtype == np.float16:
        W = W.view(np.uint16)
    assert W.dtype == np.uint16 and W.ndim == 2
    return W


def f16_to_f64(bits: int) -> float:
    return float(_load().oracle_f16_to_f64(int(bits) & 0xFFFF))


def pair_hash(x: int) -> int:
    return int(_load().oracle_pair_hash(int(x) & 0xFFFFFFFFFFFFFFFF))


def probes(W, P: int) -> np.ndarray:
    W = _w(W)
    m, n = W.shape
    out = np.empty((m, P), dtype=np.float32)
    rc = _load().oracle_probes(_ptr(W), m, n, P, _ptr(out))
    if rc:
        raise ValueError("oracle_probes: invalid argument")
    return out


def chart(v, pr) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float32)
    pr = np.ascontiguousarray(pr, dtype=np.float32)
    m, P = pr.shape
    out = np.empty((m, P), dtype=np.float32)
    rc = _load().oracle_chart(_ptr(v), _ptr(pr), m, P, _ptr(out))
    if rc:
        raise ValueError("oracle_chart: invalid argument")
    return out


def cutoff(ch, effort: float):
    ch = np.ascontiguousarray(ch, dtype=np.float32).ravel()
    K = ctypes.c_int64()
    Kp = ctypes.c_int64()
    c = ctypes.c_float()
    rc = _load().oracle_cutoff(_ptr(ch), ch.size, effort, ctypes.byref(K), ctypes.byref(c),
                               ctypes.byref(Kp))
    if rc:
        raise ValueError("oracle_cutoff: invalid argument")
    return int(K.value), np.float32(c.value), int(Kp.value)


def keep_sum(W, v, cut, mask: bool = False) -> dict:
    W = _w(W)
    m, n = W.shape
    v = np.ascontiguousarray(v, dtype=np.float32)
    y = np.empty(n, dtype=np.float64)
    rk = np.empty(m, dtype=np.int64)
    fp = ctypes.c_uint64()
    tot = ctypes.c_int64()
    mk = np.empty((m, n), dtype=np.uint8) if mask else None
    rc = _load().oracle_keep_sum(_ptr(W), m, n, _ptr(v), np.float32(cut), _ptr(y), _ptr(rk),
                                 ctypes.byref(fp), _ptr(mk), ctypes.byref(tot))
    if rc:
        raise ValueError("oracle_keep_sum: invalid argument")
    return {"y": y, "row_kept": rk, "fingerprint": int(fp.value), "mask": mk,
            "total_kept": int(tot.value)}


def run(W, pr, v, effort: float, mask: bool = False) -> dict:
    """Whole rule for one vector.  ``pr`` = probes(W, P)."""
    W = _w(W)
    m, n = W.shape
    pr = np.ascontiguousarray(pr, dtype=np.float32)
    P = pr.shape[1]
    v = np.ascontiguousarray(v, dtype=np.float32)
    y = np.empty(n, dtype=np.float64)
    rk = np.empty(m, dtype=np.int64)
    rck = np.empty(m, dtype=np.int64)
    fp = ctypes.c_uint64()
    tot = ctypes.c_int64()
    K = ctypes.c_int64()
    Kp = ctypes.c_int64()
    c = ctypes.c_float()
    mk = np.empty((m, n), dtype=np.uint8) if mask else None
    rc = _load().oracle_run(_ptr(W), m, n, _ptr(pr), P, _ptr(v), effort, ctypes.byref(c),
                            ctypes.byref(K), ctypes.byref(Kp), _ptr(y), _ptr(rk), _ptr(rck),
                            ctypes.byref(fp), _ptr(mk), ctypes.byref(tot))
    if rc:
        raise ValueError("oracle_run: invalid argument")
    return {"cutoff": np.float32(c.value), "K": int(K.value), "Kprime": int(Kp.value),
            "y": y, "row_kept": rk, "row_chart_kept": rck, "fingerprint": int(fp.value),
            "mask": mk, "total_kept": int(tot.value), "m": m, "n": n, "P": P}


def stored_mask(W, P: int, crop: int) -> np.ndarray:
    """uint8 [m][n]: the pairs a layout cropped to segments 0..crop-1 stores."""
    W = _w(W)
    m, n = W.shape
    out = np.empty((m, n), dtype=np.uint8)
    if _load().oracle_stored_mask(_ptr(W), m, n, P, crop, _ptr(out)):
        raise ValueError("oracle_stored_mask: invalid argument")
    return out


def run_cropped(W, pr, v, effort: float, crop: int, mask: bool = False) -> dict:
    """The rule on a layout cropped to segments 0..crop-1 of P = pr.shape[1]."""
    W = _w(W)
    m, n = W.shape
    pr = np.ascontiguousarray(pr, dtype=np.float32)
    P = pr.shape[1]
    v = np.ascontiguousarray(v, dtype=np.float32)
    y = np.empty(n, dtype=np.float64)
    rk = np.empty(m, dtype=np.int64)
    fp, tot, K, Kp = ctypes.c_uint64(), ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    c, reached = ctypes.c_float(), ctypes.c_int32()
    mk = np.empty((m, n), dtype=np.uint8) if mask else None
    rc = _load().oracle_run_cropped(_ptr(W), m, n, _ptr(pr), P, crop, _ptr(v), effort,
                                    ctypes.byref(c), ctypes.byref(K), ctypes.byref(Kp), _ptr(y),
                                    _ptr(rk), ctypes.byref(fp), _ptr(mk), ctypes.byref(tot),
                                    ctypes.byref(reached))
    if rc:
        raise ValueError("oracle_run_cropped: invalid argument")
    return {"cutoff": np.float32(c.value), "K": int(K.value), "Kprime": int(Kp.value), "y": y,
            "row_kept": rk, "fingerprint": int(fp.value), "mask": mk, "total_kept": int(tot.value),
            "crop_reached": bool(reached.value), "m": m, "n": n, "P": P}


def quantize_q8(W, P: int) -> np.ndarray:
    """fp16 bits of W in the Q8 bucketed form (each magnitude on its rank
    bucket's 16-level grid, sign kept); the rule runs on the result."""
    W = _w(W)
    m, n = W.shape
    out = np.empty((m, n), dtype=np.uint16)
    if _load().oracle_quantize_q8(_ptr(W), m, n, P, _ptr(out)):
        raise ValueError("oracle_quantize_q8: invalid argument")
    return out


def dense(W, v) -> np.ndarray:
    W = _w(W)
    m, n = W.shape
    v = np.ascontiguousarray(v, dtype=np.float32)
    y = np.empty(n, dtype=np.float64)
    rc = _load().oracle_dense(_ptr(W), m, n, _ptr(v), _ptr(y))
    if rc:
        raise ValueError("oracle_dense: invalid argument")
    return y


def silu_mul(h1, h3) -> np.ndarray:
    """Gated FFN glue in float64: silu(h1) * h3, silu(x) = x / (1 + exp(-x))."""
    h1 = np.asarray(h1, dtype=np.float64)
    h3 = np.asarray(h3, dtype=np.float64)
    return h1 / (1.0 + np.exp(-h1)) * h3
