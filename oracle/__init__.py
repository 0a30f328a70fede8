"""ctypes wrapper of the plain CPU reference (``tbe_oracle.c``).

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's CPU
baseline use this to check the GPU library.  The product package never
imports it.  All arithmetic is fp64; see ``tbe_oracle.c`` for what each
function computes and which page passage it follows.

``build_timed`` compiles the same source with fp32 accumulators for the
benchmark's CPU baseline only (``-O3 -march=native``, so it is built on the
host that runs it); every function below takes ``lib=`` to run on it.  The
fp64 build is the only one the tests compare against.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "tbe_oracle.c")
_LIB = os.path.join(_HERE, "libtbe_oracle.so")

F32, F16, BF16 = 0, 1, 2
POOL_SUM, POOL_MEAN = 0, 1
OPT_SGD, OPT_ROWWISE_ADAGRAD = 0, 1

_lib = None


def build() -> str:
    """Compile the oracle into ``oracle/libtbe_oracle.so`` (always rebuilds)."""
    tmp = _LIB + ".tmp"
    subprocess.check_call(
        ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra",
         "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, _LIB)
    return _LIB


def build_timed(path: str) -> str:
    """Compile the fp32-accumulator timing build of the oracle to ``path``, tuned for the
    CPU this runs on (CPU baseline only; never a parity reference)."""
    tmp = path + ".tmp"
    subprocess.check_call(
        ["gcc", "-O3", "-march=native", "-fopenmp", "-fPIC", "-shared", "-std=c11",
         "-DORACLE_ACC=float", "-o", tmp, _SRC, "-lm"])
    os.replace(tmp, path)
    return path


def load_timed(path: str):
    """The timing build at ``path`` (see build_timed), for the ``lib=`` argument."""
    return _bind(ctypes.CDLL(path))


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    _lib = _bind(ctypes.CDLL(_LIB))
    return _lib


def _bind(lib):
    P = ctypes.c_void_p
    i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
    lib.tbe_oracle_widen.argtypes = [i32, ctypes.c_uint32]
    lib.tbe_oracle_widen.restype = f64
    lib.tbe_oracle_narrow.argtypes = [i32, f64]
    lib.tbe_oracle_narrow.restype = ctypes.c_uint32
    lib.tbe_oracle_widen_array.argtypes = [i32, P, P, i64]
    lib.tbe_oracle_widen_array.restype = None
    lib.tbe_oracle_narrow_array.argtypes = [i32, P, P, i64]
    lib.tbe_oracle_narrow_array.restype = None
    lib.tbe_oracle_forward.argtypes = [i32, P, P, i32, i32, P, i64, P, P, i64, P, P]
    lib.tbe_oracle_forward.restype = ctypes.c_int
    lib.tbe_oracle_forward_bags.argtypes = [i32, P, P, i32, i32, P, i64, P, P, i64, P, i64, P, P]
    lib.tbe_oracle_forward_bags.restype = ctypes.c_int
    lib.tbe_oracle_runs.argtypes = [i32, P, i64, P, P, i64, P, P, P]
    lib.tbe_oracle_runs.restype = ctypes.c_int
    lib.tbe_oracle_dense_grad.argtypes = [i32, P, P, i32, i64, P, P, i64, P, P, P]
    lib.tbe_oracle_dense_grad.restype = ctypes.c_int
    lib.tbe_oracle_psw_grad.argtypes = [i32, P, P, i32, i32, P, i64, P, P, i64, P, P]
    lib.tbe_oracle_psw_grad.restype = ctypes.c_int
    lib.tbe_oracle_backward_update.argtypes = [i32, P, P, i32, i32, i32, P, P, i64, P, P, i64,
                                               P, P, f64, f64, i64, P]
    lib.tbe_oracle_backward_update.restype = ctypes.c_int
    lib.tbe_oracle_set_threads.argtypes = [i32]
    lib.tbe_oracle_set_threads.restype = None
    lib.tbe_oracle_get_threads.argtypes = []
    lib.tbe_oracle_get_threads.restype = i32
    return lib


def _ptr(a):
    if a is None:
        return None
    return ctypes.c_void_p(a.ctypes.data)


def _i64(a):
    return np.ascontiguousarray(a, dtype=np.int64)


def _i32(a):
    return np.ascontiguousarray(a, dtype=np.int32)


def _f32(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float32)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its input (code {rc})")


def _storage_view(dtype: int, weights: np.ndarray) -> np.ndarray:
    """The flat storage array as raw bits (uint32 for fp32, uint16 otherwise)."""
    w = np.ascontiguousarray(weights)
    want = np.uint32 if dtype == F32 else np.uint16
    if w.dtype.itemsize != np.dtype(want).itemsize:
        raise TypeError(f"weights itemsize {w.dtype.itemsize} does not match storage dtype {dtype}")
    return w.view(want).reshape(-1)


def widen(dtype: int, bits: np.ndarray) -> np.ndarray:
    """Exact value of each stored element, as float64."""
    src = _storage_view(dtype, bits)
    out = np.empty(src.size, dtype=np.float64)
    _load().tbe_oracle_widen_array(dtype, _ptr(src), _ptr(out), src.size)
    return out


def narrow(dtype: int, x: np.ndarray) -> np.ndarray:
    """Round float64 values to the storage dtype (ties to even); returns raw bits."""
    src = np.ascontiguousarray(x, dtype=np.float64).reshape(-1)
    out = np.empty(src.size, dtype=np.uint32 if dtype == F32 else np.uint16)
    _load().tbe_oracle_narrow_array(dtype, _ptr(src), _ptr(out), src.size)
    return out


def forward(rows, dims, dtype, pooling, weights, B, indices, offsets, psw=None, lib=None):
    """Y [B, sum(dims)] float64."""
    rows, dims, indices, offsets, psw = _i64(rows), _i32(dims), _i64(indices), _i64(offsets), _f32(psw)
    w = _storage_view(dtype, weights)
    out = np.empty((B, int(dims.sum())), dtype=np.float64)
    rc = (lib or _load()).tbe_oracle_forward(len(rows), _ptr(rows), _ptr(dims), dtype, pooling,
                                             _ptr(w), B,
                                    _ptr(indices), _ptr(offsets), indices.size, _ptr(psw), _ptr(out))
    _check(rc, "forward")
    return out


def forward_bags(rows, dims, dtype, pooling, weights, B, indices, offsets, psw, bag_ids):
    """Pooled vectors of the listed bags: list of float64 arrays (len dims[t])."""
    rows, dims, indices, offsets, psw = _i64(rows), _i32(dims), _i64(indices), _i64(offsets), _f32(psw)
    bag_ids = _i64(bag_ids)
    w = _storage_view(dtype, weights)
    sizes = dims[bag_ids // B].astype(np.int64) if bag_ids.size else np.zeros(0, np.int64)
    out = np.empty(int(sizes.sum()), dtype=np.float64)
    rc = _load().tbe_oracle_forward_bags(len(rows), _ptr(rows), _ptr(dims), dtype, pooling, _ptr(w),
                                         B, _ptr(indices), _ptr(offsets), indices.size, _ptr(psw),
                                         bag_ids.size, _ptr(bag_ids), _ptr(out))
    _check(rc, "forward_bags")
    return np.split(out, np.cumsum(sizes)[:-1]) if bag_ids.size else []


def runs(rows, B, indices, offsets):
    """(unique linear row ids ascending, lookup count of each) as int64 arrays."""
    rows, indices, offsets = _i64(rows), _i64(indices), _i64(offsets)
    n = indices.size
    uniq = np.empty(max(n, 1), dtype=np.int64)
    cnt = np.empty(max(n, 1), dtype=np.int64)
    u = ctypes.c_int64(0)
    rc = _load().tbe_oracle_runs(len(rows), _ptr(rows), B, _ptr(indices), _ptr(offsets), n,
                                 _ptr(uniq), _ptr(cnt), ctypes.byref(u))
    _check(rc, "runs")
    return uniq[:u.value].copy(), cnt[:u.value].copy()


def dense_grad(rows, dims, pooling, B, indices, offsets, psw, grad_output):
    """Summed row gradients in the flat weights layout, float64."""
    rows, dims, indices, offsets, psw = _i64(rows), _i32(dims), _i64(indices), _i64(offsets), _f32(psw)
    g = np.ascontiguousarray(grad_output, dtype=np.float32)
    out = np.empty(int((rows * dims.astype(np.int64)).sum()), dtype=np.float64)
    rc = _load().tbe_oracle_dense_grad(len(rows), _ptr(rows), _ptr(dims), pooling, B, _ptr(indices),
                                       _ptr(offsets), indices.size, _ptr(psw), _ptr(g), _ptr(out))
    _check(rc, "dense_grad")
    return out


def psw_grad(rows, dims, dtype, pooling, weights, B, indices, offsets, grad_output):
    """dL/dp_i for every lookup (float64 [N])."""
    rows, dims, indices, offsets = _i64(rows), _i32(dims), _i64(indices), _i64(offsets)
    g = np.ascontiguousarray(grad_output, dtype=np.float32)
    w = _storage_view(dtype, np.ascontiguousarray(weights))
    out = np.empty(indices.size, dtype=np.float64)
    rc = _load().tbe_oracle_psw_grad(len(rows), _ptr(rows), _ptr(dims), dtype, pooling, _ptr(w), B,
                                     _ptr(indices), _ptr(offsets), indices.size, _ptr(g), _ptr(out))
    _check(rc, "psw_grad")
    return out


def backward_update(rows, dims, dtype, pooling, optimizer, weights, state, B, indices, offsets,
                    psw, grad_output, lr, eps, selected_rows=None, lib=None):
    """Apply one optimizer step in place on ``weights`` (storage dtype) and ``state`` (fp32)."""
    rows, dims, indices, offsets, psw = _i64(rows), _i32(dims), _i64(indices), _i64(offsets), _f32(psw)
    g = np.ascontiguousarray(grad_output, dtype=np.float32)
    if not weights.flags.c_contiguous:
        raise ValueError("weights must be contiguous (updated in place)")
    w = _storage_view(dtype, weights)
    if state is not None and (state.dtype != np.float32 or not state.flags.c_contiguous):
        raise ValueError("state must be a contiguous float32 array (updated in place)")
    sel = None if selected_rows is None else _i64(selected_rows)
    nsel = 0 if sel is None else sel.size
    if sel is not None and nsel == 0:
        return
    rc = (lib or _load()).tbe_oracle_backward_update(len(rows), _ptr(rows), _ptr(dims), dtype,
                                                     pooling,
                                            optimizer, _ptr(w), _ptr(state), B, _ptr(indices),
                                            _ptr(offsets), indices.size, _ptr(psw), _ptr(g),
                                            float(lr), float(eps), nsel, _ptr(sel))
    _check(rc, "backward_update")


def set_threads(n: int, lib=None) -> None:
    (lib or _load()).tbe_oracle_set_threads(int(n))


def get_threads(lib=None) -> int:
    return int((lib or _load()).tbe_oracle_get_threads())
