"""Python binding of the gfx950 TBE library (``libtbe.so``, C ABI in ``include/tbe.h``).

The functions here carry the C names and only marshal arguments: torch tensors
become device pointers, the current torch stream becomes the HIP stream, and
status codes become exceptions.  Every step of the computation runs in the HIP
kernels of the library.  There is no fallback: if the library is missing or
cannot be loaded, importing the binding's entry points raises.

Forward (pooled multi-table lookup) and fused backward (linearize, sort,
run-length encode, segment-reduce, one optimizer update per touched row) are
described in kimbodo.com/?p=28372, "What Happened".
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

__all__ = [
    "TBEError", "library_path", "load", "tbe_create", "tbe_destroy", "tbe_forward",
    "tbe_backward_workspace_size", "tbe_backward_update", "tbe_forward_group",
    "tbe_backward_update_grouped", "tbe_psw_grad", "tbe_set_option", "tbe_stage_times",
    "tbe_status_string", "tbe_abi_version", "tbe_check_device_status",
    "tbe_backward_update_no_alloc", "tbe_forward_scratch_size", "tbe_set_forward_scratch",
    "STATIC_SCRATCH_BYTES", "TBE",
    "F32", "F16", "BF16", "POOL_SUM", "POOL_MEAN", "OPT_SGD", "OPT_ROWWISE_ADAGRAD",
    "FLAG_VALIDATE", "FLAG_NO_HISTOGRAM", "FLAG_FORCE_HISTOGRAM", "FLAG_HISTOGRAM",
    "FLAG_SPLIT_BAGS", "FLAG_COUNT_BACKWARD",
    "OPTION_LONG_RUN_THRESHOLD", "OPTION_PROFILE", "OPTION_SORT", "OPTION_SPIN_LIMIT",
    "OPTION_LDS_FORWARD",
    "EXPORTED_SYMBOLS",
]

F32, F16, BF16 = 0, 1, 2
I32, I64 = 0, 1
POOL_SUM, POOL_MEAN = 0, 1
OPT_SGD, OPT_ROWWISE_ADAGRAD = 0, 1
FLAG_VALIDATE, FLAG_NO_HISTOGRAM, FLAG_FORCE_HISTOGRAM, FLAG_HISTOGRAM = 1, 2, 4, 8
FLAG_SPLIT_BAGS = 16
FLAG_COUNT_BACKWARD = 32
OPTION_LONG_RUN_THRESHOLD, OPTION_PROFILE, OPTION_SORT, OPTION_SPIN_LIMIT = 1, 2, 3, 4
OPTION_LDS_FORWARD = 5
STATIC_SCRATCH_BYTES = 64 << 20   # TBE_STATIC_SCRATCH_BYTES

STATUS = {
    0: "TBE_OK", 1: "TBE_ERR_INVALID_ARGUMENT", 2: "TBE_ERR_UNSUPPORTED",
    3: "TBE_ERR_INDEX_OUT_OF_RANGE", 4: "TBE_ERR_WORKSPACE_TOO_SMALL", 5: "TBE_ERR_HIP",
    6: "TBE_ERR_OUT_OF_MEMORY", 7: "TBE_ERR_DEVICE_WAIT",
}

EXPORTED_SYMBOLS = (
    "tbe_create", "tbe_destroy", "tbe_forward", "tbe_backward_workspace_size",
    "tbe_backward_update", "tbe_forward_group", "tbe_backward_update_grouped", "tbe_psw_grad",
    "tbe_set_option", "tbe_stage_times", "tbe_status_string", "tbe_abi_version",
    "tbe_check_device_status", "tbe_backward_update_no_alloc", "tbe_forward_scratch_size",
    "tbe_set_forward_scratch",
)

_HERE = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_HERE, "libtbe.so")


class TBEError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS.get(status, status)} ({_status_string(status)})")


class _Config(ctypes.Structure):
    _fields_ = [("num_tables", ctypes.c_int32), ("rows", ctypes.POINTER(ctypes.c_int64)),
                ("dims", ctypes.POINTER(ctypes.c_int32)), ("weight_dtype", ctypes.c_int32),
                ("pooling", ctypes.c_int32), ("optimizer", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class _Runs(ctypes.Structure):
    _fields_ = [("unique_ids", ctypes.c_void_p), ("run_lengths", ctypes.c_void_p),
                ("num_unique", ctypes.c_void_p)]


_lib = None


def load():
    """Load ``libtbe.so`` (built by ``table_embedding_bag_amd.build``); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run table_embedding_bag_amd/build.py")
    lib = ctypes.CDLL(path)
    P, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    lib.tbe_create.argtypes = [ctypes.POINTER(_Config), P, P, ctypes.POINTER(P)]
    lib.tbe_destroy.argtypes = [P]
    lib.tbe_destroy.restype = None
    lib.tbe_forward.argtypes = [P, i32, P, P, i32, i64, P, P, P]
    lib.tbe_backward_workspace_size.argtypes = [P, i32, i64, ctypes.POINTER(ctypes.c_size_t)]
    lib.tbe_backward_update.argtypes = [P, i32, P, P, i32, i64, P, P, f32, f32, P,
                                        ctypes.c_size_t, ctypes.POINTER(_Runs), P]
    lib.tbe_forward_group.argtypes = [P, i32, P, P, i32, i64, P, P, P, ctypes.c_size_t, P]
    lib.tbe_backward_update_grouped.argtypes = lib.tbe_backward_update.argtypes
    lib.tbe_backward_update_no_alloc.argtypes = [P, i32, P, P, i32, i64, P, P, f32, f32,
                                                 ctypes.POINTER(_Runs), P]
    lib.tbe_psw_grad.argtypes = [P, i32, P, P, i32, i64, P, P, P]
    lib.tbe_set_option.argtypes = [P, i32, i64]
    lib.tbe_check_device_status.argtypes = [P, P]
    lib.tbe_stage_times.argtypes = [P, ctypes.POINTER(f32), ctypes.POINTER(ctypes.c_char_p), i32,
                                    ctypes.POINTER(i32)]
    lib.tbe_status_string.argtypes = [ctypes.c_int]
    lib.tbe_status_string.restype = ctypes.c_char_p
    lib.tbe_forward_scratch_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.tbe_set_forward_scratch.argtypes = [P, P, ctypes.c_size_t]
    lib.tbe_abi_version.argtypes = []
    lib.tbe_abi_version.restype = i32
    for name in ("tbe_create", "tbe_forward", "tbe_backward_workspace_size", "tbe_backward_update",
                 "tbe_forward_group", "tbe_backward_update_grouped", "tbe_psw_grad",
                 "tbe_set_option", "tbe_stage_times", "tbe_check_device_status",
                 "tbe_backward_update_no_alloc", "tbe_forward_scratch_size",
                 "tbe_set_forward_scratch"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _status_string(status: int) -> str:
    try:
        return load().tbe_status_string(status).decode()
    except Exception:  # library not loadable: keep the numeric code
        return "?"


def _check(status: int, what: str) -> None:
    if status != 0:
        raise TBEError(status, what)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    import torch
    return torch.cuda.current_stream().cuda_stream


def _index_dtype(indices, offsets) -> int:
    import torch
    if indices.dtype != offsets.dtype:
        raise ValueError("indices and offsets must have the same dtype")
    if indices.dtype == torch.int64:
        return I64
    if indices.dtype == torch.int32:
        return I32
    raise ValueError("indices must be int32 or int64")


def tbe_status_string(status: int) -> str:
    return load().tbe_status_string(status).decode()


def tbe_abi_version() -> int:
    return int(load().tbe_abi_version())


def tbe_create(rows: Sequence[int], dims: Sequence[int], weight_dtype: int, pooling: int,
               optimizer: int, weights, state=None, flags: int = 0) -> int:
    """Create a handle over ``weights`` (flat device tensor) and ``state`` (fp32 or None)."""
    T = len(rows)
    if len(dims) != T:
        raise ValueError("rows and dims differ in length")
    r = (ctypes.c_int64 * T)(*[int(x) for x in rows])
    d = (ctypes.c_int32 * T)(*[int(x) for x in dims])
    cfg = _Config(T, r, d, weight_dtype, pooling, optimizer, flags)
    out = ctypes.c_void_p()
    _check(load().tbe_create(ctypes.byref(cfg), _ptr(weights), _ptr(state), ctypes.byref(out)),
           "tbe_create")
    return out.value


def tbe_destroy(handle) -> None:
    if handle:
        load().tbe_destroy(handle)


def tbe_forward_scratch_size(handle) -> int:
    n = ctypes.c_size_t(0)
    _check(load().tbe_forward_scratch_size(handle, ctypes.byref(n)), "tbe_forward_scratch_size")
    return int(n.value)


def tbe_set_forward_scratch(handle, scratch, nbytes: int) -> None:
    _check(load().tbe_set_forward_scratch(handle, _ptr(scratch), int(nbytes)),
           "tbe_set_forward_scratch")


def tbe_forward(handle, B: int, indices, offsets, per_sample_weights, output, stream=None) -> None:
    _check(load().tbe_forward(handle, B, _ptr(indices), _ptr(offsets),
                              _index_dtype(indices, offsets), indices.numel(),
                              _ptr(per_sample_weights), _ptr(output), _stream(stream)),
           "tbe_forward")


def tbe_backward_workspace_size(handle, B: int, num_indices: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load().tbe_backward_workspace_size(handle, B, num_indices, ctypes.byref(n)),
           "tbe_backward_workspace_size")
    return int(n.value)


def tbe_backward_update(handle, B: int, indices, offsets, per_sample_weights, grad_output,
                        lr: float, eps: float, workspace, runs=None, stream=None) -> None:
    """runs: optional (unique_ids int32, run_lengths int32, num_unique int32[1]) device tensors."""
    r = None
    if runs is not None:
        r = ctypes.byref(_Runs(_ptr(runs[0]), _ptr(runs[1]), _ptr(runs[2])))
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().tbe_backward_update(handle, B, _ptr(indices), _ptr(offsets),
                                      _index_dtype(indices, offsets), indices.numel(),
                                      _ptr(per_sample_weights), _ptr(grad_output), float(lr),
                                      float(eps), _ptr(workspace), nbytes, r, _stream(stream)),
           "tbe_backward_update")


def tbe_backward_update_no_alloc(handle, B: int, indices, offsets, per_sample_weights,
                                 grad_output, lr: float, eps: float, runs=None,
                                 stream=None) -> None:
    """tbe_backward_update on the library's static device scratch (no workspace argument)."""
    r = None
    if runs is not None:
        r = ctypes.byref(_Runs(_ptr(runs[0]), _ptr(runs[1]), _ptr(runs[2])))
    _check(load().tbe_backward_update_no_alloc(handle, B, _ptr(indices), _ptr(offsets),
                                               _index_dtype(indices, offsets), indices.numel(),
                                               _ptr(per_sample_weights), _ptr(grad_output),
                                               float(lr), float(eps), r, _stream(stream)),
           "tbe_backward_update_no_alloc")


def tbe_forward_group(handle, B: int, indices, offsets, per_sample_weights, output, workspace,
                      stream=None) -> None:
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().tbe_forward_group(handle, B, _ptr(indices), _ptr(offsets),
                                    _index_dtype(indices, offsets), indices.numel(),
                                    _ptr(per_sample_weights), _ptr(output), _ptr(workspace), nbytes,
                                    _stream(stream)),
           "tbe_forward_group")


def tbe_backward_update_grouped(handle, B: int, indices, offsets, per_sample_weights, grad_output,
                                lr: float, eps: float, workspace, runs=None, stream=None) -> None:
    r = None
    if runs is not None:
        r = ctypes.byref(_Runs(_ptr(runs[0]), _ptr(runs[1]), _ptr(runs[2])))
    nbytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(load().tbe_backward_update_grouped(handle, B, _ptr(indices), _ptr(offsets),
                                              _index_dtype(indices, offsets), indices.numel(),
                                              _ptr(per_sample_weights), _ptr(grad_output), float(lr),
                                              float(eps), _ptr(workspace), nbytes, r,
                                              _stream(stream)),
           "tbe_backward_update_grouped")


def tbe_psw_grad(handle, B: int, indices, offsets, grad_output, grad_psw, stream=None) -> None:
    _check(load().tbe_psw_grad(handle, B, _ptr(indices), _ptr(offsets),
                               _index_dtype(indices, offsets), indices.numel(), _ptr(grad_output),
                               _ptr(grad_psw), _stream(stream)),
           "tbe_psw_grad")


def tbe_check_device_status(handle, stream=None) -> None:
    """Waits for the stream; raises TBEError (TBE_ERR_DEVICE_WAIT) if a backward call since
    the last check skipped its update because a device-side wait gave up."""
    _check(load().tbe_check_device_status(handle, _stream(stream)), "tbe_check_device_status")


def tbe_set_option(handle, option: int, value: int) -> None:
    _check(load().tbe_set_option(handle, option, int(value)), "tbe_set_option")


def tbe_stage_times(handle, capacity: int = 1 << 16):
    """[(stage name, milliseconds)] of the last call (profiling option must be on)."""
    ms = (ctypes.c_float * capacity)()
    names = (ctypes.c_char_p * capacity)()
    n = ctypes.c_int32(0)
    _check(load().tbe_stage_times(handle, ms, names, capacity, ctypes.byref(n)), "tbe_stage_times")
    return [(names[i].decode(), float(ms[i])) for i in range(n.value)]


_DTYPE_CODE = {"f32": F32, "f16": F16, "bf16": BF16}


class TBE:
    """A handle plus the torch allocations a caller needs (output, workspace).

    ``weights`` is the flat device tensor of all tables, ``state`` the fp32
    row-wise Adagrad state (or None for SGD); both stay owned by the caller.
    """

    def __init__(self, rows, dims, weights, state=None, pooling="sum", optimizer="sgd", flags=0):
        import torch
        dt = {torch.float32: F32, torch.float16: F16, torch.bfloat16: BF16}[weights.dtype]
        self.rows = [int(x) for x in rows]
        self.dims = [int(x) for x in dims]
        self.sum_dims = sum(self.dims)
        self.weights = weights
        self.state = state
        self.handle = tbe_create(self.rows, self.dims, dt, {"sum": POOL_SUM, "mean": POOL_MEAN}[pooling],
                                 {"sgd": OPT_SGD, "rowwise_adagrad": OPT_ROWWISE_ADAGRAD}[optimizer],
                                 weights, state, flags)
        self._ws = None
        # the forward's opt-in paths (count-matrix forward, split bags) take
        # their scratch from the caller
        self._fscratch = None
        need = tbe_forward_scratch_size(self.handle)
        if need:
            self._fscratch = torch.empty(need, dtype=torch.uint8, device=weights.device)
            tbe_set_forward_scratch(self.handle, self._fscratch, need)

    def forward(self, B, indices, offsets, per_sample_weights=None, out=None):
        import torch
        if out is None:
            out = torch.empty((B, self.sum_dims), dtype=torch.float32, device=self.weights.device)
        tbe_forward(self.handle, B, indices, offsets, per_sample_weights, out)
        return out

    def workspace(self, B, num_indices):
        import torch
        need = tbe_backward_workspace_size(self.handle, B, num_indices)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.weights.device)
        return self._ws

    def backward_update(self, B, indices, offsets, per_sample_weights, grad_output, lr, eps=1e-8,
                        runs=None):
        ws = self.workspace(B, indices.numel())
        tbe_backward_update(self.handle, B, indices, offsets, per_sample_weights, grad_output, lr,
                            eps, ws, runs)

    def forward_group(self, B, indices, offsets, per_sample_weights=None, out=None):
        """Forward plus the backward's grouping of this batch (kept in the handle's workspace
        for backward_update_grouped)."""
        import torch
        if out is None:
            out = torch.empty((B, self.sum_dims), dtype=torch.float32, device=self.weights.device)
        ws = self.workspace(B, indices.numel())
        tbe_forward_group(self.handle, B, indices, offsets, per_sample_weights, out, ws)
        return out

    def backward_update_grouped(self, B, indices, offsets, per_sample_weights, grad_output, lr,
                                eps=1e-8, runs=None):
        ws = self.workspace(B, indices.numel())
        tbe_backward_update_grouped(self.handle, B, indices, offsets, per_sample_weights,
                                    grad_output, lr, eps, ws, runs)

    def psw_grad(self, B, indices, offsets, grad_output, out=None):
        """dL/dp for every lookup (fp32 [N]); call before backward_update changes the weights."""
        import torch
        if out is None:
            out = torch.empty(indices.numel(), dtype=torch.float32, device=self.weights.device)
        tbe_psw_grad(self.handle, B, indices, offsets, grad_output, out)
        return out

    def set_option(self, option, value):
        tbe_set_option(self.handle, option, value)

    def check_device_status(self):
        tbe_check_device_status(self.handle)

    def stage_times(self):
        return tbe_stage_times(self.handle)

    def close(self):
        if self.handle:
            tbe_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
