"""ctypes binding of libi4s (include/i4s.h), same names as the C ABI.

Argument marshalling only: every step of packing and of the GEMV runs in the
HIP kernels of libi4s.so.  There is no fallback: if the library is missing,
loading raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libi4s.so")

I4S_OK = 0
I4S_ERR_INVALID_ARGUMENT = 1
I4S_ERR_UNSUPPORTED = 2
I4S_ERR_NONFINITE_WEIGHT = 3
I4S_ERR_WORKSPACE_TOO_SMALL = 4
I4S_ERR_DEVICE = 5
I4S_MAX_BATCH = 16
I4S_MAX_MULTI = 8
I4S_NOALLOC_SCRATCH_BYTES = 32 << 20
I4S_FORMAT_VERSION = 1


class i4s_packed(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_int32),
        ("cols", ctypes.c_int32),
        ("n_keep", ctypes.c_int32),
        ("group_size", ctypes.c_int32),
        ("nnz", ctypes.c_int64),
        ("row_ptr", ctypes.c_void_p),
        ("vals", ctypes.c_void_p),
        ("codes", ctypes.c_void_p),
        ("scales", ctypes.c_void_p),
    ]


class i4s_sizes(ctypes.Structure):
    _fields_ = [
        ("row_ptr", ctypes.c_uint64),
        ("vals", ctypes.c_uint64),
        ("codes", ctypes.c_uint64),
        ("scales", ctypes.c_uint64),
        ("workspace", ctypes.c_uint64),
    ]


class i4s_pack_report(ctypes.Structure):
    _fields_ = [
        ("group_size", ctypes.c_int32),
        ("n_candidates", ctypes.c_int32),
        ("candidates", ctypes.c_int32 * 3),
        ("reserved", ctypes.c_int32),
        ("sse_hi", ctypes.c_uint64 * 3),
        ("sse_lo", ctypes.c_uint64 * 3),
    ]


# every symbol include/i4s.h declares, with its ctypes signature
SIGNATURES = {
    "i4s_pack_sizes": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(i4s_sizes)]),
    "i4s_pack": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                ctypes.c_int32, ctypes.c_void_p, ctypes.c_uint64,
                                ctypes.POINTER(i4s_packed), ctypes.POINTER(i4s_pack_report),
                                ctypes.c_void_p]),
    "i4s_pack_ex": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_uint64, ctypes.POINTER(i4s_packed),
                                   ctypes.POINTER(i4s_pack_report), ctypes.c_void_p]),
    "i4s_run": (ctypes.c_int, [ctypes.POINTER(i4s_packed), ctypes.c_void_p, ctypes.c_int32,
                               ctypes.c_void_p, ctypes.c_void_p]),
    "i4s_run_workspace_size": (ctypes.c_int, [ctypes.POINTER(i4s_packed), ctypes.c_int32,
                                              ctypes.POINTER(ctypes.c_uint64)]),
    "i4s_run_ws": (ctypes.c_int, [ctypes.POINTER(i4s_packed), ctypes.c_void_p, ctypes.c_int32,
                                  ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint64, ctypes.c_void_p]),
    "i4s_run_noalloc": (ctypes.c_int, [ctypes.POINTER(i4s_packed), ctypes.c_void_p, ctypes.c_int32,
                                       ctypes.c_void_p, ctypes.c_void_p]),
    "i4s_run_multi": (ctypes.c_int, [ctypes.POINTER(i4s_packed), ctypes.c_int32, ctypes.c_void_p, ctypes.c_int32,
                                     ctypes.POINTER(ctypes.c_void_p), ctypes.c_void_p]),
    "i4s_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "i4s_last_error": (ctypes.c_char_p, []),
    "i4s_version": (ctypes.c_int32, []),
    "i4s_format_version": (ctypes.c_int32, []),
}

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libi4s.so (once) and attach the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m int4_sparse_gemv_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


class I4SError(RuntimeError):
    def __init__(self, status: int, where: str):
        lib = load()
        self.status = status
        msg = lib.i4s_last_error().decode(errors="replace")
        super().__init__(f"{where}: {lib.i4s_status_string(status).decode()} ({status}): {msg}")


def check(status: int, where: str) -> None:
    if status != I4S_OK:
        raise I4SError(status, where)


# thin wrappers with the C names --------------------------------------------

def i4s_pack_sizes(rows, cols, n_keep, group_size, out):
    return load().i4s_pack_sizes(rows, cols, n_keep, group_size, ctypes.byref(out))


def i4s_pack(w_ptr, rows, cols, n_keep, group_size, ws_ptr, ws_bytes, inout, report, stream):
    rep = ctypes.byref(report) if report is not None else None
    return load().i4s_pack(w_ptr, rows, cols, n_keep, group_size, ws_ptr, ws_bytes,
                           ctypes.byref(inout), rep, stream)


def i4s_pack_ex(w_ptr, rows, cols, n_keep, group_size, norm_ptr, grad_ptr, ws_ptr, ws_bytes, inout,
                report, stream):
    rep = ctypes.byref(report) if report is not None else None
    return load().i4s_pack_ex(w_ptr, rows, cols, n_keep, group_size, norm_ptr, grad_ptr, ws_ptr,
                              ws_bytes, ctypes.byref(inout), rep, stream)


def i4s_run(packed, x_ptr, batch, y_ptr, stream):
    return load().i4s_run(ctypes.byref(packed), x_ptr, batch, y_ptr, stream)


def i4s_run_workspace_size(packed, batch, out):
    return load().i4s_run_workspace_size(ctypes.byref(packed), batch, ctypes.byref(out))


def i4s_run_ws(packed, x_ptr, batch, y_ptr, ws_ptr, ws_bytes, stream):
    return load().i4s_run_ws(ctypes.byref(packed), x_ptr, batch, y_ptr, ws_ptr, ws_bytes, stream)


def i4s_run_noalloc(packed, x_ptr, batch, y_ptr, stream):
    return load().i4s_run_noalloc(ctypes.byref(packed), x_ptr, batch, y_ptr, stream)


def i4s_run_multi(packed_list, x_ptr, batch, y_ptrs, stream):
    """packed_list: sequence of i4s_packed; y_ptrs: sequence of device addresses."""
    n = len(packed_list)
    arr = (i4s_packed * max(n, 1))(*packed_list)
    ys = (ctypes.c_void_p * max(n, 1))(*y_ptrs)
    return load().i4s_run_multi(arr, n, x_ptr, batch, ys, stream)


def i4s_status_string(status):
    return load().i4s_status_string(status).decode()


def i4s_last_error():
    return load().i4s_last_error().decode()


def i4s_version():
    return load().i4s_version()


def i4s_format_version():
    return load().i4s_format_version()
