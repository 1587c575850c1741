"""ctypes binding of ``librsx.so`` (the C ABI in ``include/rsx.h``).

Argument marshalling only: every element of every collective is computed by
the HIP kernels inside the library.  There is no fallback: if the library is
missing, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("RSX_LIB", os.path.join(PKG, "librsx.so"))

RSX_FLOAT32, RSX_BFLOAT16, RSX_INT32 = 0, 1, 2
RSX_FLOAT64, RSX_FLOAT16, RSX_INT64, RSX_UINT64, RSX_INT8 = 3, 4, 5, 6, 7
RSX_FLOAT32_HALF_WIRE = 8
RSX_SUM, RSX_MAX, RSX_MIN, RSX_AVG, RSX_PROD = 0, 1, 2, 3, 4
RSX_ALGO_RING, RSX_ALGO_NAIVE, RSX_ALGO_AUTO, RSX_ALGO_RING_FUSED, RSX_ALGO_RING_SPLIT = 0, 1, 2, 3, 4
RSX_SPARSE_THRESHOLD, RSX_SPARSE_TOPK = 0, 1
RSX_MAX_RANKS = 16
RSX_NAIVE_MAX_BYTES = 32768
RSX_FUSE_BATCH = 248
RSX_FUSION_THRESHOLD_DEFAULT = 64 * 1024 * 1024   # Horovod's default tensor_fusion_threshold

STATUS = {
    0: "RSX_SUCCESS",
    1: "RSX_ERR_INVALID_ARGUMENT",
    2: "RSX_ERR_INVALID_TYPE",
    3: "RSX_ERR_INVALID_OP",
    4: "RSX_ERR_UNSUPPORTED",
    5: "RSX_ERR_ALIASING",
    6: "RSX_ERR_HIP",
}

# name -> (restype, argtypes); every function include/rsx.h declares.
_P = ctypes.c_void_p
_PP = ctypes.POINTER(ctypes.c_void_p)
_SZ = ctypes.c_size_t
_I = ctypes.c_int
SIGNATURES = {
    "rsx_reduce_scatter": (_I, [_PP, _PP, _I, _SZ, _I, _I, _P]),
    "rsx_all_gather": (_I, [_PP, _PP, _I, _SZ, _I, _P]),
    "rsx_all_reduce": (_I, [_PP, _PP, _I, _SZ, _I, _I, _I, _P]),
    "rsx_all_reduce_bucketed": (_I, [_PP, _PP, _I, _SZ, _SZ, _I, _I, _I, _P]),
    "rsx_all_reduce_bucket": (_I, [_PP, _PP, _I, _SZ, _SZ, _SZ, _I, _I, _I, _P]),
    "rsx_bucket_count": (_SZ, [_SZ, _SZ]),
    "rsx_fuse_pack": (_I, [_PP, ctypes.POINTER(_SZ), _I, _P, _I, _P]),
    "rsx_fuse_unpack": (_I, [_P, _PP, ctypes.POINTER(_SZ), _I, _I, _P]),
    "rsx_fused_all_reduce": (_I, [_PP, _PP, ctypes.POINTER(_SZ), _I, _I, _I, _I, _I, _P]),
    "rsx_fusion_plan": (_I, [ctypes.POINTER(_SZ), ctypes.POINTER(_I), _I, _SZ, ctypes.POINTER(_I)]),
    "rsx_sparse_topk_count": (_SZ, [_SZ, ctypes.c_float]),
    "rsx_sparse_workspace_size": (_SZ, [_I, _SZ, _I, _I]),
    "rsx_sparse_all_reduce": (_I, [_PP, _PP, _PP, _I, _SZ, _I, ctypes.c_float, _SZ, _PP, _PP, _SZ,
                                   _P, _P, _SZ, _P]),
    "rsx_sparse_all_reduce_noalloc": (_I, [_PP, _PP, _PP, _I, _SZ, _I, ctypes.c_float, _SZ, _PP, _PP,
                                           _SZ, _P, _P]),
    "rsx_segment_begin": (_SZ, [_SZ, _I, _I]),
    "rsx_dtype_size": (_SZ, [_I]),
    "rsx_status_string": (ctypes.c_char_p, [_I]),
    "rsx_version": (_I, []),
    "rsx_set_occupancy_caps": (_I, [_I]),
}


class RsxError(RuntimeError):
    """A non-success status from librsx."""

    def __init__(self, fn: str, status: int, text: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({text})")
        self.status = status
        self.fn = fn


_lock = threading.Lock()
_lib = None


def _check_single_hip_runtime() -> None:
    """Refuse to run with two HIP runtimes mapped (e.g. torch's and /opt/rocm's)."""
    try:
        with open("/proc/self/maps") as f:
            libs = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    if len(libs) > 1:
        raise RuntimeError(f"two HIP runtimes loaded in one process: {sorted(libs)}")


def lib():
    """The loaded library; raises if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"librsx.so not found at {LIB_PATH}; build it with "
                "`python -m collective_reduction_ring_amd.build`")
        # Load torch first so the library binds to the HIP runtime torch uses.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _check_single_hip_runtime()
        _lib = handle
    return _lib


def check(fn: str, status: int) -> None:
    if status != 0:
        text = lib().rsx_status_string(status).decode()
        raise RsxError(fn, status, text)


def ptr_array(ptrs) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(ptrs)))()
    for i, p in enumerate(ptrs):
        arr[i] = p
    return arr


def size_array(vals) -> ctypes.Array:
    arr = (ctypes.c_size_t * max(1, len(vals)))()
    for i, v in enumerate(vals):
        arr[i] = int(v)
    return arr
