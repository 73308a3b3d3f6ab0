"""ctypes view of the C ABI in include/linattn.h (argument marshalling only).

The shared library is built in-tree by ``kernelized_causal_attention_amd.build``
into ``_lib/liblinattn.so``.  If it is missing, importing this module raises:
there is no fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "_lib", "liblinattn.so")

LA_OK, LA_ERR_INVALID, LA_ERR_UNSUPPORTED, LA_ERR_DEVICE = 0, 1, 2, 3
LA_F32, LA_BF16 = 0, 1
LA_OP_FORWARD, LA_OP_BACKWARD, LA_OP_PREFIX_STATE, LA_OP_DECODE = 0, 1, 2, 3
LA_OP_FORWARD_STATE, LA_OP_BACKWARD_STATE = 4, 5
LA_OP_RETENTION_FORWARD, LA_OP_RETENTION_BACKWARD = 6, 7
LA_OP_POLY_BACKWARD = 8
LA_KERNEL_AUTO, LA_KERNEL_GENERIC, LA_KERNEL_MFMA, LA_KERNEL_MFMA_ONE_LAUNCH = 0, 1, 2, 3

# Every symbol include/linattn.h declares.
EXPORTS = (
    "la_forward", "la_forward_ex", "la_backward", "la_backward_ex", "la_decode_step",
    "la_prefix_state", "la_workspace_bytes", "la_workspace_bytes_ex", "la_resolve_plan",
    "la_status_str", "la_last_error", "la_version", "la_profile_enable", "la_profile_report",
    "la_profile_select", "la_saved_bytes", "la_forward_state", "la_backward_state", "la_retention_forward",
    "la_retention_backward",
    "la_retention_decode_step",
    "la_retention_saved_bytes",
    "la_poly_forward",
    "la_poly_backward",
    "la_poly_prefix_state",
    "la_poly_decode_step",
    "la_softmax_forward",
    "la_softmax_decode_step",
    "la_forward_noalloc",
    "la_device_error",
)


class la_plan(ctypes.Structure):
    _fields_ = [("chunk", ctypes.c_int32), ("segments", ctypes.c_int32), ("kernel", ctypes.c_int32)]


class LinAttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{_status_name(status)}: {msg}")
        self.status = status


_lib = None


def _status_name(s: int) -> str:
    return {0: "LA_OK", 1: "LA_ERR_INVALID", 2: "LA_ERR_UNSUPPORTED", 3: "LA_ERR_DEVICE"}.get(s, f"status {s}")


def load() -> ctypes.CDLL:
    """Load the library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python -m kernelized_causal_attention_amd.build` "
            "(hipcc, gfx950).  There is no fallback path."
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    fp = ctypes.c_void_p
    plan_p = ctypes.POINTER(la_plan)
    fwd = [vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, fp, vp, sz, vp]
    bwd = [vp, vp, vp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp, sz, vp]
    sigs = {
        "la_forward": (fwd, i32),
        "la_forward_ex": (fwd[:12] + [fp, sz] + fwd[12:] + [plan_p], i32),
        "la_forward_noalloc": (fwd[:12] + [vp], i32),
        "la_backward": (bwd, i32),
        "la_backward_ex": (bwd[:6] + [fp, sz] + bwd[6:] + [plan_p], i32),
        "la_saved_bytes": ([i64, i64, i64, i64, i64, i32, i32, plan_p], sz),
        "la_forward_state": ([vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, fp, fp, fp, fp, fp, vp, sz, vp], i32),
        "la_retention_forward": ([vp, vp, vp, fp, vp, i64, i64, i64, i64, i64, i32, fp, fp, fp, sz, vp, sz, vp],
                                 i32),
        "la_retention_saved_bytes": ([i64, i64, i64, i64, i64, i32], sz),
        "la_poly_prefix_state": ([vp, vp, vp, vp, i64, i64, i64, i64, i64, i32, vp], i32),
        "la_poly_decode_step": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp], i32),
        "la_softmax_forward": ([vp, vp, vp, vp, fp, i64, i64, i64, i64, i64, i32, i32, vp], i32),
        "la_softmax_decode_step": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, i32, vp], i32),
        "la_poly_forward": ([vp, vp, vp, vp, fp, i64, i64, i64, i64, i64, i32, i32, vp], i32),
        "la_poly_backward": ([vp, vp, vp, vp, vp, fp, vp, vp, vp, i64, i64, i64, i64, i64, i32, i32, vp, sz, vp], i32),
        "la_retention_decode_step": ([vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp], i32),
        "la_retention_backward": ([vp, vp, vp, fp, vp, fp, fp, sz, vp, vp, vp, fp, fp, i64, i64, i64, i64, i64, i32,
                                   vp, sz, vp], i32),
        "la_backward_state": ([vp, vp, vp, vp, vp, fp, fp, fp, vp, vp, vp, fp, fp, i64, i64, i64, i64, i64, i32,
                               vp, sz, vp], i32),
        "la_decode_step": ([fp, fp, vp, vp, vp, vp, i64, i64, i64, i64, i32, vp], i32),
        "la_prefix_state": ([vp, vp, fp, fp, i64, i64, i64, i64, i64, i32, vp, sz, vp], i32),
        "la_workspace_bytes": ([i32, i64, i64, i64, i64, i64, i32, i32], sz),
        "la_workspace_bytes_ex": ([i32, i64, i64, i64, i64, i64, i32, i32, plan_p], sz),
        "la_resolve_plan": ([i32, i64, i64, i64, i64, i64, i32, i32, plan_p, plan_p], i32),
        "la_status_str": ([i32], ctypes.c_char_p),
        "la_last_error": ([], ctypes.c_char_p),
        "la_device_error": ([vp], i32),
        "la_version": ([], i32),
        "la_profile_enable": ([i32], i32),
        "la_profile_report": ([ctypes.c_char_p, sz], i32),
        "la_profile_select": ([ctypes.c_char_p], i32),
    }
    for name, (args, res) in sigs.items():
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = res
    _lib = lib
    return lib


def check(status: int) -> None:
    if status != LA_OK:
        raise LinAttnError(status, load().la_last_error().decode())
