"""ctypes declarations of the C ABI in include/bissd.h.

Loads the in-tree libbissd.so built by ``state_space_denoisers_amd.build``.
There is no fallback: if the library is missing or fails to load, every call
raises.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libbissd.so")

BISSD_F32 = 0
BISSD_BF16 = 1
OP_FORWARD, OP_BACKWARD, OP_BLOCK = 0, 1, 2
SAVE = 1  # shape flag: the forward keeps what the backward reads

STATUS = {
    0: "BISSD_OK", -1: "BISSD_ERR_NULL", -2: "BISSD_ERR_SHAPE", -3: "BISSD_ERR_UNSUPPORTED",
    -4: "BISSD_ERR_ALIGN", -5: "BISSD_ERR_WORKSPACE", -6: "BISSD_ERR_HIP", -7: "BISSD_ERR_ALIAS",
    -8: "BISSD_ERR_SCRATCH",
}
NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/bissd.h declares
EXPORTS = ("bissd_workspace_size", "bissd_forward", "bissd_forward_noalloc", "bissd_backward",
           "bissd_block_update",
           "bissd_forward_phase", "bissd_attention_forward", "bissd_attention_backward",
           "bissd_attention_workspace_size", "bissd_status_string", "bissd_last_hip_error",
           "bissd_timer_arm", "bissd_timer_read", "bissd_version")


class Shape(C.Structure):
    _fields_ = [("batch", C.c_int64), ("seqlen", C.c_int64), ("nheads", C.c_int64),
                ("headdim", C.c_int64), ("dstate", C.c_int64), ("ngroups", C.c_int64),
                ("chunk", C.c_int64), ("dtype", C.c_int32), ("rev_block", C.c_int32),
                ("conv_width", C.c_int32), ("flags", C.c_int32)]


class AttnShape(C.Structure):
    _fields_ = [("batch", C.c_int64), ("seqlen", C.c_int64), ("nheads", C.c_int64),
                ("headdim", C.c_int64), ("block", C.c_int64), ("dtype", C.c_int32),
                ("reserved", C.c_int32)]


class Dir(C.Structure):
    _fields_ = [("dt", C.c_void_p), ("A", C.c_void_p), ("B", C.c_void_p), ("C", C.c_void_p),
                ("dt_bias", C.c_void_p), ("dt_min", C.c_float), ("dt_max", C.c_float),
                ("conv_w", C.c_void_p), ("conv_b", C.c_void_p), ("conv_act", C.c_int32),
                ("reserved", C.c_int32)]


class Grad(C.Structure):
    _fields_ = [("ddt", C.c_void_p), ("dA", C.c_void_p), ("dB", C.c_void_p), ("dC", C.c_void_p),
                ("ddt_bias", C.c_void_p)]


class BissdError(RuntimeError):
    def __init__(self, fn: str, status: int, detail: str = ""):
        self.status = status
        msg = f"{fn} failed: {STATUS.get(status, status)}"
        if detail:
            msg += f" ({detail})"
        super().__init__(msg)


_lock = threading.Lock()
_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load libbissd.so (once).  Raises if it has not been built."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError(
                f"HIP library not built: {path} is missing "
                "(run `python -c 'import __graft_entry__ as g; g.build()'`)")
        lib = C.CDLL(path)
        lib.bissd_workspace_size.restype = C.c_size_t
        lib.bissd_workspace_size.argtypes = [C.POINTER(Shape), C.c_int]
        lib.bissd_forward.restype = C.c_int
        lib.bissd_forward.argtypes = [C.POINTER(Shape), C.c_void_p, Dir, Dir, C.c_void_p,
                                      C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                      C.c_size_t, C.c_void_p]
        lib.bissd_forward_noalloc.restype = C.c_int
        lib.bissd_forward_noalloc.argtypes = [C.POINTER(Shape), C.c_void_p, Dir, Dir, C.c_void_p,
                                              C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]
        lib.bissd_forward_phase.restype = C.c_int
        lib.bissd_forward_phase.argtypes = lib.bissd_forward.argtypes + [C.c_int]
        lib.bissd_backward.restype = C.c_int
        lib.bissd_backward.argtypes = [C.POINTER(Shape), C.c_void_p, Dir, Dir, C.c_void_p,
                                       C.c_void_p, C.c_void_p, C.c_void_p, Grad, Grad,
                                       C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        lib.bissd_block_update.restype = C.c_int
        lib.bissd_block_update.argtypes = [C.POINTER(Shape), C.c_void_p, C.c_void_p, Dir, Dir,
                                           C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p,
                                           C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        lib.bissd_attention_forward.restype = C.c_int
        lib.bissd_attention_forward.argtypes = [C.POINTER(AttnShape), C.c_void_p, C.c_void_p,
                                                C.c_void_p, C.c_float, C.c_void_p, C.c_void_p,
                                                C.c_void_p]
        lib.bissd_attention_workspace_size.restype = C.c_size_t
        lib.bissd_attention_workspace_size.argtypes = [C.POINTER(AttnShape)]
        lib.bissd_attention_backward.restype = C.c_int
        lib.bissd_attention_backward.argtypes = [C.POINTER(AttnShape)] + [C.c_void_p] * 6 + [
            C.c_float, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_size_t, C.c_void_p]
        lib.bissd_status_string.restype = C.c_char_p
        lib.bissd_status_string.argtypes = [C.c_int]
        lib.bissd_last_hip_error.restype = C.c_int
        lib.bissd_last_hip_error.argtypes = []
        lib.bissd_timer_arm.restype = C.c_int
        lib.bissd_timer_arm.argtypes = [C.c_int32]
        lib.bissd_timer_read.restype = C.c_int
        lib.bissd_timer_read.argtypes = [C.c_int32, C.POINTER(C.c_float)]
        lib.bissd_version.restype = C.c_int
        lib.bissd_version.argtypes = []
        _lib = lib
        return lib


def check(fn: str, status: int) -> None:
    if status != 0:
        lib = load()
        detail = lib.bissd_status_string(status).decode()
        if status == -6:
            detail += f"; hipError {lib.bissd_last_hip_error()}"
        raise BissdError(fn, status, detail)
