"""ctypes front end of the fp64 C oracle (ssd_oracle.c) -- TEST INFRASTRUCTURE.

Every function takes float64 numpy arrays laid out as the GPU library's
buffers (x [Z,L,H,P], dt [Z,L,H], B/C [Z,L,G,N], A/D [H], states
[Z,H,P,N]) and returns float64 results.  The arithmetic lives in
ssd_oracle.c; this file only marshals arrays.  See that file's header for the
passages each routine follows.
"""
from __future__ import annotations

import ctypes as C
import os
import threading

import numpy as np

from . import build as _build
from . import dt_act as _dt

_lock = threading.Lock()
_lib = None


class _Shape(C.Structure):
    _fields_ = [("Z", C.c_int64), ("L", C.c_int64), ("H", C.c_int64),
                ("P", C.c_int64), ("N", C.c_int64), ("G", C.c_int64),
                ("RB", C.c_int64)]


class _Dir(C.Structure):
    _fields_ = [("dt", C.c_void_p), ("A", C.c_void_p), ("B", C.c_void_p),
                ("C", C.c_void_p)]


def lib():
    global _lib
    with _lock:
        if _lib is None:
            path = _build.build(force=False)
            l = C.CDLL(path)
            l.ssdo_forward.restype = C.c_int
            l.ssdo_block_update.restype = C.c_int
            l.ssdo_backward.restype = C.c_int
            l.ssdo_thread_count.restype = C.c_int
            l.ssdo_thread_count.argtypes = [C.c_int]
            _lib = l
    return _lib


def thread_count(nthreads: int = 0) -> int:
    return lib().ssdo_thread_count(int(nthreads))


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _shape_of(inp, rev_block=0):
    Z, L, H, P = inp["x"].shape
    N = inp["B_f"].shape[-1]
    G = inp["B_f"].shape[-2]
    return _Shape(Z, L, H, P, N, G, int(rev_block))


def _dirs(inp, keep):
    out = []
    for d in ("f", "r"):
        arrs = [_f64(inp[f"{k}_{d}"]) for k in ("dt", "A", "B", "C")]
        keep.extend(arrs)
        out.append(_Dir(*[_ptr(a) for a in arrs]))
    return out


def forward(inp: dict, init_state=None, parts: bool = False, final_state: bool = False,
            nthreads: int = 0, rev_block: int = 0):
    """y = y_fwd + y_rev + D x.  Returns y, or a dict with y, y_f, y_r and
    final_state when ``parts`` or ``final_state`` is set.  ``rev_block`` > 0
    restarts the reverse scan from zero at the end of every block of that
    many tokens (0: one reverse scan over the whole sequence).  A direction
    with ``dt_bias_<d>`` in ``inp`` takes its dt through the post-processing
    of dt_act.py first."""
    inp = _dt.effective(inp)
    keep = []
    x = _f64(inp["x"])
    D = _f64(inp["D"])
    fwd, rev = _dirs(inp, keep)
    s = _shape_of(inp, rev_block)
    y = np.empty_like(x)
    yf = np.empty_like(x) if parts else None
    yr = np.empty_like(x) if parts else None
    S0 = None if init_state is None else _f64(init_state)
    fs = np.empty((s.Z, s.H, s.P, s.N)) if final_state else None
    rc = lib().ssdo_forward(C.byref(s), _ptr(x), fwd, rev, _ptr(D), _ptr(S0), _ptr(y),
                            _ptr(yf), _ptr(yr), _ptr(fs), C.c_int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssdo_forward failed ({rc})")
    if parts or final_state:
        return {"y": y, "y_f": yf, "y_r": yr, "final_state": fs}
    return y


def block_update(inp: dict, state_in, want_state_out: bool = True, nthreads: int = 0):
    """Block update with partial bidirectionality.  ``inp`` holds the active
    block's tensors; returns (y_blk, state_out or None)."""
    inp = _dt.effective(inp)
    keep = []
    x = _f64(inp["x"])
    D = _f64(inp["D"])
    fwd, rev = _dirs(inp, keep)
    s = _shape_of(inp)
    S0 = _f64(state_in)
    y = np.empty_like(x)
    so = np.empty_like(S0) if want_state_out else None
    rc = lib().ssdo_block_update(C.byref(s), _ptr(S0), _ptr(x), fwd, rev, _ptr(D), _ptr(y),
                                 _ptr(so), C.c_int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssdo_block_update failed ({rc})")
    return y, so


def backward(inp: dict, dy, init_state=None, nthreads: int = 0, rev_block: int = 0) -> dict:
    """Gradients of sum(dy * y): dx, ddt_f, dA_f, dB_f, dC_f, ddt_r, dA_r,
    dB_r, dC_r, dD (``rev_block`` as in forward).  For a direction with a dt
    bias, ddt_<d> is the gradient of its pre-activation dt and ddt_bias_<d>
    that of the bias."""
    raw = inp
    inp = _dt.effective(inp)
    keep = []
    x = _f64(inp["x"])
    D = _f64(inp["D"])
    dyv = _f64(dy)
    fwd, rev = _dirs(inp, keep)
    s = _shape_of(inp, rev_block)
    S0 = None if init_state is None else _f64(init_state)
    Z, L, H, P, N, G = s.Z, s.L, s.H, s.P, s.N, s.G
    g = {
        "dx": np.empty((Z, L, H, P)),
        "ddt_f": np.empty((Z, L, H)), "dA_f": np.empty(H),
        "dB_f": np.empty((Z, L, G, N)), "dC_f": np.empty((Z, L, G, N)),
        "ddt_r": np.empty((Z, L, H)), "dA_r": np.empty(H),
        "dB_r": np.empty((Z, L, G, N)), "dC_r": np.empty((Z, L, G, N)),
        "dD": np.empty(H),
    }
    order = ["dx", "ddt_f", "dA_f", "dB_f", "dC_f", "ddt_r", "dA_r", "dB_r", "dC_r", "dD"]
    rc = lib().ssdo_backward(C.byref(s), _ptr(x), fwd, rev, _ptr(D), _ptr(S0), _ptr(dyv),
                             *[_ptr(g[k]) for k in order], C.c_int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssdo_backward failed ({rc})")
    for d in ("f", "r"):
        if _dt.has_act(raw, d):
            lo, hi = _dt.limits(raw, d)
            g[f"ddt_{d}"], g[f"ddt_bias_{d}"] = _dt.backward(raw[f"dt_{d}"], raw[f"dt_bias_{d}"],
                                                           lo, hi, g[f"ddt_{d}"])
    return g


def library_path() -> str:
    return os.path.abspath(_build.LIB)
