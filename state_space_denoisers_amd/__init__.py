"""Bidirectional SSD (Mamba-2) scan for AMD Instinct MI355X.

Thin Python binding over the C ABI of libbissd.so (include/bissd.h).  The
functions carry the ABI's names and only marshal arguments: torch provides
device memory and the current stream, and every step of the scan runs in the
library's HIP kernels.  There is no CPU or PyTorch fallback.

    y = bissd_forward(x, fwd, rev, D, chunk=256)
    y, state_out = bissd_block_update(state_in, x_blk, fwd, rev, D)
    grads = bissd_backward(x, fwd, rev, D, dy)

``fwd`` / ``rev`` are (dt, A, B, C) tuples or ``Dir``s: dt [Z,L,H], A [H]
fp32, B and C [Z,L,G,N]; x [Z,L,H,P]; D [H] fp32.  x, dt, B, C (and dy) share
one dtype, torch.float32 or torch.bfloat16.  A ``Dir`` with ``dt_bias`` ([H]
fp32) makes the kernels read dt as clamp(softplus(dt + dt_bias), dt_min,
dt_max).
"""
from __future__ import annotations

import ctypes as C
from typing import NamedTuple, Optional

import torch

from . import _abi

__all__ = ["Dir", "bissd_forward", "bissd_forward_phase", "bissd_block_update", "bissd_backward",
           "bissd_attention_forward", "bissd_attention_backward", "bissd_workspace_size",
           "shape_of", "library_path", "BissdError"]

BissdError = _abi.BissdError


class Dir(NamedTuple):
    dt: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    C: torch.Tensor
    dt_bias: Optional[torch.Tensor] = None
    dt_min: float = 0.0
    dt_max: float = float("inf")


def library_path() -> str:
    return _abi.LIB_PATH


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.BISSD_BF16
    if t.dtype == torch.float32:
        return _abi.BISSD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


_SHAPES: dict = {}


def shape_of(x: torch.Tensor, B: torch.Tensor, chunk: int, rev_block: int = 0) -> _abi.Shape:
    """The ABI shape struct for x / B (memoised: block updates call this in
    tight loops, and the C side only reads it)."""
    key = (x.shape, B.shape, x.dtype, chunk, rev_block)
    s = _SHAPES.get(key)
    if s is None:
        Z, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        s = _abi.Shape(Z, L, H, P, N, G, int(chunk), _dtype_code(x), int(rev_block))
        if len(_SHAPES) > 1024:
            _SHAPES.clear()
        _SHAPES[key] = s
    return s


def _ptr(t: Optional[torch.Tensor]):
    """Device address of a contiguous tensor (None for NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to libbissd must be contiguous")
    return t.data_ptr()


def _dir(d) -> _abi.Dir:
    d = Dir(*d)
    if d.A.dtype != torch.float32:
        raise TypeError(f"A must be torch.float32, got {d.A.dtype}")
    if d.dt_bias is not None and d.dt_bias.dtype != torch.float32:
        raise TypeError(f"dt_bias must be torch.float32, got {d.dt_bias.dtype}")
    return _abi.Dir(_ptr(d.dt), _ptr(d.A), _ptr(d.B), _ptr(d.C), _ptr(d.dt_bias),
                    float(d.dt_min), float(d.dt_max))


def _stream(device: torch.device, stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def bissd_workspace_size(shape: _abi.Shape, op: int) -> int:
    return int(_abi.load().bissd_workspace_size(C.byref(shape), int(op)))


def _workspace(shape, op, device, workspace):
    if workspace is not None:
        return workspace, workspace.numel() * workspace.element_size()
    n = bissd_workspace_size(shape, op)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


def bissd_forward(x: torch.Tensor, fwd, rev, D: torch.Tensor, *, chunk: int = 256,
                  rev_block: int = 0, init_state: Optional[torch.Tensor] = None,
                  y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """y = yf + yr + D x (see include/bissd.h, bissd_forward).  ``rev_block``
    > 0 restarts the reverse scan at the end of every block of that many
    tokens (the block-segmented reverse of full-block training)."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    shape = shape_of(x, fwd.B, chunk, rev_block)
    if y is None:
        y = torch.empty_like(x)
    ws, nws = _workspace(shape, _abi.OP_FORWARD, x.device, workspace)
    st = lib.bissd_forward(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                           _ptr(init_state), _ptr(y), _ptr(final_state), _ptr(ws),
                           C.c_size_t(nws), _stream(x.device, stream))
    _abi.check("bissd_forward", st)
    return y


def bissd_forward_phase(phase: int, x: torch.Tensor, fwd, rev, D: torch.Tensor, *,
                        chunk: int = 256, rev_block: int = 0, y: torch.Tensor,
                        workspace: torch.Tensor, init_state: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue one phase of bissd_forward (0 chunk states, 3 Gram tiles, 1 carry pass,
    2 output) for timing single kernels (include/bissd.h)."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    shape = shape_of(x, fwd.B, chunk, rev_block)
    st = lib.bissd_forward_phase(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                                 _ptr(init_state), _ptr(y), _ptr(final_state), _ptr(workspace),
                                 C.c_size_t(workspace.numel() * workspace.element_size()),
                                 _stream(x.device, stream), int(phase))
    _abi.check("bissd_forward_phase", st)


def bissd_block_update(state_in: torch.Tensor, x_blk: torch.Tensor, fwd, rev,
                       D: torch.Tensor, *, chunk: Optional[int] = None,
                       y_blk: Optional[torch.Tensor] = None,
                       state_out: Optional[torch.Tensor] = None, commit: bool = True,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Block update with a cached forward prefix state (include/bissd.h,
    bissd_block_update).  Returns (y_blk, state_out); state_out is None when
    ``commit`` is false and none was given."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    L = x_blk.shape[1]
    if chunk is None:
        chunk = 64 if L <= 64 else (128 if L <= 128 else 256)
    shape = shape_of(x_blk, fwd.B, chunk)
    if y_blk is None:
        y_blk = torch.empty_like(x_blk)
    if state_out is None and commit:
        state_out = torch.empty_like(state_in)
    ws, nws = _workspace(shape, _abi.OP_BLOCK, x_blk.device, workspace)
    st = lib.bissd_block_update(C.byref(shape), _ptr(state_in), _ptr(x_blk), _dir(fwd),
                                _dir(rev), _ptr(D), _ptr(y_blk), _ptr(state_out), _ptr(ws),
                                C.c_size_t(nws), _stream(x_blk.device, stream))
    _abi.check("bissd_block_update", st)
    return y_blk, state_out


GRAD_KEYS = ("dx", "ddt_f", "dA_f", "dB_f", "dC_f", "ddt_r", "dA_r", "dB_r", "dC_r", "dD")


def bissd_backward(x: torch.Tensor, fwd, rev, D: torch.Tensor, dy: torch.Tensor, *,
                   chunk: int = 256, rev_block: int = 0,
                   init_state: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of sum(dy * y) (include/bissd.h, bissd_backward).  Returns a
    dict with dx, ddt_f, dA_f, dB_f, dC_f, ddt_r, dA_r, dB_r, dC_r, dD (fp32),
    plus ddt_bias_<d> for a direction with a dt bias; ``grads`` may hold
    preallocated tensors under those keys.  ``rev_block`` as in bissd_forward."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    shape = shape_of(x, fwd.B, chunk, rev_block)
    f32 = dict(dtype=torch.float32, device=x.device)
    g = dict(grads) if grads is not None else {}
    if "dx" not in g:
        g["dx"] = torch.empty(x.shape, **f32)
    if "dD" not in g:
        g["dD"] = torch.empty(D.shape, **f32)
    for d, p in (("f", fwd), ("r", rev)):
        for k, like in (("ddt", p.dt), ("dA", p.A), ("dB", p.B), ("dC", p.C)):
            if f"{k}_{d}" not in g:
                g[f"{k}_{d}"] = torch.empty(like.shape, **f32)
        if p.dt_bias is not None and f"ddt_bias_{d}" not in g:
            g[f"ddt_bias_{d}"] = torch.empty(p.dt_bias.shape, **f32)
    for k in GRAD_KEYS:
        if g[k].dtype != torch.float32:
            raise TypeError(f"{k} must be float32")
    gf = _abi.Grad(_ptr(g["ddt_f"]), _ptr(g["dA_f"]), _ptr(g["dB_f"]), _ptr(g["dC_f"]),
                   _ptr(g.get("ddt_bias_f")))
    gr = _abi.Grad(_ptr(g["ddt_r"]), _ptr(g["dA_r"]), _ptr(g["dB_r"]), _ptr(g["dC_r"]),
                   _ptr(g.get("ddt_bias_r")))
    ws, nws = _workspace(shape, _abi.OP_BACKWARD, x.device, workspace)
    st = lib.bissd_backward(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                            _ptr(init_state), _ptr(dy), _ptr(g["dx"]), gf, gr, _ptr(g["dD"]),
                            _ptr(ws), C.c_size_t(nws), _stream(x.device, stream))
    _abi.check("bissd_backward", st)
    return g


def _attn_shape(q, k, v, block):
    Z, L, H, Dh = q.shape
    if k.shape != q.shape or v.shape != q.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k and v must have one shape and dtype")
    return _abi.AttnShape(Z, L, H, Dh, int(block), _dtype_code(q), 0)


def bissd_attention_forward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *,
                            block: int = 0, scale: float = 0.0,
                            o: Optional[torch.Tensor] = None,
                            lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """O = softmax(scale Q K^T + M) V per head (include/bissd.h,
    bissd_attention_forward): q, k, v [Z, L, H, 64]; block 0 for full
    bidirectional attention, > 0 for block-wise; scale 0 for 1/sqrt(64).
    ``lse`` (fp32 [Z, H, L]) receives what the backward needs."""
    lib = _abi.load()
    shape = _attn_shape(q, k, v, block)
    if o is None:
        o = torch.empty_like(q)
    st = lib.bissd_attention_forward(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), float(scale),
                                     _ptr(o), _ptr(lse), _stream(q.device, stream))
    _abi.check("bissd_attention_forward", st)
    return o


def bissd_attention_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                             o: torch.Tensor, dout: torch.Tensor, lse: torch.Tensor, *,
                             block: int = 0, scale: float = 0.0,
                             workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """dq, dk, dv (fp32) of sum(dout * o) for o, lse from bissd_attention_forward
    with the same arguments (include/bissd.h, bissd_attention_backward)."""
    lib = _abi.load()
    shape = _attn_shape(q, k, v, block)
    g = {n: torch.empty(q.shape, dtype=torch.float32, device=q.device) for n in ("dq", "dk", "dv")}
    if workspace is None:
        n = int(lib.bissd_attention_workspace_size(C.byref(shape)))
        workspace = torch.empty(max(n, 256), dtype=torch.uint8, device=q.device)
    st = lib.bissd_attention_backward(C.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                      _ptr(dout), _ptr(lse), float(scale), _ptr(g["dq"]),
                                      _ptr(g["dk"]), _ptr(g["dv"]), _ptr(workspace),
                                      workspace.numel() * workspace.element_size(),
                                      _stream(q.device, stream))
    _abi.check("bissd_attention_backward", st)
    return g
