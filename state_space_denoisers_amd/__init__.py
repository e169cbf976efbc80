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
dt_max); one with ``conv_w`` ([H, P, K] fp32 taps, ``conv_b`` [H, P] fp32,
``conv_act`` SiLU) makes that direction's scan read its causal (forward) or
anti-causal (reverse) depthwise convolution of x (include/bissd.h).
"""
from __future__ import annotations

import ctypes as C
from typing import NamedTuple, Optional

import torch

from . import _abi

__all__ = ["Dir", "bissd_forward", "bissd_forward_noalloc", "bissd_forward_phase", "bissd_block_update", "bissd_backward",
           "bissd_attention_forward", "bissd_attention_backward", "bissd_workspace_size",
           "bissd_timer_arm", "bissd_timer_read", "shape_of", "library_path", "BissdError"]

BissdError = _abi.BissdError


class Dir(NamedTuple):
    dt: torch.Tensor
    A: torch.Tensor
    B: torch.Tensor
    C: torch.Tensor
    dt_bias: Optional[torch.Tensor] = None
    dt_min: float = 0.0
    dt_max: float = float("inf")
    conv_w: Optional[torch.Tensor] = None
    conv_b: Optional[torch.Tensor] = None
    conv_act: bool = True


def library_path() -> str:
    return _abi.LIB_PATH


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return _abi.BISSD_BF16
    if t.dtype == torch.float32:
        return _abi.BISSD_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


_SHAPES: dict = {}


def shape_of(x: torch.Tensor, B: torch.Tensor, chunk: int, rev_block: int = 0,
             conv_width: int = 0, flags: int = 0) -> _abi.Shape:
    """The ABI shape struct for x / B (memoised: block updates call this in
    tight loops, and the C side only reads it)."""
    key = (x.shape, B.shape, x.dtype, chunk, rev_block, conv_width, flags)
    s = _SHAPES.get(key)
    if s is None:
        Z, L, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        s = _abi.Shape(Z, L, H, P, N, G, int(chunk), _dtype_code(x), int(rev_block),
                       int(conv_width), int(flags))
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


# ------------------------------------------------------------ validation
#
# The C library sizes every buffer from x's dtype and from the shapes of x
# and B, so a tensor of another dtype, shape or device would be read or
# written past its end.  Every entry point below checks its tensors first:
# shapes and dtypes, then that every tensor lives on x's GPU.  Nothing is
# launched when a check fails.

def _need(t, name: str, shape, dtype) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _on_device(named: dict, device: torch.device) -> None:
    """Every given tensor is a CUDA (HIP) tensor on `device`."""
    if device.type != "cuda":
        raise ValueError(f"x must be a GPU tensor, got device {device}")
    for name, t in named.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} is on {t.device}, expected {device} (the device of x)")


def _scan_dims(x: torch.Tensor, B: torch.Tensor):
    if not isinstance(x, torch.Tensor) or x.dim() != 4:
        raise ValueError("x must be a 4-D tensor [Z, L, H, P]")
    _dtype_code(x)
    if not isinstance(B, torch.Tensor) or B.dim() != 4:
        raise ValueError("B must be a 4-D tensor [Z, L, G, N]")
    Z, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    if G <= 0 or H % G != 0:
        raise ValueError(f"nheads ({H}) must be a multiple of ngroups ({G})")
    return Z, L, H, P, G, N


def _check_dir(d: "Dir", tag: str, x: torch.Tensor, G: int, N: int, named: dict) -> None:
    Z, L, H, _ = x.shape
    _need(d.dt, f"{tag}.dt", (Z, L, H), x.dtype)
    _need(d.A, f"{tag}.A", (H,), torch.float32)
    _need(d.B, f"{tag}.B", (Z, L, G, N), x.dtype)
    _need(d.C, f"{tag}.C", (Z, L, G, N), x.dtype)
    if d.dt_bias is not None:
        _need(d.dt_bias, f"{tag}.dt_bias", (H,), torch.float32)
    P = x.shape[3]
    if d.conv_w is not None:
        if not isinstance(d.conv_w, torch.Tensor) or d.conv_w.dim() != 3 or not 1 <= d.conv_w.shape[2] <= 4:
            raise ValueError(f"{tag}.conv_w must be [H, P, K] with 1 <= K <= 4")
        _need(d.conv_w, f"{tag}.conv_w", (H, P, d.conv_w.shape[2]), torch.float32)
        if d.conv_b is not None:
            _need(d.conv_b, f"{tag}.conv_b", (H, P), torch.float32)
    elif d.conv_b is not None:
        raise ValueError(f"{tag}.conv_b given without conv_w")
    for k in ("dt", "A", "B", "C", "dt_bias", "conv_w", "conv_b"):
        named[f"{tag}.{k}"] = getattr(d, k)


def _check_scan(x, fwd: "Dir", rev: "Dir", D, *, states=(), acts=(), outs=()) -> dict:
    """Validate the tensors of one scan call; returns them by name.
    states: (name, tensor) pairs of [Z, H, P, N] fp32 states (None allowed);
    acts: (name, tensor) pairs shaped and typed like x; outs: (name, tensor,
    shape, dtype) of caller-given outputs (None allowed)."""
    Z, L, H, P, G, N = _scan_dims(x, fwd.B)
    named = {"x": x}
    _check_dir(fwd, "fwd", x, G, N, named)
    _check_dir(rev, "rev", x, G, N, named)
    _need(D, "D", (H,), torch.float32)
    named["D"] = D
    for name, t in states:
        if t is not None:
            _need(t, name, (Z, H, P, N), torch.float32)
            named[name] = t
    for name, t in acts:
        if t is not None:
            _need(t, name, tuple(x.shape), x.dtype)
            named[name] = t
    for name, t, shp, dt in outs:
        if t is not None:
            _need(t, name, shp, dt)
            named[name] = t
    _on_device(named, x.device)
    return named


def _check_workspace(ws, device) -> None:
    if ws is None:
        return
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor")
    if ws.device != device:
        raise ValueError(f"workspace is on {ws.device}, expected {device}")


def _dir(d) -> _abi.Dir:
    d = Dir(*d)
    if d.A.dtype != torch.float32:
        raise TypeError(f"A must be torch.float32, got {d.A.dtype}")
    if d.dt_bias is not None and d.dt_bias.dtype != torch.float32:
        raise TypeError(f"dt_bias must be torch.float32, got {d.dt_bias.dtype}")
    act = int(bool(d.conv_act)) if d.conv_w is not None else 0
    return _abi.Dir(_ptr(d.dt), _ptr(d.A), _ptr(d.B), _ptr(d.C), _ptr(d.dt_bias),
                    float(d.dt_min), float(d.dt_max), _ptr(d.conv_w), _ptr(d.conv_b), act, 0)


def _conv_width(fwd: "Dir", rev: "Dir") -> int:
    """The convolution width the directions' taps share (0: none)."""
    ks = {d.conv_w.shape[-1] for d in (fwd, rev) if d.conv_w is not None}
    if len(ks) > 1:
        raise ValueError(f"the directions' convolutions must have one width, got {sorted(ks)}")
    return ks.pop() if ks else 0


def _stream(device: torch.device, stream) -> C.c_void_p:
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return C.c_void_p(s.cuda_stream)


def bissd_workspace_size(shape: _abi.Shape, op: int) -> int:
    return int(_abi.load().bissd_workspace_size(C.byref(shape), int(op)))


def _workspace(shape, op, device, workspace):
    """The caller's workspace, or a new one (allocated on the stream the call
    runs on: see _on_stream)."""
    if workspace is not None:
        _check_workspace(workspace, device)
        return workspace, workspace.numel() * workspace.element_size()
    n = bissd_workspace_size(shape, op)
    ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)
    return ws, ws.numel()


def _on_stream(device: torch.device, stream):
    """Context under which a call allocates its outputs and workspace: the
    caller's stream when one is given, so that torch's caching allocator
    does not hand that memory to work on another stream while the library's
    kernels still use it."""
    import contextlib
    if stream is None:
        return contextlib.nullcontext()
    return torch.cuda.stream(stream)


def bissd_forward(x: torch.Tensor, fwd, rev, D: torch.Tensor, *, chunk: int = 256,
                  rev_block: int = 0, init_state: Optional[torch.Tensor] = None,
                  y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None, save: bool = False, stream=None):
    """y = yf + yr + D x (see include/bissd.h, bissd_forward).  ``rev_block``
    > 0 restarts the reverse scan at the end of every block of that many
    tokens (the block-segmented reverse of full-block training).  With
    ``save`` (the forward of a training step) it returns ``(y, saved)``:
    ``saved`` is the workspace holding what ``bissd_backward(..., saved=saved)``
    of the same inputs reads instead of recomputing (BISSD_SAVE)."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    _check_scan(x, fwd, rev, D, states=(("init_state", init_state), ("final_state", final_state)),
                acts=(("y", y),))
    shape = shape_of(x, fwd.B, chunk, rev_block, _conv_width(fwd, rev), _abi.SAVE if save else 0)
    with _on_stream(x.device, stream):
        if y is None:
            y = torch.empty_like(x)
        ws, nws = _workspace(shape, _abi.OP_FORWARD, x.device, workspace)
    st = lib.bissd_forward(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                           _ptr(init_state), _ptr(y), _ptr(final_state), _ptr(ws),
                           C.c_size_t(nws), _stream(x.device, stream))
    _abi.check("bissd_forward", st)
    return (y, ws) if save else y


def bissd_forward_noalloc(x: torch.Tensor, fwd, rev, D: torch.Tensor, *, y: torch.Tensor,
                          chunk: int = 256, rev_block: int = 0,
                          init_state: Optional[torch.Tensor] = None,
                          final_state: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """bissd_forward with the library's static scratch array as workspace
    (include/bissd.h, bissd_forward_noalloc): nothing is allocated, so the
    caller passes y.  Shapes whose workspace exceeds the array
    (BISSD_NOALLOC_SCRATCH_BYTES) raise BissdError (BISSD_ERR_SCRATCH)."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    _check_scan(x, fwd, rev, D, states=(("init_state", init_state), ("final_state", final_state)),
                acts=(("y", y),))
    if y is None:
        raise ValueError("y is required")
    shape = shape_of(x, fwd.B, chunk, rev_block, _conv_width(fwd, rev))
    st = lib.bissd_forward_noalloc(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                                   _ptr(init_state), _ptr(y), _ptr(final_state),
                                   _stream(x.device, stream))
    _abi.check("bissd_forward_noalloc", st)
    return y


def bissd_forward_phase(phase: int, x: torch.Tensor, fwd, rev, D: torch.Tensor, *,
                        chunk: int = 256, rev_block: int = 0, y: torch.Tensor,
                        workspace: torch.Tensor, init_state: Optional[torch.Tensor] = None,
                        final_state: Optional[torch.Tensor] = None, stream=None) -> None:
    """Enqueue one phase of bissd_forward (0 chunk states, 3 Gram tiles, 1 carry pass,
    2 output) for timing single kernels (include/bissd.h)."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    _check_scan(x, fwd, rev, D, states=(("init_state", init_state), ("final_state", final_state)),
                acts=(("y", y),))
    _check_workspace(workspace, x.device)
    shape = shape_of(x, fwd.B, chunk, rev_block, _conv_width(fwd, rev))
    st = lib.bissd_forward_phase(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                                 _ptr(init_state), _ptr(y), _ptr(final_state), _ptr(workspace),
                                 C.c_size_t(workspace.numel() * workspace.element_size()),
                                 _stream(x.device, stream), int(phase))
    _abi.check("bissd_forward_phase", st)


def bissd_block_update(state_in: torch.Tensor, x_blk: torch.Tensor, fwd, rev,
                       D: torch.Tensor, *, chunk: Optional[int] = None,
                       y_blk: Optional[torch.Tensor] = None,
                       state_out: Optional[torch.Tensor] = None, commit: bool = True,
                       conv_state: Optional[torch.Tensor] = None,
                       conv_state_out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None, stream=None):
    """Block update with a cached forward prefix state (include/bissd.h,
    bissd_block_update).  Returns (y_blk, state_out); state_out is None when
    ``commit`` is false and none was given.  With the directions'
    convolutions (width K), ``conv_state`` [Z, K-1, H, P] holds the last K-1
    x rows before the block (None: zeros) and ``conv_state_out`` (may be
    ``conv_state``) receives the last K-1 rows of [conv_state | x_blk]."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    K = _conv_width(fwd, rev)
    cst = (K - 1, x_blk.shape[2], x_blk.shape[3]) if K > 1 else None
    outs = ()
    if cst is not None:
        outs = tuple((n, t, (x_blk.shape[0],) + cst, x_blk.dtype)
                     for n, t in (("conv_state", conv_state), ("conv_state_out", conv_state_out)))
    elif conv_state is not None or conv_state_out is not None:
        raise ValueError("conv states need directions with a convolution wider than one tap")
    _check_scan(x_blk, fwd, rev, D, states=(("state_in", state_in), ("state_out", state_out)),
                acts=(("y_blk", y_blk),), outs=outs)
    L = x_blk.shape[1]
    if chunk is None:
        chunk = 64 if L <= 64 else (128 if L <= 128 else 256)
    shape = shape_of(x_blk, fwd.B, chunk, 0, K)
    with _on_stream(x_blk.device, stream):
        if y_blk is None:
            y_blk = torch.empty_like(x_blk)
        if state_out is None and commit:
            state_out = torch.empty_like(state_in)
        ws, nws = _workspace(shape, _abi.OP_BLOCK, x_blk.device, workspace)
    st = lib.bissd_block_update(C.byref(shape), _ptr(state_in), _ptr(x_blk), _dir(fwd),
                                _dir(rev), _ptr(D), _ptr(y_blk), _ptr(state_out),
                                _ptr(conv_state), _ptr(conv_state_out), _ptr(ws),
                                C.c_size_t(nws), _stream(x_blk.device, stream))
    _abi.check("bissd_block_update", st)
    return y_blk, state_out


GRAD_KEYS = ("dx", "ddt_f", "dA_f", "dB_f", "dC_f", "ddt_r", "dA_r", "dB_r", "dC_r", "dD")


def bissd_backward(x: torch.Tensor, fwd, rev, D: torch.Tensor, dy: torch.Tensor, *,
                   chunk: int = 256, rev_block: int = 0,
                   init_state: Optional[torch.Tensor] = None, grads: Optional[dict] = None,
                   workspace: Optional[torch.Tensor] = None,
                   saved: Optional[torch.Tensor] = None, stream=None) -> dict:
    """Gradients of sum(dy * y) (include/bissd.h, bissd_backward).  Returns a
    dict with dx, ddt_f, dA_f, dB_f, dC_f, ddt_r, dA_r, dB_r, dC_r, dD (fp32),
    plus ddt_bias_<d> for a direction with a dt bias; ``grads`` may hold
    preallocated tensors under those keys.  ``rev_block`` as in bissd_forward.
    ``saved``: the second result of ``bissd_forward(..., save=True)`` with the
    same inputs, used as the workspace (BISSD_SAVE); it is consumed."""
    lib = _abi.load()
    fwd, rev = Dir(*fwd), Dir(*rev)
    g = dict(grads) if grads is not None else {}
    Z, L, H, P, G, N = _scan_dims(x, fwd.B)
    gshape = {"dx": (Z, L, H, P), "dD": (H,)}
    for d, p in (("f", fwd), ("r", rev)):
        gshape.update({f"ddt_{d}": (Z, L, H), f"dA_{d}": (H,), f"dB_{d}": (Z, L, G, N),
                       f"dC_{d}": (Z, L, G, N)})
        if p.dt_bias is not None:
            gshape[f"ddt_bias_{d}"] = (H,)
    unknown = set(g) - set(gshape)
    if unknown:
        raise ValueError(f"unexpected gradient buffers {sorted(unknown)}")
    _check_scan(x, fwd, rev, D, states=(("init_state", init_state),), acts=(("dy", dy),),
                outs=tuple((k, g.get(k), shp, torch.float32) for k, shp in gshape.items()))
    if dy is None:
        raise ValueError("dy is required")
    if saved is not None and workspace is not None:
        raise ValueError("pass saved or workspace, not both")
    shape = shape_of(x, fwd.B, chunk, rev_block, _conv_width(fwd, rev),
                     _abi.SAVE if saved is not None else 0)
    if saved is not None:
        workspace = saved
    with _on_stream(x.device, stream):
        for k, shp in gshape.items():
            if k not in g:
                g[k] = torch.empty(shp, dtype=torch.float32, device=x.device)
    gf = _abi.Grad(_ptr(g["ddt_f"]), _ptr(g["dA_f"]), _ptr(g["dB_f"]), _ptr(g["dC_f"]),
                   _ptr(g.get("ddt_bias_f")))
    gr = _abi.Grad(_ptr(g["ddt_r"]), _ptr(g["dA_r"]), _ptr(g["dB_r"]), _ptr(g["dC_r"]),
                   _ptr(g.get("ddt_bias_r")))
    with _on_stream(x.device, stream):
        ws, nws = _workspace(shape, _abi.OP_BACKWARD, x.device, workspace)
    st = lib.bissd_backward(C.byref(shape), _ptr(x), _dir(fwd), _dir(rev), _ptr(D),
                            _ptr(init_state), _ptr(dy), _ptr(g["dx"]), gf, gr, _ptr(g["dD"]),
                            _ptr(ws), C.c_size_t(nws), _stream(x.device, stream))
    _abi.check("bissd_backward", st)
    return g


def _attn_shape(q, k, v, block, **more):
    """ABI shape of q, k, v [Z, L, H, 64] after checking them and the further
    tensors in `more` (name -> (tensor or None, shape, dtype))."""
    if not isinstance(q, torch.Tensor) or q.dim() != 4:
        raise ValueError("q must be a 4-D tensor [Z, L, H, 64]")
    _dtype_code(q)
    Z, L, H, Dh = q.shape
    named = {"q": q}
    for name, t in (("k", k), ("v", v)):
        _need(t, name, tuple(q.shape), q.dtype)
        named[name] = t
    for name, (t, shp, dt) in more.items():
        if t is not None:
            _need(t, name, shp, dt)
            named[name] = t
    _on_device(named, q.device)
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
    Z, L, H = q.shape[0], q.shape[1], q.shape[2]
    shape = _attn_shape(q, k, v, block, o=(o, tuple(q.shape), q.dtype),
                        lse=(lse, (Z, H, L), torch.float32))
    with _on_stream(q.device, stream):
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
    Z, L, H = q.shape[0], q.shape[1], q.shape[2]
    if o is None or dout is None or lse is None:
        raise ValueError("o, dout and lse are required")
    shape = _attn_shape(q, k, v, block, o=(o, tuple(q.shape), q.dtype),
                        dout=(dout, tuple(q.shape), q.dtype), lse=(lse, (Z, H, L), torch.float32))
    _check_workspace(workspace, q.device)
    with _on_stream(q.device, stream):
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


TIMER_SLOTS = 4096


def bissd_timer_arm(slot: int) -> None:
    """Hand timer slot ``slot`` to the library's next kernel launch, which
    records its dispatch start and end in the slot's events; -1 disarms
    (include/bissd.h, bissd_timer_arm)."""
    _abi.check("bissd_timer_arm", _abi.load().bissd_timer_arm(int(slot)))


def bissd_timer_read(slot: int) -> float:
    """Duration in ms of the kernel launch that took timer slot ``slot``
    (waits for it; include/bissd.h, bissd_timer_read)."""
    ms = C.c_float(0.0)
    _abi.check("bissd_timer_read", _abi.load().bissd_timer_read(int(slot), C.byref(ms)))
    return float(ms.value)
