"""The mixer's causal depthwise convolution in front of the scan -- TEST
INFRASTRUCTURE.

Each direction of the bidirectional denoiser is a Mamba-2 layer ("DiffMamba
Checkpoints" model card, Model details: forward plus flipped-reverse Mamba-2
with weight-tied projections; "DiffuMamba: High-Throughput Diffusion LMs
with Mamba Backbone", Core Architecture), and a Mamba-2 layer passes its x
through a short causal depthwise convolution and a SiLU before the scan.
The pages give no formula; the plain reading (R21):

  forward   xc_f[t, c] = act(b_f[c] + sum_{k=0}^{K-1} w_f[c, k] x[t - (K-1) + k, c])
  reverse   xc_r[t, c] = act(b_r[c] + sum_{k=0}^{K-1} w_r[c, k] x[t + (K-1) - k, c])

with act = SiLU (z * sigmoid(z)) or the identity, channel c = (h, p), and x
the shared pre-convolution input (the tied in-projection's x).  The reverse
is the forward convolution of the flipped sequence, flipped back.  Outside
the sequence x reads as zero, except that a block update's forward
convolution continues from a conv state: the last K-1 raw x rows before the
block.  The reverse never reads past the end of its block (the end of the
sequence, or with a block-segmented reverse the end of the token's reverse
block).  Each direction's scan then runs on its own xc_d, and the skip is
D_h x on the raw x:  y = scan_f(xc_f) + scan_r(xc_r) + D x.

numpy float64; the scan itself stays in ssd_oracle.c (oracle.py).
"""
from __future__ import annotations

import numpy as np

from . import oracle as _O


def silu(z):
    return z / (1.0 + np.exp(-z))


def conv(x, w, b, direction: str, act: bool = True, state=None, rev_block: int = 0):
    """The convolution of x [Z, L, H, P] with taps w [H, P, K] (and bias b
    [H, P] or None) in `direction` ("f" or "r"), activated by SiLU if `act`.
    `state` [Z, K-1, H, P]: raw rows before x (forward only; default zeros).
    `rev_block` > 0: the reverse reads nothing past the end of each block of
    that many tokens."""
    x = np.asarray(x, np.float64)
    w = np.asarray(w, np.float64)
    Z, L, H, P = x.shape
    K = w.shape[-1]
    out = np.zeros_like(x) if b is None else np.broadcast_to(np.asarray(b, np.float64), x.shape).copy()
    if direction == "f":
        pad = np.zeros((Z, K - 1, H, P)) if state is None else np.asarray(state, np.float64)
        xp = np.concatenate([pad, x], axis=1)       # xp[j] = x[j - (K-1)]
        for k in range(K):
            out += w[None, None, :, :, k] * xp[:, k:k + L]
    else:
        ends = np.full(L, L) if rev_block <= 0 else np.minimum((np.arange(L) // rev_block + 1) * rev_block, L)
        for k in range(K):
            j = np.arange(L) + (K - 1) - k                # tap k reads x[t + K-1-k]
            ok = j < ends
            sh = np.zeros_like(x)
            sh[:, ok] = x[:, j[ok]]
            out += w[None, None, :, :, k] * sh
    return silu(out) if act else out


def next_state(x_blk, state, K: int):
    """The conv state after a block: the last K-1 raw rows of [state | x_blk]."""
    Z, L, H, P = np.asarray(x_blk).shape
    pad = np.zeros((Z, K - 1, H, P)) if state is None else np.asarray(state, np.float64)
    return np.concatenate([pad, np.asarray(x_blk, np.float64)], axis=1)[:, -(K - 1):] if K > 1 \
        else np.zeros((Z, 0, H, P))


def _dir_only(inp, d, xc):
    """Inputs whose scan output is direction d's alone, on input xc."""
    q = dict(inp)
    q["x"] = xc
    q["D"] = np.zeros_like(inp["D"])
    other = "r" if d == "f" else "f"
    q[f"C_{other}"] = np.zeros_like(inp[f"C_{other}"])
    return q


def forward(inp: dict, convs: dict, rev_block: int = 0, init_state=None):
    """y = scan_f(xc_f) + scan_r(xc_r) + D x.  `convs` maps "f" / "r" to
    (w, b, act) or None (that direction's scan reads x as given)."""
    x = np.asarray(inp["x"], np.float64)
    y = np.asarray(inp["D"], np.float64)[None, None, :, None] * x
    for d in ("f", "r"):
        cv = convs.get(d)
        xc = x if cv is None else conv(x, cv[0], cv[1], d, cv[2], rev_block=rev_block)
        kw = {"init_state": init_state} if (d == "f" and init_state is not None) else {}
        y = y + _O.forward(_dir_only(inp, d, xc), rev_block=rev_block, **kw)
    return y


def block_update(inp: dict, convs: dict, state_in, conv_state=None):
    """Block update with the directions' convolutions: the forward's continues
    from `conv_state` (zeros if None), the reverse's stays in the block.
    Returns (y_blk, state_out, conv_state_out)."""
    x = np.asarray(inp["x"], np.float64)
    y = np.asarray(inp["D"], np.float64)[None, None, :, None] * x
    so = None
    for d in ("f", "r"):
        cv = convs.get(d)
        if cv is None:
            xc = x
        else:
            xc = conv(x, cv[0], cv[1], d, cv[2], state=conv_state if d == "f" else None)
        yd, sd = _O.block_update(_dir_only(inp, d, xc), state_in)
        y = y + yd
        if d == "f":
            so = sd
    K = convs["f"][0].shape[-1] if convs.get("f") is not None else (
        convs["r"][0].shape[-1] if convs.get("r") is not None else 1)
    return y, so, next_state(x, conv_state, K)
