"""Dense (materialised) form of the bidirectional SSD scan -- TEST INFRASTRUCTURE.

An independent second formulation used to pin the recurrence in
ssd_oracle.c.  Unrolling the per-direction recurrence
S_t = exp(dt_t A) S_{t-1} + dt_t x_t (outer) B_t,  y_t = S_t C_t  gives, per head, a
lower-triangular semiseparable matrix for the forward scan

    M_f[t, s] = dt_s (C_t . B_s) exp(A * sum_{k=s+1..t} dt_k)     (s <= t)

and, for the scan over the flipped sequence mapped back to natural order, an
upper-triangular one

    M_r[t, s] = dt'_s (C'_t . B'_s) exp(A' * sum_{k=t..s-1} dt'_k)  (s >= t)

so that y = (M_f + M_r) x + D x, plus exp(A * sum_{k<=t} dt_k) S0 C_t for a
forward start state S0.  Both directions count the diagonal (token t sees
itself in each scan), which is the literal reading of "forward plus
flipped-reverse" (DiffMamba Checkpoints, Model details; DiffuMamba Technical
Summary, Methodology / Core Architecture).

A block-segmented reverse scan (blocks of RB tokens, each its own reverse
scan: the full-block objective of "Training Hybrid Block Diffusion Language
Models with Partial Bidirectionality", Methodology) keeps only the entries of
M_r whose row and column fall in the same block:
M_r[t, s] = 0 unless floor(t / RB) = floor(s / RB).

Written with plain torch CPU float64 ops so that autograd gives exact
reference gradients of sum(dy * y) for the backward pins.  Sized for tiny
inputs only (L up to a few hundred).
"""
from __future__ import annotations

import numpy as np
import torch


def _t(a, requires_grad=False):
    t = torch.as_tensor(np.asarray(a, dtype=np.float64)).clone()
    t.requires_grad_(requires_grad)
    return t


def direction_matrices(dt_f, A_f, B_f, C_f, dt_r, A_r, B_r, C_r, rev_block=0):
    """M_f, M_r for one (batch row, head): dt [L], A scalar, B/C [L, N]."""
    L = dt_f.shape[0]
    idx = torch.arange(L)
    lower = idx[:, None] >= idx[None, :]   # s <= t
    upper = idx[:, None] <= idx[None, :]   # s >= t
    if rev_block:
        blk = idx // rev_block
        upper = upper & (blk[:, None] == blk[None, :])
    cf = torch.cumsum(dt_f, 0)             # sum_{k<=t}
    seg_f = cf[:, None] - cf[None, :]      # sum_{k=s+1..t}
    ef = torch.where(lower, A_f * seg_f, torch.full_like(seg_f, -torch.inf))
    Mf = (C_f @ B_f.T) * torch.exp(ef) * dt_f[None, :]
    xr = torch.cumsum(dt_r, 0) - dt_r      # sum_{k<s}
    seg_r = xr[None, :] - xr[:, None]      # sum_{k=t..s-1}
    er = torch.where(upper, A_r * seg_r, torch.full_like(seg_r, -torch.inf))
    Mr = (C_r @ B_r.T) * torch.exp(er) * dt_r[None, :]
    return Mf, Mr


def forward_torch(T: dict, init_state=None, rev_block=0):
    """y (and per-direction parts) from torch float64 tensors in the GPU
    library's layouts.  Differentiable.  A direction with "dt_bias_<d>" in T
    first maps its dt through clamp(softplus(dt + bias), lo, hi) (torch's own
    softplus and clamp)."""
    T = dict(T)
    for d in ("f", "r"):
        if T.get(f"dt_bias_{d}") is not None:
            z = T[f"dt_{d}"] + T[f"dt_bias_{d}"][None, None, :]
            T[f"dt_{d}"] = torch.clamp(torch.nn.functional.softplus(z, threshold=1e9),
                                       float(T.get(f"dt_min_{d}", 0.0)),
                                       float(T.get(f"dt_max_{d}", float("inf"))))
    x = T["x"]
    Z, L, H, P = x.shape
    G = T["B_f"].shape[2]
    ys, yfs, yrs = [], [], []
    for b in range(Z):
        yb, yfb, yrb = [], [], []
        for h in range(H):
            g = h * G // H
            Mf, Mr = direction_matrices(
                T["dt_f"][b, :, h], T["A_f"][h], T["B_f"][b, :, g], T["C_f"][b, :, g],
                T["dt_r"][b, :, h], T["A_r"][h], T["B_r"][b, :, g], T["C_r"][b, :, g],
                rev_block)
            xh = x[b, :, h]
            yf = Mf @ xh
            if init_state is not None:
                cf = torch.cumsum(T["dt_f"][b, :, h], 0)
                carry = torch.exp(T["A_f"][h] * cf)[:, None] * (T["C_f"][b, :, g] @ init_state[b, h].T)
                yf = yf + carry
            yr = Mr @ xh
            yb.append(yf + yr + T["D"][h] * xh)
            yfb.append(yf)
            yrb.append(yr)
        ys.append(torch.stack(yb, 1))
        yfs.append(torch.stack(yfb, 1))
        yrs.append(torch.stack(yrb, 1))
    return torch.stack(ys, 0), torch.stack(yfs, 0), torch.stack(yrs, 0)


KEYS = ("x", "dt_f", "A_f", "B_f", "C_f", "dt_r", "A_r", "B_r", "C_r", "D")


def forward(inp: dict, init_state=None, rev_block=0) -> dict:
    """numpy in, numpy out: y, y_f, y_r."""
    T = {k: _t(inp[k]) for k in KEYS}
    S0 = None if init_state is None else _t(init_state)
    with torch.no_grad():
        y, yf, yr = forward_torch(T, S0, rev_block)
    return {"y": y.numpy(), "y_f": yf.numpy(), "y_r": yr.numpy()}


def gradients(inp: dict, dy, init_state=None, rev_block=0) -> dict:
    """Reverse-mode gradients of sum(dy * y) by torch autograd on the dense
    form: dx, ddt_f, dA_f, dB_f, dC_f, ddt_r, dA_r, dB_r, dC_r, dD (and
    ddt_bias_<d> for a direction with a dt bias)."""
    keys = list(KEYS) + [f"dt_bias_{d}" for d in ("f", "r") if inp.get(f"dt_bias_{d}") is not None]
    T = {k: _t(inp[k], requires_grad=True) for k in keys}
    for d in ("f", "r"):
        for lim in ("dt_min", "dt_max"):
            if f"{lim}_{d}" in inp:
                T[f"{lim}_{d}"] = inp[f"{lim}_{d}"]
    S0 = None if init_state is None else _t(init_state)
    y, _, _ = forward_torch(T, S0, rev_block)
    loss = (y * _t(dy)).sum()
    loss.backward()
    out = {("d" + k): T[k].grad.numpy().copy() for k in keys}
    return out


def matrices(inp: dict, b: int, h: int):
    """(M_f, M_r) of one batch row and head, as numpy arrays."""
    G = inp["B_f"].shape[2]
    H = inp["x"].shape[2]
    g = h * G // H
    with torch.no_grad():
        Mf, Mr = direction_matrices(
            _t(inp["dt_f"][b, :, h]), _t(inp["A_f"][h]), _t(inp["B_f"][b, :, g]),
            _t(inp["C_f"][b, :, g]), _t(inp["dt_r"][b, :, h]), _t(inp["A_r"][h]),
            _t(inp["B_r"][b, :, g]), _t(inp["C_r"][b, :, g]))
    return Mf.numpy(), Mr.numpy()
