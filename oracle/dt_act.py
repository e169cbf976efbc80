"""Mamba-2's dt post-processing in front of the scan -- TEST INFRASTRUCTURE.

The bidirectional scan's per-direction step dt comes out of the mixer's
projection through a per-head bias, a softplus and a clamp ("DiffMamba
Checkpoints" model card, Model details, and "DiffuMamba: High-Throughput
Diffusion LMs with Mamba Backbone", Core Architecture, name Mamba-2 mixers;
this is the plain Mamba-2 form of their dt, the pages give no formula):

    dt[b, t, h] = clamp(softplus(raw[b, t, h] + bias[h]), lo, hi)

with softplus(z) = log(1 + e^z).  Its reverse mode for an incoming ddt:

    draw = ddt * sigmoid(z) * [lo <= softplus(z) <= hi],   dbias[h] = sum_{b,t} draw

(the clamp passes the gradient where the value lies inside [lo, hi], ends
included: there the clamp is the identity on its argument).  numpy float64
throughout; the forward value and the backward's pass/stop decision come
from the one helper `inside`, so the two always agree: the gradient passes
exactly where the clamped value is the softplus itself.  The scan stays in
ssd_oracle.c.
"""
from __future__ import annotations

import numpy as np


def softplus(z):
    return np.logaddexp(0.0, z)


def preact(raw, bias) -> np.ndarray:
    """z = raw + bias[h] in float64 (raw [Z, L, H], bias [H])."""
    return np.asarray(raw, np.float64) + np.asarray(bias, np.float64)[None, None, :]


def inside(z, lo: float, hi: float) -> np.ndarray:
    """Where the clamp is the identity: lo <= softplus(z) <= hi (fp64)."""
    sp = softplus(z)
    return (sp >= lo) & (sp <= hi)


def forward(raw, bias, lo: float, hi: float) -> np.ndarray:
    z = preact(raw, bias)
    sp = softplus(z)
    keep = inside(z, lo, hi)
    return np.where(keep, sp, np.where(sp < lo, lo, hi))


def backward(raw, bias, lo: float, hi: float, ddt):
    """(draw, dbias) for the gradient ddt with respect to the clamped dt."""
    z = preact(raw, bias)
    draw = np.asarray(ddt, np.float64) * (1.0 / (1.0 + np.exp(-z))) * inside(z, lo, hi)
    return draw, draw.sum(axis=(0, 1))


def has_act(inp: dict, d: str) -> bool:
    return inp.get(f"dt_bias_{d}") is not None


def limits(inp: dict, d: str):
    return float(inp.get(f"dt_min_{d}", 0.0)), float(inp.get(f"dt_max_{d}", np.inf))


def effective(inp: dict) -> dict:
    """The inputs with each direction's dt replaced by its post-processed
    value where that direction carries a bias."""
    out = dict(inp)
    for d in ("f", "r"):
        if has_act(inp, d):
            lo, hi = limits(inp, d)
            out[f"dt_{d}"] = forward(inp[f"dt_{d}"], inp[f"dt_bias_{d}"], lo, hi)
    return out
