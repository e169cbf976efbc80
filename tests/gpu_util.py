"""Helpers for the GPU parity tests: move seeded inputs to the device, call
the HIP library through its C ABI binding, and compare with the oracle."""
from __future__ import annotations

import numpy as np
import torch

from synth import gen

ACT = ("x", "dt_f", "B_f", "C_f", "dt_r", "B_r", "C_r", "dy")
PARAM = ("A_f", "A_r", "D")
TOL = {"fp32": 1e-4, "bf16": 2e-2}


def device():
    return torch.device("cuda", 0)


def to_dev(inp: dict, dtype: str) -> dict:
    T = {}
    for k in ACT:
        if k in inp:
            T[k] = gen.as_torch(inp[k], dtype, device())
    for k in PARAM:
        T[k] = gen.as_torch(inp[k], "fp32", device())
    return T


def dirs(T: dict):
    return ((T["dt_f"], T["A_f"], T["B_f"], T["C_f"]),
            (T["dt_r"], T["A_r"], T["B_r"], T["C_r"]))


def f32_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device())


def host(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def maxrel(g, r) -> float:
    """max |g - r| / max |r| (fp64)."""
    g = np.asarray(g, np.float64)
    r = np.asarray(r, np.float64)
    m = float(np.max(np.abs(r)))
    return float(np.max(np.abs(g - r))) / (m if m > 0 else 1.0)


def gpu_forward(inp: dict, dtype: str, chunk: int, init_state=None, final=False):
    import state_space_denoisers_amd as ssd
    T = to_dev(inp, dtype)
    fwd, rev = dirs(T)
    Z, L, H, P = inp["x"].shape
    N = inp["B_f"].shape[-1]
    fs = torch.full((Z, H, P, N), float("nan"), device=device()) if final else None
    init = None if init_state is None else f32_dev(init_state)
    y = ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=chunk, init_state=init,
                          final_state=fs)
    torch.cuda.synchronize()
    return (host(y), host(fs)) if final else host(y)


def select_heads(inp: dict, heads) -> dict:
    """Sub-problem on a subset of heads (valid when every head reads group 0)."""
    hs = np.asarray(heads)
    out = {}
    for k, v in inp.items():
        if k in ("x", "dy"):
            out[k] = v[:, :, hs]
        elif k.startswith("dt"):
            out[k] = v[:, :, hs]
        elif k in PARAM:
            out[k] = v[hs]
        else:
            out[k] = v
    return out


def select_rows(inp: dict, rows) -> dict:
    rs = np.asarray(rows)
    return {k: (v if k in PARAM or k == "mask_vec" else v[rs]) for k, v in inp.items()}
