"""Seeded synthetic inputs for the bidirectional SSD (Mamba-2) scan.

The pages describe bidirectional Mamba-2 denoisers at the 130M scale (hidden
768 -> d_inner 1536 = 24 heads x head dim 64), trained at sequence length 1024
and evaluated for long-context throughput up to 65K-262K tokens, plus a
block-diffusion variant whose active block carries mask tokens.  None of their
datasets or weights is available, so every tensor here is drawn from a fixed,
seeded distribution with those shapes:

* x ~ N(0, 1); B, C ~ N(0, 1) / sqrt(d_state)
* dt = clamp(softplus(N(0, 1) - shift), 1e-3, 0.1), shift 4 (5 for long context)
* A_h = -exp(U(0, ln 16)); D_h ~ N(0, 1)
* the reverse direction draws its own dt / A / B / C from independent streams.

Each tensor is drawn in float64 and rounded once, round-to-nearest-even, to the
workload's dtype (fp32 or bf16); A and D are always fp32.  The arrays returned
hold exactly those rounded values (as float64), so the CPU oracle and the GPU
path read identical numbers.

This module draws random numbers and rounds them.  It computes no part of the
scan and is shared by the oracle's tests and by the GPU path's tests and bench.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

# Named sub-stream keys: each tensor has its own independent stream.
_KEYS = {
    "x": 0, "D": 1, "dt_f": 2, "A_f": 3, "B_f": 4, "C_f": 5,
    "dt_r": 6, "A_r": 7, "B_r": 8, "C_r": 9, "dy": 10,
    "mask_pos": 11, "mask_vec": 12, "prefix": 13,
    "attn_q": 14, "attn_k": 15, "attn_v": 16,
    "dtraw_f": 17, "dtraw_r": 18, "dtbias_f": 19, "dtbias_r": 20,
    "convw_f": 21, "convw_r": 22, "convb_f": 23, "convb_r": 24, "convstate": 25,
}


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""
    name: str
    Z: int            # batch
    L: int            # sequence length (block length for block updates)
    H: int            # heads
    P: int            # head dim
    N: int            # state dim (d_state)
    G: int            # B/C groups
    chunk: int        # chunk length of the chunked evaluation
    dtype: str        # "fp32" or "bf16": dtype of x, dt, B, C, y, dy
    dt_shift: float = 4.0
    seed: int = 0
    prefix_len: int = 0       # block update: tokens before the active block
    mask_count: int = 0       # block update: masked positions per batch row
    mask_std: float = 0.1     # block update: std of the shared mask embedding

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def tokens(self) -> int:
        return self.Z * self.L


# The five workloads: a tiny fp32 correctness case, the 130M-class layer at
# L=1K, the long-context L=65K scan, the block-diffusion update and the
# training step (forward + backward).
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", Z=1, L=128, H=4, P=64, N=64, G=1,
                          chunk=64, dtype="fp32", seed=1000),
    "layer130m_L1k": Workload("layer130m_L1k", Z=8, L=1024, H=24, P=64, N=128,
                              G=1, chunk=256, dtype="bf16", seed=1001),
    "long_L65k": Workload("long_L65k", Z=1, L=65536, H=24, P=64, N=128, G=1,
                          chunk=256, dtype="bf16", dt_shift=5.0, seed=1002),
    "block_update": Workload("block_update", Z=4, L=64, H=24, P=64, N=128,
                             G=1, chunk=64, dtype="bf16", seed=1003,
                             prefix_len=262144, mask_count=16),
    "train_L2k": Workload("train_L2k", Z=16, L=2048, H=24, P=64, N=128, G=1,
                          chunk=256, dtype="bf16", seed=1004),
}


def _rng(seed: int, key: str, extra: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), _KEYS[key], int(extra)])))


def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even).

    bfloat16 keeps 8 significant bits; frexp gives a = m * 2**e with
    0.5 <= |m| < 1, so m * 256 rounded to an integer keeps exactly 8 bits.
    """
    a = np.asarray(a, dtype=np.float64)
    m, e = np.frexp(a)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def round_fp32(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float32).astype(np.float64)


def quantize(a, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_bf16(a)
    if dtype == "fp32":
        return round_fp32(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def _softplus(z: np.ndarray) -> np.ndarray:
    # numerically safe log(1 + e^z)
    return np.where(z > 30.0, z, np.log1p(np.exp(np.minimum(z, 30.0))))


def draw_dt(rng: np.random.Generator, shape, shift: float) -> np.ndarray:
    z = rng.standard_normal(shape)
    return np.clip(_softplus(z - shift), 1e-3, 0.1)


def draw_A(rng: np.random.Generator, H: int) -> np.ndarray:
    return -np.exp(rng.uniform(0.0, math.log(16.0), size=H))


def make_inputs(w: Workload, mode: str = "full", with_dy: bool = False,
                seed: int | None = None) -> dict:
    """All inputs of one call of the bidirectional scan for workload ``w``.

    ``mode`` selects a check mode: "full" as configured, "scan" (D = 0),
    "fwd" (D = 0 and C_r = 0, so only the forward scan reaches y) or
    "rev" (D = 0 and C_f = 0).  Arrays are float64 holding values exactly
    representable in the workload dtype.
    """
    s = w.seed if seed is None else seed
    Z, L, H, P, N, G = w.Z, w.L, w.H, w.P, w.N, w.G
    q = lambda a: quantize(a, w.dtype)  # noqa: E731
    out = {}
    out["x"] = q(_rng(s, "x").standard_normal((Z, L, H, P)))
    for d in ("f", "r"):
        out[f"dt_{d}"] = q(draw_dt(_rng(s, f"dt_{d}"), (Z, L, H), w.dt_shift))
        out[f"A_{d}"] = round_fp32(draw_A(_rng(s, f"A_{d}"), H))
        scale = 1.0 / math.sqrt(N)
        out[f"B_{d}"] = q(_rng(s, f"B_{d}").standard_normal((Z, L, G, N)) * scale)
        out[f"C_{d}"] = q(_rng(s, f"C_{d}").standard_normal((Z, L, G, N)) * scale)
    out["D"] = round_fp32(_rng(s, "D").standard_normal(H))
    if w.mask_count:
        # One shared mask-token embedding sits at mask_count seeded positions
        # of every batch row.
        m = q(_rng(s, "mask_vec").standard_normal((H, P)) * w.mask_std)
        rp = _rng(s, "mask_pos")
        for b in range(Z):
            pos = rp.permutation(L)[: w.mask_count]
            out["x"][b, pos] = m
        out["mask_vec"] = m
    if with_dy:
        out["dy"] = q(_rng(s, "dy").standard_normal((Z, L, H, P)))
    apply_mode(out, mode)
    return out


def apply_mode(inp: dict, mode: str) -> dict:
    if mode == "full":
        return inp
    if mode not in ("scan", "fwd", "rev"):
        raise ValueError(f"unknown check mode {mode!r}")
    inp["D"] = np.zeros_like(inp["D"])
    if mode == "fwd":
        inp["C_r"] = np.zeros_like(inp["C_r"])
    elif mode == "rev":
        inp["C_f"] = np.zeros_like(inp["C_f"])
    return inp


def make_prefix(w: Workload, length: int, seed: int | None = None) -> dict:
    """Forward-direction inputs of a synthetic prefix preceding an active
    block: x, dt_f, B_f, C_f with the workload's distributions.  The layer
    parameters (A_f, D) are the block's own, drawn by ``make_inputs``."""
    s = w.seed if seed is None else seed
    Z, H, P, N, G = w.Z, w.H, w.P, w.N, w.G
    q = lambda a: quantize(a, w.dtype)  # noqa: E731
    r = _rng(s, "prefix", 1)
    scale = 1.0 / math.sqrt(N)
    return {
        "x": q(r.standard_normal((Z, length, H, P))),
        "dt_f": q(draw_dt(r, (Z, length, H), w.dt_shift)),
        "B_f": q(r.standard_normal((Z, length, G, N)) * scale),
        "C_f": q(r.standard_normal((Z, length, G, N)) * scale),
    }


def prefix_on_device(w: Workload, length: int, device, seed: int | None = None):
    """Large prefix drawn directly on the device with torch's seeded Philox
    generator (same distributions as ``make_prefix``, different stream).
    Used where the prefix is too long to draw on the host; returns torch
    tensors in the workload dtype."""
    import torch
    s = w.seed if seed is None else seed
    gen = torch.Generator(device=device)
    gen.manual_seed(s * 64 + _KEYS["prefix"])
    Z, H, P, N, G = w.Z, w.H, w.P, w.N, w.G
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    x = torch.randn((Z, length, H, P), generator=gen, device=device).to(tdt)
    z = torch.randn((Z, length, H), generator=gen, device=device)
    dt = torch.nn.functional.softplus(z - w.dt_shift).clamp_(1e-3, 0.1).to(tdt)
    scale = 1.0 / math.sqrt(N)
    B = (torch.randn((Z, length, G, N), generator=gen, device=device) * scale).to(tdt)
    C = (torch.randn((Z, length, G, N), generator=gen, device=device) * scale).to(tdt)
    return {"x": x, "dt_f": dt, "B_f": B, "C_f": C}


def as_torch(a: np.ndarray, dtype: str, device=None):
    """Move quantised float64 values to a torch tensor of ``dtype``
    ("fp32", "bf16" or "f32param"); exact because the values are
    representable."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    if device is not None:
        t = t.to(device)
    return t.contiguous()


def make_attention_inputs(Z: int, L: int, H: int, dtype: str, seed: int, D: int = 64) -> dict:
    """q, k, v [Z, L, H, D] ~ N(0, 1) for the hybrids' attention layers (the
    scale of normalised activations), rounded once to ``dtype``."""
    return {n: quantize(_rng(seed, "attn_" + n).standard_normal((Z, L, H, D)), dtype)
            for n in ("q", "k", "v")}


def with_dt_post(inp: dict, w: Workload, lo: float = 1e-3, hi: float = 0.1) -> dict:
    """The same inputs with each direction's dt given as the mixer's
    pre-activation for the library's dt post-processing: raw ~ N(0, 1)
    (rounded to the workload dtype), per-head bias ~ -shift + 0.5 N(0, 1)
    (fp32) and the clamp [lo, hi] -- the synthetic dt recipe with the
    softplus, shift and clamp moved into the scan."""
    out = dict(inp)
    Z, L, H = inp["dt_f"].shape
    for d in ("f", "r"):
        raw = quantize(_rng(w.seed, f"dtraw_{d}").standard_normal((Z, L, H)), w.dtype)
        bias = round_fp32(-w.dt_shift + 0.5 * _rng(w.seed, f"dtbias_{d}").standard_normal(H))
        out[f"dt_{d}"] = off_clamp_edges(raw, bias, lo, hi, w.dtype)
        out[f"dt_bias_{d}"] = bias
        out[f"dt_min_{d}"], out[f"dt_max_{d}"] = lo, hi
    return out


# Half-width of the band of pre-activations kept clear around each point
# where the clamp engages.
CLAMP_EDGE_BAND = 1e-4


def off_clamp_edges(raw, bias, lo: float, hi: float, dtype: str,
                    band: float = CLAMP_EDGE_BAND) -> np.ndarray:
    """Move every pre-activation raw + bias that lies within `band` of one of
    the two points where the clamp engages, z_lo = log(e^lo - 1) and
    z_hi = log(e^hi - 1), to the nearest value of `dtype` that is at least
    2 * band further away from that point.  Whether such a token sits inside
    the clamp range is decided by a rounding (it depends on the precision the
    step is formed in); everywhere else any precision decides alike."""
    raw = np.array(raw, dtype=np.float64)
    b = np.asarray(bias, np.float64)[None, None, :]
    for edge in (lo, hi):
        if not np.isfinite(edge) or edge <= 0.0:
            continue
        ze = math.log(math.expm1(edge))
        z = raw + b
        for idx in zip(*np.nonzero(np.abs(z - ze) < band)):
            sgn = 1.0 if z[idx] >= ze else -1.0
            step = 2.0 * band
            while True:
                cand = float(quantize(np.array([raw[idx] + sgn * step]), dtype)[0])
                if abs(cand + b[0, 0, idx[2]] - ze) >= 2.0 * band:
                    break
                step *= 2.0
            raw[idx] = cand
    return raw



def make_conv(w: Workload, K: int = 4, seed: int | None = None, dirs=("f", "r")) -> dict:
    """Taps and biases of the mixer's depthwise convolution per direction:
    conv_w_<d> [H, P, K] ~ U(-1/sqrt(K), 1/sqrt(K)) (the default init of a
    depthwise Conv1d with K taps per channel), conv_b_<d> [H, P] ~ the same,
    fp32."""
    s = w.seed if seed is None else seed
    bound = 1.0 / math.sqrt(K)
    out = {}
    for d in dirs:
        out[f"conv_w_{d}"] = round_fp32(_rng(s, f"convw_{d}").uniform(-bound, bound, (w.H, w.P, K)))
        out[f"conv_b_{d}"] = round_fp32(_rng(s, f"convb_{d}").uniform(-bound, bound, (w.H, w.P)))
    return out


def make_conv_state(w: Workload, K: int, seed: int | None = None) -> np.ndarray:
    """A conv state (the last K-1 x rows before a block), x's distribution,
    rounded to the workload dtype: [Z, K-1, H, P]."""
    s = w.seed if seed is None else seed
    return quantize(_rng(s, "convstate").standard_normal((w.Z, K - 1, w.H, w.P)), w.dtype)
