"""GPU parity of the fused dt post-processing (a direction's dt given as the
mixer's pre-activation with a per-head bias: the kernels read
clamp(softplus(dt + bias), lo, hi)) against the fp64 oracle, which applies the
same map before its scan: forward, block-segmented forward, block update and
backward (including the pre-activation and bias gradients).
Tolerance: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32), 2e-2 (bf16), on
every output; the bf16 bias gradients, sums over Z L tokens whose terms
cancel, are held to the error bound of such a sum (2e-2 times the sum of
the terms' magnitudes, per head), the fp32 ones to the plain bar.  The inputs keep every
pre-activation clear of the two points where the clamp engages (synth.gen's
off_clamp_edges), where the in-range decision would depend on the precision
the step is formed in.
"""
import math

import numpy as np
import pytest
import torch

import state_space_denoisers_amd as ssd
from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, f32_dev, host, maxrel, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS


def dirs_post(inp, T):
    out = []
    for d in ("f", "r"):
        b = gen.as_torch(inp[f"dt_bias_{d}"], "fp32", T["x"].device)
        out.append(ssd.Dir(T[f"dt_{d}"], T[f"A_{d}"], T[f"B_{d}"], T[f"C_{d}"], b,
                           inp[f"dt_min_{d}"], inp[f"dt_max_{d}"]))
    return out


@pytest.mark.parametrize("dtype,L,chunk,rb", [("fp32", 300, 64, 0), ("fp32", 1000, 256, 64),
                                              ("fp32", 777, 128, 256), ("bf16", 1000, 256, 0)])
def test_forward(dtype, L, chunk, rb):
    w = W["tiny_fp32"].replace(L=L, chunk=chunk, Z=2, H=6, N=128, dtype=dtype)
    inp = gen.with_dt_post(gen.make_inputs(w), w)
    T = to_dev(inp, dtype)
    f, r = dirs_post(inp, T)
    print("dtpost fwd", dtype, L, chunk, rb, flush=True)
    y = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=chunk, rev_block=rb)
    torch.cuda.synchronize()
    e = maxrel(host(y), O.forward(inp, rev_block=rb))
    print(f"err={e:.1e}", flush=True)
    assert e <= TOL[dtype]


@pytest.mark.parametrize("dtype,Lb", [("fp32", 64), ("bf16", 37), ("bf16", 200)])
def test_block_update(dtype, Lb):
    w = W["block_update"].replace(Z=2, L=Lb, H=6, dtype=dtype)
    inp = gen.with_dt_post(gen.make_inputs(w), w)
    S0 = gen.round_fp32(np.random.default_rng(5).standard_normal((2, 6, 64, 128)) * 0.05)
    T = to_dev(inp, dtype)
    f, r = dirs_post(inp, T)
    print("dtpost block", dtype, Lb, flush=True)
    y, so = ssd.bissd_block_update(f32_dev(S0), T["x"], f, r, T["D"])
    torch.cuda.synchronize()
    ry, rso = O.block_update(inp, S0)
    assert maxrel(host(y), ry) <= TOL[dtype]
    assert maxrel(host(so), rso) <= TOL[dtype]


@pytest.mark.parametrize("dtype,L,chunk,rb", [("fp32", 300, 64, 0), ("fp32", 700, 256, 128),
                                              ("bf16", 1000, 256, 0)])
def test_backward(dtype, L, chunk, rb):
    w = W["tiny_fp32"].replace(L=L, chunk=chunk, Z=2, H=6, N=128, dtype=dtype)
    inp = gen.with_dt_post(gen.make_inputs(w, with_dy=True), w)
    T = to_dev(inp, dtype)
    f, r = dirs_post(inp, T)
    print("dtpost bwd", dtype, L, chunk, rb, flush=True)
    g = ssd.bissd_backward(T["x"], f, r, T["D"], T["dy"], chunk=chunk, rev_block=rb)
    torch.cuda.synchronize()
    ref = O.backward(inp, inp["dy"], rev_block=rb)
    errs = {k: maxrel(host(g[k]), ref[k]) for k in ref}
    print(" ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    assert "ddt_bias_f" in errs and "ddt_bias_r" in errs
    for d in ("f", "r"):
        gb, graw = host(g[f"ddt_bias_{d}"]), host(g[f"ddt_{d}"])
        # the bias gradient is the fixed-order sum of the pre-activation ddt
        assert maxrel(gb, graw.sum(axis=(0, 1))) <= 1e-5
        if dtype == "bf16":
            # A sum over Z L tokens whose terms cancel: its bar is the forward
            # error bound of a sum, tol * sum_t |term_t| per head, where each
            # term (ddt of one token) is itself held to tol above.  fp32 holds
            # the bias gradient to the plain max-relative bar.
            scale = np.abs(ref[f"ddt_{d}"]).sum(axis=(0, 1))
            cond = scale / np.abs(ref[f"ddt_bias_{d}"]).max()
            print(f"ddt_bias_{d}: sum |terms| / max |sum| = {cond.max():.1f}", flush=True)
            assert np.all(np.abs(gb - ref[f"ddt_bias_{d}"]) <= TOL[dtype] * scale), d
            errs.pop(f"ddt_bias_{d}")
    bad = {k: v for k, v in errs.items() if v > TOL[dtype]}
    assert not bad, (bad, errs)


def test_unclamped_post_processing_equals_the_plain_scan():
    """softplus^{-1}(dt) - bias fed with a bias and no clamp gives the scan
    of dt itself (both on the GPU)."""
    w = W["tiny_fp32"].replace(L=500, chunk=128, Z=1)
    inp = gen.make_inputs(w)
    T = to_dev(inp, "fp32")
    post = []
    for d in ("f", "r"):
        b = np.random.default_rng(7).standard_normal(w.H)
        raw = np.log(np.expm1(inp[f"dt_{d}"])) - b[None, None, :]
        post.append(ssd.Dir(f32_dev(raw), T[f"A_{d}"], T[f"B_{d}"], T[f"C_{d}"], f32_dev(b),
                            0.0, math.inf))
    y1 = ssd.bissd_forward(T["x"], post[0], post[1], T["D"], chunk=128)
    y0 = ssd.bissd_forward(T["x"], (T["dt_f"], T["A_f"], T["B_f"], T["C_f"]),
                           (T["dt_r"], T["A_r"], T["B_r"], T["C_r"]), T["D"], chunk=128)
    torch.cuda.synchronize()
    assert maxrel(host(y1), host(y0)) <= 1e-5
