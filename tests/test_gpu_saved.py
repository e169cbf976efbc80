"""The training step's saved path (BISSD_SAVE): a forward call that keeps its
chunk states, carry-ins, decays and Gram tiles in the workspace, then a
backward that reads them instead of forming them again.

The saved backward must equal the recomputing backward bit for bit (the same
kernels form the same values in the same order), and the saving forward's y
must equal the plain forward's.  The recomputing backward is held to the fp64
oracle by the other backward tests; one case here checks the saved path
against the oracle directly too.  Cases cover both Gram-tile producers
(formed by the chunk-state kernel, or by the Gram kernel when the head tiles
are too few), a start state, the block-segmented reverse, dt post-processing
and groups.
"""
import numpy as np
import pytest
import torch

import state_space_denoisers_amd as ssd
from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, f32_dev, host, maxrel, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS
KEYS = ("dx", "ddt_f", "dA_f", "dB_f", "dC_f", "ddt_r", "dA_r", "dB_r", "dC_r", "dD")


def directions(inp, T, post):
    out = []
    for d in ("f", "r"):
        if post:
            b = gen.as_torch(inp[f"dt_bias_{d}"], "fp32", T["x"].device)
            out.append(ssd.Dir(T[f"dt_{d}"], T[f"A_{d}"], T[f"B_{d}"], T[f"C_{d}"], b,
                               inp[f"dt_min_{d}"], inp[f"dt_max_{d}"]))
        else:
            out.append(ssd.Dir(T[f"dt_{d}"], T[f"A_{d}"], T[f"B_{d}"], T[f"C_{d}"]))
    return out


def both_paths(inp, dtype, chunk, rb=0, init_state=None, post=False):
    """(plain y, plain grads, saving y, saved grads), all on the host."""
    T = to_dev(inp, dtype)
    f, r = directions(inp, T, post)
    init = None if init_state is None else f32_dev(init_state)
    kw = dict(chunk=chunk, rev_block=rb, init_state=init)
    y0 = ssd.bissd_forward(T["x"], f, r, T["D"], **kw)
    g0 = ssd.bissd_backward(T["x"], f, r, T["D"], T["dy"], **kw)
    y1, saved = ssd.bissd_forward(T["x"], f, r, T["D"], save=True, **kw)
    g1 = ssd.bissd_backward(T["x"], f, r, T["D"], T["dy"], saved=saved, **kw)
    torch.cuda.synchronize()
    return host(y0), {k: host(v) for k, v in g0.items()}, host(y1), {k: host(v) for k, v in g1.items()}


CASES = {
    # 6 heads: too few two-head tiles for the chunk-state kernel to form every
    # Gram pair, so the Gram kernel runs (in the forward and in the recompute)
    "bf16_gram_kernel": (W["train_L2k"].replace(Z=2, L=700, H=6), "bf16", 256, 0, False, False),
    # 24 heads: the chunk-state kernel forms the Gram tiles
    "bf16_gram_in_k1": (W["train_L2k"].replace(Z=2, L=2048), "bf16", 256, 0, False, False),
    "fp32_init_state": (W["tiny_fp32"].replace(L=200, Z=2), "fp32", 64, 0, True, False),
    "bf16_rev_block64": (W["train_L2k"].replace(Z=2, L=1000), "bf16", 256, 64, False, False),
    "fp32_rev_block256_dt_post": (W["tiny_fp32"].replace(L=777, Z=2, chunk=128), "fp32", 128, 256,
                                  False, True),
    "fp32_groups": (W["tiny_fp32"].replace(L=300, H=8, G=2, N=128, chunk=128, Z=2), "fp32", 128, 0,
                    False, False),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_saved_equals_recomputed(name):
    w, dtype, chunk, rb, with_init, post = CASES[name]
    inp = gen.make_inputs(w, with_dy=True)
    if post:
        inp = gen.with_dt_post(inp, w)
    S0 = None
    if with_init:
        S0 = np.random.default_rng(5).standard_normal((w.Z, w.H, 64, w.N)).astype(np.float32) * 0.5
        S0 = S0.astype(np.float64)
    print("saved", name, flush=True)
    y0, g0, y1, g1 = both_paths(inp, dtype, chunk, rb, S0, post)
    assert np.array_equal(y0, y1)
    assert sorted(g0) == sorted(g1)
    for k in g0:
        assert np.array_equal(g0[k], g1[k]), k


def test_saved_against_the_oracle():
    w = W["train_L2k"].replace(Z=2, L=700, H=6)
    inp = gen.make_inputs(w, mode="scan", with_dy=True)
    print("saved vs oracle", flush=True)
    _, _, y1, g1 = both_paths(inp, "bf16", 256)
    assert maxrel(y1, O.forward(inp)) <= TOL["bf16"]
    r = O.backward(inp, inp["dy"])
    errs = {k: maxrel(g1[k], r[k]) for k in KEYS}
    print(" ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    assert max(errs.values()) <= TOL["bf16"], errs


def test_saving_forward_takes_the_backward_workspace():
    """A saving forward needs the backward's workspace size; a forward-sized
    workspace is refused before anything runs, and the binding hands the
    workspace it allocated back as the saved values."""
    w = W["tiny_fp32"].replace(L=300, Z=1)
    inp = gen.make_inputs(w, with_dy=True)
    T = to_dev(inp, "fp32")
    f, r = directions(inp, T, False)
    plain = ssd.shape_of(T["x"], T["B_f"], 64)
    nf = ssd.bissd_workspace_size(plain, 0)
    nb = ssd.bissd_workspace_size(plain, 1)
    small = torch.empty(nf, dtype=torch.uint8, device=T["x"].device)
    with pytest.raises(RuntimeError):
        ssd.bissd_forward(T["x"], f, r, T["D"], chunk=64, workspace=small, save=True)
    y, saved = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=64, save=True)
    torch.cuda.synchronize()
    assert saved.numel() * saved.element_size() >= nb
