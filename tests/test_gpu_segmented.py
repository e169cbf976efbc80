"""GPU parity of the block-segmented reverse scan (shape rev_block > 0: the
reverse state restarts at every block end, the forward scan spans the whole
sequence) against the fp64 oracle, forward and backward, element by element.

Covers blocks shorter than a chunk (64 and 128 tokens inside chunks of 128
and 256), blocks of exactly one chunk, blocks spanning several chunks, ragged
last blocks and chunks, a forward start state, and a block at least as long
as the sequence (which must equal the unsegmented scan bit for bit).
Tolerance: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32), 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, dirs, f32_dev, host, maxrel, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS
GKEYS = ("dx", "ddt_f", "dA_f", "dB_f", "dC_f", "ddt_r", "dA_r", "dB_r", "dC_r", "dD")


def gpu_fwd(inp, dtype, chunk, rb, init_state=None, final=False):
    import state_space_denoisers_amd as ssd
    T = to_dev(inp, dtype)
    fwd, rev = dirs(T)
    Z, L, H, P = inp["x"].shape
    N = inp["B_f"].shape[-1]
    fs = torch.full((Z, H, P, N), float("nan"), device=T["x"].device) if final else None
    init = None if init_state is None else f32_dev(init_state)
    y = ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=chunk, rev_block=rb,
                          init_state=init, final_state=fs)
    torch.cuda.synchronize()
    return (host(y), host(fs)) if final else host(y)


def gpu_bwd(inp, dtype, chunk, rb, init_state=None):
    import state_space_denoisers_amd as ssd
    T = to_dev(inp, dtype)
    fwd, rev = dirs(T)
    init = None if init_state is None else f32_dev(init_state)
    g = ssd.bissd_backward(T["x"], fwd, rev, T["D"], T["dy"], chunk=chunk, rev_block=rb,
                           init_state=init)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in g.items()}


def check_bwd(inp, dtype, chunk, rb, init_state=None):
    g = gpu_bwd(inp, dtype, chunk, rb, init_state)
    r = O.backward(inp, inp["dy"], init_state=init_state, rev_block=rb)
    errs = {}
    for k in GKEYS:
        assert np.all(np.isfinite(g[k])), k
        errs[k] = maxrel(g[k], r[k])
    print(" ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if v > TOL[dtype]}
    assert not bad, (bad, errs)


# (chunk, rev_block, L): blocks inside a chunk, one chunk, several chunks;
# ragged last blocks and chunks
CASES = [(256, 64, 1000), (256, 128, 700), (128, 64, 450), (64, 64, 300), (256, 256, 900),
         (64, 192, 500), (128, 256, 1100), (256, 512, 1300)]


@pytest.mark.parametrize("chunk,rb,L", CASES)
def test_forward_fp32(chunk, rb, L):
    w = W["tiny_fp32"].replace(L=L, chunk=chunk, Z=2)
    inp = gen.make_inputs(w)
    print("seg fwd fp32", chunk, rb, L, flush=True)
    y = gpu_fwd(inp, "fp32", chunk, rb)
    e = maxrel(y, O.forward(inp, rev_block=rb))
    print(f"err={e:.1e}", flush=True)
    assert e <= TOL["fp32"]


@pytest.mark.parametrize("chunk,rb,L", [(256, 64, 1000), (256, 512, 1300)])
def test_forward_bf16_layer(chunk, rb, L):
    w = W["layer130m_L1k"].replace(L=L, chunk=chunk, Z=2)
    inp = gen.make_inputs(w)
    print("seg fwd bf16", chunk, rb, L, flush=True)
    y = gpu_fwd(inp, "bf16", chunk, rb)
    e = maxrel(y, O.forward(inp, rev_block=rb))
    print(f"err={e:.1e}", flush=True)
    assert e <= TOL["bf16"]


def test_forward_start_state_and_final_state():
    """The forward direction (and so the cache it leaves) is unchanged by the
    reverse blocks."""
    w = W["tiny_fp32"].replace(L=600, chunk=128, Z=2, N=128)
    inp = gen.make_inputs(w)
    S0 = np.random.default_rng(91).standard_normal((2, w.H, 64, w.N)) * 0.5
    print("seg fwd init/final", flush=True)
    y, fs = gpu_fwd(inp, "fp32", 128, 64, init_state=S0, final=True)
    o = O.forward(inp, init_state=S0, final_state=True, rev_block=64)
    assert maxrel(y, o["y"]) <= TOL["fp32"]
    assert maxrel(fs, o["final_state"]) <= TOL["fp32"]


def test_block_at_least_the_sequence_is_the_unsegmented_scan():
    w = W["tiny_fp32"].replace(L=300, chunk=64, Z=2)
    inp = gen.make_inputs(w, with_dy=True)
    print("seg rb>=L", flush=True)
    for rb in (320, 1024):
        assert np.array_equal(gpu_fwd(inp, "fp32", 64, rb), gpu_fwd(inp, "fp32", 64, 0))
        a, b = gpu_bwd(inp, "fp32", 64, rb), gpu_bwd(inp, "fp32", 64, 0)
        for k in GKEYS:
            assert np.array_equal(a[k], b[k]), (rb, k)


@pytest.mark.parametrize("chunk,rb,L", CASES)
def test_backward_fp32(chunk, rb, L):
    w = W["tiny_fp32"].replace(L=L, chunk=chunk, Z=2)
    inp = gen.make_inputs(w, with_dy=True)
    print("seg bwd fp32", chunk, rb, L, flush=True)
    check_bwd(inp, "fp32", chunk, rb)


def test_backward_start_state_groups_fp32():
    w = W["tiny_fp32"].replace(L=520, H=8, G=2, N=128, chunk=256, Z=2)
    inp = gen.make_inputs(w, with_dy=True)
    S0 = np.random.default_rng(92).standard_normal((2, w.H, 64, w.N)) * 0.5
    print("seg bwd init groups", flush=True)
    check_bwd(inp, "fp32", 256, 128, init_state=S0)


@pytest.mark.parametrize("rb", (64, 512))
def test_backward_bf16_train_shape(rb):
    """The training layer shape (24 heads, N = 128, chunk 256, bf16) on two
    batch rows of 2048 tokens."""
    w = W["train_L2k"].replace(Z=2)
    inp = gen.make_inputs(w, with_dy=True)
    print("seg bwd bf16 train", rb, flush=True)
    check_bwd(inp, "bf16", w.chunk, rb)
