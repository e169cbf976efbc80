"""GPU parity of the backward pass (bissd_backward) against the fp64 oracle's
reverse-mode recurrence, element by element on the same seeded inputs.

Every gradient (dx, ddt, dA, dB, dC per direction, dD) must satisfy
max|gpu - oracle| / max|oracle| <= 1e-4 (fp32) or 2e-2 (bf16), in the check
modes "full" (as configured) and "scan" (D = 0).
"""
import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, dirs, f32_dev, host, maxrel, select_rows, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS
KEYS = ("dx", "ddt_f", "dA_f", "dB_f", "dC_f", "ddt_r", "dA_r", "dB_r", "dC_r", "dD")


def gpu_backward(inp, dtype, chunk, init_state=None):
    import state_space_denoisers_amd as ssd
    T = to_dev(inp, dtype)
    fwd, rev = dirs(T)
    init = None if init_state is None else f32_dev(init_state)
    g = ssd.bissd_backward(T["x"], fwd, rev, T["D"], T["dy"], chunk=chunk, init_state=init)
    torch.cuda.synchronize()
    return {k: host(v) for k, v in g.items()}


def check(inp, dtype, chunk, init_state=None, rows=None):
    g = gpu_backward(inp, dtype, chunk, init_state)
    ref_in = inp if rows is None else select_rows(inp, rows)
    r = O.backward(ref_in, ref_in["dy"], init_state=init_state)
    errs = {}
    for k in KEYS:
        gk = g[k]
        if rows is not None and gk.ndim > 1:
            gk = gk[rows]
        if rows is not None and gk.ndim == 1:
            continue  # batch-reduced gradients need every row
        assert np.all(np.isfinite(gk)), k
        errs[k] = maxrel(gk, r[k])
    print(" ".join(f"{k}={v:.1e}" for k, v in errs.items()), flush=True)
    bad = {k: v for k, v in errs.items() if v > TOL[dtype]}
    assert not bad, (bad, errs)
    return errs


@pytest.mark.parametrize("mode", ("full", "scan"))
def test_tiny_fp32(mode):
    w = W["tiny_fp32"]
    inp = gen.make_inputs(w, mode=mode, with_dy=True)
    print("bwd tiny_fp32", mode, flush=True)
    check(inp, "fp32", w.chunk)


@pytest.mark.parametrize("chunk,L", [(64, 1), (64, 63), (64, 65), (128, 255), (256, 257),
                                     (256, 1000), (128, 1000)])
def test_chunks_and_ragged_lengths_fp32(chunk, L):
    w = W["tiny_fp32"].replace(L=L, chunk=chunk, Z=2)
    inp = gen.make_inputs(w, mode="scan", with_dy=True)
    print("bwd ragged", chunk, L, flush=True)
    check(inp, "fp32", chunk)


@pytest.mark.parametrize("L", (356, 456))
def test_ragged_last_chunk_bf16(L):
    """bf16 at chunk 256 with a last chunk of 100 or 200 tokens: the
    carried-state kernels split a chunk's rows in halves of 128, so the
    second half is empty in one case and partly filled in the other."""
    w = W["tiny_fp32"].replace(L=L, chunk=256, Z=2, H=4, N=128, dtype="bf16")
    for mode in ("full", "scan"):
        inp = gen.make_inputs(w, mode=mode, with_dy=True)
        print("bwd ragged bf16", L, mode, flush=True)
        check(inp, "bf16", 256)


@pytest.mark.parametrize("chunk,L", [(256, 520), (128, 300)])
def test_dstate64_bf16(chunk, L):
    """bf16 with d_state 64 (the model card's width) and a ragged last chunk:
    the N = 64 instantiations of every backward kernel."""
    w = W["tiny_fp32"].replace(L=L, chunk=chunk, Z=2, H=4, N=64, dtype="bf16", seed=64 + L)
    for mode in ("full", "scan"):
        inp = gen.make_inputs(w, mode=mode, with_dy=True)
        print("bwd dstate64 bf16", chunk, L, mode, flush=True)
        check(inp, "bf16", chunk)


@pytest.mark.parametrize("dtype", ("fp32", "bf16"))
def test_groups_and_dstate(dtype):
    w = W["tiny_fp32"].replace(L=300, H=8, G=2, N=128, chunk=128, Z=2, dtype=dtype)
    inp = gen.make_inputs(w, with_dy=True)
    print("bwd groups", dtype, flush=True)
    check(inp, dtype, w.chunk)


def test_init_state_fp32():
    w = W["tiny_fp32"].replace(L=200, Z=2)
    inp = gen.make_inputs(w, with_dy=True)
    S0 = np.random.default_rng(77).standard_normal((2, w.H, 64, w.N)).astype(np.float32) * 0.5
    print("bwd init_state", flush=True)
    check(inp, "fp32", w.chunk, init_state=S0.astype(np.float64))


def test_weight_tied_directions():
    w = W["tiny_fp32"].replace(L=190, Z=2)
    inp = gen.make_inputs(w, with_dy=True)
    for k in ("dt", "A", "B", "C"):
        inp[k + "_r"] = inp[k + "_f"]
    print("bwd weight-tied", flush=True)
    check(inp, "fp32", 64)


@pytest.mark.parametrize("mode", ("full", "scan"))
def test_layer_bf16(mode):
    """bf16, N=128, chunk 256, ragged last chunk."""
    w = W["train_L2k"].replace(Z=2, L=700, H=6)
    inp = gen.make_inputs(w, mode=mode, with_dy=True)
    print("bwd layer bf16", mode, flush=True)
    check(inp, "bf16", w.chunk)


@pytest.mark.parametrize("mode", ("full", "scan"))
def test_train_L2k_full(mode):
    """The training workload at full size (Z=16, L=2048, 24 heads, N=128,
    chunk 256, bf16); every gradient against the oracle on every row.  In
    mode "scan" (D = 0) the scan part of dx is the whole of dx (with D it is
    about 1% of it)."""
    w = W["train_L2k"]
    inp = gen.make_inputs(w, mode=mode, with_dy=True)
    print("bwd train_L2k", mode, flush=True)
    check(inp, "bf16", w.chunk)


@pytest.mark.parametrize("mode", ("full", "scan", "fwd", "rev"))
def test_two_head_tiles_fp32(mode):
    """fp32 at Z=8, L=1024, 24 heads, N=128, chunk 256: a size at which the
    chunk-state pass runs two heads per workgroup (problems that fit one round
    of one-head workgroups run one); every gradient against the oracle on
    batch rows 0 and 5, in every check mode ("fwd": C_r = 0, so only the
    forward scan reaches y; "rev": C_f = 0)."""
    w = W["train_L2k"].replace(Z=8, L=1024, dtype="fp32")
    inp = gen.make_inputs(w, mode=mode, with_dy=True)
    print("bwd two-head tiles fp32", mode, flush=True)
    check(inp, "fp32", w.chunk, rows=[0, 5])


def test_extreme_decays_fp32():
    """Large dt A (decays underflow inside a chunk) and dt = 0 tokens."""
    w = W["tiny_fp32"].replace(L=256, Z=1, chunk=128)
    inp = gen.make_inputs(w, with_dy=True)
    inp["dt_f"][:, ::7] = 0.0
    inp["A_f"][:] = -40.0
    inp["A_r"][0] = -1e4
    print("bwd extreme decays", flush=True)
    check(inp, "fp32", w.chunk)


def test_determinism_bitwise():
    w = W["tiny_fp32"].replace(L=777, Z=2, H=8, N=128, chunk=256, dtype="bf16")
    inp = gen.make_inputs(w, with_dy=True)
    a = gpu_backward(inp, "bf16", 256)
    b = gpu_backward(inp, "bf16", 256)
    for k in KEYS:
        assert np.array_equal(a[k], b[k]), k


def test_chunk_invariance_fp32():
    w = W["tiny_fp32"].replace(L=512, Z=1)
    inp = gen.make_inputs(w, with_dy=True)
    a = gpu_backward(inp, "fp32", 64)
    b = gpu_backward(inp, "fp32", 256)
    for k in KEYS:
        assert maxrel(a[k], b[k]) <= 1e-5, k


@pytest.mark.parametrize("H,G", [(40, 2), (33, 1)])
def test_many_heads_fp32(H, G):
    """More heads than one decay-gradient workgroup takes (32): the heads
    split into equal groups (40 -> 2 x 20; 33 -> 17 + 16, an odd and an even
    LDS pitch); every gradient against the oracle."""
    w = W["tiny_fp32"].replace(L=300, Z=1, H=H, G=G, chunk=128)
    inp = gen.make_inputs(w, mode="scan", with_dy=True)
    print("bwd many heads", H, G, flush=True)
    check(inp, "fp32", w.chunk)
