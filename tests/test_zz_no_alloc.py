"""bissd_forward_noalloc (the forward with the library's static scratch array
as its workspace, for callers that cannot allocate) against bissd_forward
with a caller workspace, through the C ABI: bit for bit on two calls in a
row, the second with a smaller input (the array keeps the first call's
contents), and both within the bf16 tolerance of the fp64 oracle.  A shape
whose workspace exceeds the array is rejected before anything is launched.
"""
import numpy as np
import pytest
import torch

import state_space_denoisers_amd as ssd
from state_space_denoisers_amd import _abi
from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, dirs, host, maxrel, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS


def both(inp, dtype, chunk, final=False):
    T = to_dev(inp, dtype)
    f, r = dirs(T)
    Z, L, H, P = T["x"].shape
    N = T["B_f"].shape[-1]
    fs_a = torch.full((Z, H, P, N), float("nan"), device=T["x"].device) if final else None
    fs_b = torch.full((Z, H, P, N), float("nan"), device=T["x"].device) if final else None
    y_ref = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=chunk, final_state=fs_a)
    y = torch.full_like(T["x"], float("nan"))
    ssd.bissd_forward_noalloc(T["x"], f, r, T["D"], chunk=chunk, y=y, final_state=fs_b)
    torch.cuda.synchronize()
    return host(y), host(y_ref), (host(fs_b), host(fs_a)) if final else None


def test_noalloc_matches_the_workspace_call_on_two_calls():
    # first call: the 130M-class layer at full size (56 MiB of workspace)
    w1 = W["layer130m_L1k"]
    inp1 = gen.make_inputs(w1)
    print("noalloc call 1", flush=True)
    y, y_ref, _ = both(inp1, "bf16", w1.chunk)
    assert np.array_equal(y, y_ref)
    rows = [0, 7]
    assert maxrel(y[rows], O.forward({k: (v if v.ndim == 1 else v[rows]) for k, v in inp1.items()})) <= TOL["bf16"]
    # second call, smaller, in scan mode, with an end state: the array still
    # holds the first call's states and Gram tiles
    w2 = W["layer130m_L1k"].replace(Z=2, L=700, H=8, seed=77)
    inp2 = gen.make_inputs(w2, mode="scan")
    print("noalloc call 2", flush=True)
    y2, y2_ref, (fs, fs_ref) = both(inp2, "bf16", w2.chunk, final=True)
    assert np.array_equal(y2, y2_ref)
    assert np.array_equal(fs, fs_ref)
    ro = O.forward(inp2, final_state=True)
    assert maxrel(y2, ro["y"]) <= TOL["bf16"]
    assert maxrel(fs, ro["final_state"]) <= TOL["bf16"]


def test_noalloc_fp32_small():
    w = W["tiny_fp32"].replace(Z=2, L=300, H=4, N=128, chunk=128)
    inp = gen.make_inputs(w, mode="fwd")
    print("noalloc fp32", flush=True)
    y, y_ref, _ = both(inp, "fp32", 128)
    assert np.array_equal(y, y_ref)
    assert maxrel(y, O.forward(inp)) <= TOL["fp32"]


def test_noalloc_rejects_a_shape_beyond_the_scratch_array():
    """Z=2, L=65536 needs about 1 GB of workspace: BISSD_ERR_SCRATCH, and y
    is left untouched."""
    w = W["long_L65k"].replace(Z=2, L=65536, H=4)
    dev = torch.device("cuda", 0)
    x = torch.zeros((2, 65536, 4, 64), dtype=torch.bfloat16, device=dev)
    B = torch.zeros((2, 65536, 1, 128), dtype=torch.bfloat16, device=dev)
    dt = torch.zeros((2, 65536, 4), dtype=torch.bfloat16, device=dev)
    A = torch.zeros(4, dtype=torch.float32, device=dev)
    d = (dt, A, B, B)
    shape = ssd.shape_of(x, B, w.chunk)
    assert ssd.bissd_workspace_size(shape, _abi.OP_FORWARD) > _abi.NOALLOC_SCRATCH_BYTES
    y = torch.full_like(x, float("nan"))
    with pytest.raises(ssd.BissdError) as e:
        ssd.bissd_forward_noalloc(x, d, d, A, y=y, chunk=w.chunk)
    assert e.value.status == -8
    torch.cuda.synchronize()
    assert torch.isnan(y.float()).all()
