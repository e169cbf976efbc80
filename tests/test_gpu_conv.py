"""GPU parity of the mixer's convolution fused in front of the scan (each
direction's scan reads its own causal / anti-causal depthwise convolution of
x, SiLU-activated; the block update continues the forward convolution from a
conv state) against the fp64 oracle (oracle/conv.py: the plain convolution,
then the plain scan).  Tolerance: max|gpu - oracle| / max|oracle| <= 1e-4
(fp32), 2e-2 (bf16), in the check modes of the forward tests.
"""
import numpy as np
import pytest
import torch

import state_space_denoisers_amd as ssd
from oracle import conv as CV
from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, f32_dev, host, maxrel, select_rows, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS


def conv_dirs(inp, T, cv, which=("f", "r"), act=True):
    out = []
    for d in ("f", "r"):
        kw = {}
        if d in which:
            kw = dict(conv_w=f32_dev(cv[f"conv_w_{d}"]), conv_b=f32_dev(cv[f"conv_b_{d}"]), conv_act=act)
        out.append(ssd.Dir(T[f"dt_{d}"], T[f"A_{d}"], T[f"B_{d}"], T[f"C_{d}"], **kw))
    return out


def oracle_convs(cv, which=("f", "r"), act=True):
    return {d: ((cv[f"conv_w_{d}"], cv[f"conv_b_{d}"], act) if d in which else None) for d in ("f", "r")}


@pytest.mark.parametrize("dtype,L,chunk,K", [("fp32", 300, 64, 4), ("fp32", 1000, 256, 2),
                                             ("bf16", 1000, 256, 4), ("bf16", 777, 128, 3)])
@pytest.mark.parametrize("mode", ("full", "fwd", "rev"))
def test_forward_with_convolution(dtype, L, chunk, K, mode):
    w = W["tiny_fp32"].replace(Z=2, L=L, H=4, N=128, chunk=chunk, dtype=dtype, seed=300 + L + K)
    inp = gen.make_inputs(w, mode=mode)
    cv = gen.make_conv(w, K)
    T = to_dev(inp, dtype)
    f, r = conv_dirs(inp, T, cv)
    print("conv fwd", dtype, L, chunk, K, mode, flush=True)
    y = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=chunk)
    torch.cuda.synchronize()
    e = maxrel(host(y), CV.forward(inp, oracle_convs(cv)))
    print(f"err={e:.2e}", flush=True)
    assert e <= TOL[dtype]


@pytest.mark.parametrize("mode", ("full", "scan"))
def test_layer130m_L1k_with_convolution(mode):
    """The bench's convolution leg at its size (Z=8, L=1024, 24 heads, N=128,
    chunk 256, bf16, width 4 on both directions); the oracle checks batch
    rows 0 and 7."""
    w = W["layer130m_L1k"]
    inp = gen.make_inputs(w, mode=mode)
    cv = gen.make_conv(w, 4)
    T = to_dev(inp, "bf16")
    f, r = conv_dirs(inp, T, cv)
    print("conv layer130m_L1k", mode, flush=True)
    y = host(ssd.bissd_forward(T["x"], f, r, T["D"], chunk=w.chunk))
    rows = [0, 7]
    e = maxrel(y[rows], CV.forward(select_rows(inp, rows), oracle_convs(cv)))
    print(f"err={e:.2e}", flush=True)
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("which", [("f",), ("r",)])
def test_one_direction_with_convolution(which):
    """A convolution on one direction only: the other scans x as given."""
    w = W["layer130m_L1k"].replace(Z=2, L=600, H=8, seed=311)
    inp = gen.make_inputs(w, mode="scan")
    cv = gen.make_conv(w, 4)
    T = to_dev(inp, "bf16")
    f, r = conv_dirs(inp, T, cv, which)
    y = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=256)
    torch.cuda.synchronize()
    assert maxrel(host(y), CV.forward(inp, oracle_convs(cv, which))) <= TOL["bf16"]


def test_identity_taps_equal_the_plain_scan():
    """One tap of weight 1, no bias, no activation: the scan of x itself."""
    w = W["tiny_fp32"].replace(Z=2, L=500, H=4, N=128, chunk=128, seed=312)
    inp = gen.make_inputs(w)
    T = to_dev(inp, "fp32")
    one = torch.ones((4, 64, 1), dtype=torch.float32, device=T["x"].device)
    f = ssd.Dir(T["dt_f"], T["A_f"], T["B_f"], T["C_f"], conv_w=one, conv_act=False)
    r = ssd.Dir(T["dt_r"], T["A_r"], T["B_r"], T["C_r"], conv_w=one, conv_act=False)
    y1 = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=128)
    y0 = ssd.bissd_forward(T["x"], tuple(f[:4]), tuple(r[:4]), T["D"], chunk=128)
    torch.cuda.synchronize()
    assert maxrel(host(y1), host(y0)) <= 1e-6


@pytest.mark.parametrize("rb,chunk", [(64, 128), (256, 128)])
def test_segmented_reverse_with_convolution(rb, chunk):
    """The block-segmented reverse: the reverse's convolution reads nothing
    past the end of its block either."""
    w = W["tiny_fp32"].replace(Z=2, L=700, H=4, N=128, chunk=chunk, dtype="fp32", seed=313)
    inp = gen.make_inputs(w, mode="rev")
    cv = gen.make_conv(w, 4)
    T = to_dev(inp, "fp32")
    f, r = conv_dirs(inp, T, cv)
    y = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=chunk, rev_block=rb)
    torch.cuda.synchronize()
    assert maxrel(host(y), CV.forward(inp, oracle_convs(cv), rev_block=rb)) <= TOL["fp32"]


def test_start_state_with_convolution():
    w = W["tiny_fp32"].replace(Z=2, L=400, H=4, N=128, chunk=256, dtype="fp32", seed=314)
    inp = gen.make_inputs(w, mode="fwd")
    cv = gen.make_conv(w, 4)
    S0 = gen.round_fp32(np.random.default_rng(3).standard_normal((2, 4, 64, 128)) * 0.3)
    T = to_dev(inp, "fp32")
    f, r = conv_dirs(inp, T, cv)
    y = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=256, init_state=f32_dev(S0))
    torch.cuda.synchronize()
    assert maxrel(host(y), CV.forward(inp, oracle_convs(cv), init_state=S0)) <= TOL["fp32"]


@pytest.mark.parametrize("dtype", ("fp32", "bf16"))
@pytest.mark.parametrize("Lb,chunk,K", [(64, 64, 4), (37, 64, 4), (2, 64, 4), (1, 64, 2),
                                        (100, 128, 4), (2, 128, 3), (256, 256, 4)])
def test_block_update_with_conv_state(dtype, Lb, chunk, K):
    """The forward convolution continues from the conv state (the last K-1
    prefix rows), the reverse stays in the block; the committed conv state
    is the last K-1 rows of [conv state | block], in place and not.  Blocks
    of at most 64 tokens run the single block kernel, longer ones the
    convolution pass and the chunked kernels."""
    w = W["block_update"].replace(Z=2, L=Lb, H=4, dtype=dtype, mask_count=0, seed=320 + Lb + K)
    inp = gen.make_inputs(w)
    cv = gen.make_conv(w, K)
    cst = gen.make_conv_state(w, K)
    S0 = gen.round_fp32(np.random.default_rng(Lb).standard_normal((2, 4, 64, 128)) * 0.05)
    T = to_dev(inp, dtype)
    f, r = conv_dirs(inp, T, cv)
    ry, rso, rcs = CV.block_update(inp, oracle_convs(cv), S0, conv_state=cst)
    for alias in (False, True):
        c_in = gen.as_torch(cst, dtype, T["x"].device)
        c_out = c_in if alias else torch.full_like(c_in, float("nan"))
        s_in = f32_dev(S0)
        y, so = ssd.bissd_block_update(s_in, T["x"], f, r, T["D"], chunk=chunk, conv_state=c_in,
                                       conv_state_out=c_out)
        torch.cuda.synchronize()
        assert maxrel(host(y), ry) <= TOL[dtype], alias
        assert maxrel(host(so), rso) <= TOL[dtype], alias
        assert np.array_equal(host(c_out), rcs), alias


def test_block_update_with_conv_matches_the_full_forward():
    """Cache consistency with the convolution on the GPU: the forward scan
    over [prefix | block] restricted to the block equals the block update
    from the prefix's final state and its last three x rows as conv state
    (forward-only check mode), bf16."""
    Lp, Lb, K = 1000, 64, 4
    w = W["layer130m_L1k"].replace(Z=2, L=Lp + Lb, H=8, seed=330)
    full = gen.make_inputs(w, mode="fwd")
    cv = gen.make_conv(w, K)
    pre = {k: (v[:, :Lp] if v.ndim > 1 else v) for k, v in full.items()}
    blk = {k: (v[:, Lp:] if v.ndim > 1 else v) for k, v in full.items()}
    Tf, Tp, Tb = to_dev(full, "bf16"), to_dev(pre, "bf16"), to_dev(blk, "bf16")
    fs = torch.empty((2, 8, 64, 128), device=Tp["x"].device)
    ssd.bissd_forward(Tp["x"], *conv_dirs(pre, Tp, cv), Tp["D"], chunk=256, final_state=fs)
    y_full = ssd.bissd_forward(Tf["x"], *conv_dirs(full, Tf, cv), Tf["D"], chunk=256)
    cst = Tp["x"][:, Lp - (K - 1):].contiguous()
    y_blk, _ = ssd.bissd_block_update(fs, Tb["x"], *conv_dirs(blk, Tb, cv), Tb["D"], chunk=64,
                                      conv_state=cst)
    torch.cuda.synchronize()
    ref = CV.forward(full, oracle_convs(cv))[:, Lp:]
    assert maxrel(host(y_blk), ref) <= TOL["bf16"]
    assert maxrel(host(y_blk), host(y_full)[:, Lp:]) <= TOL["bf16"]


def test_noalloc_forward_with_convolution():
    w = W["layer130m_L1k"].replace(Z=2, L=700, H=8, seed=331)
    inp = gen.make_inputs(w, mode="scan")
    cv = gen.make_conv(w, 4)
    T = to_dev(inp, "bf16")
    f, r = conv_dirs(inp, T, cv)
    y0 = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=256)
    y1 = torch.full_like(T["x"], float("nan"))
    ssd.bissd_forward_noalloc(T["x"], f, r, T["D"], chunk=256, y=y1)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1)


def test_backward_rejects_a_convolution():
    w = W["tiny_fp32"].replace(Z=1, L=100, H=4)
    inp = gen.make_inputs(w, with_dy=True)
    cv = gen.make_conv(w, 4)
    T = to_dev(inp, "fp32")
    f, r = conv_dirs(inp, T, cv)
    with pytest.raises(ssd.BissdError):
        ssd.bissd_backward(T["x"], f, r, T["D"], T["dy"], chunk=64)


def full_dirs(inp, T, cv):
    """Directions with dt post-processing and the convolution together."""
    out = []
    for d in ("f", "r"):
        b = gen.as_torch(inp[f"dt_bias_{d}"], "fp32", T["x"].device)
        out.append(ssd.Dir(T[f"dt_{d}"], T[f"A_{d}"], T[f"B_{d}"], T[f"C_{d}"], b,
                           inp[f"dt_min_{d}"], inp[f"dt_max_{d}"],
                           conv_w=f32_dev(cv[f"conv_w_{d}"]), conv_b=f32_dev(cv[f"conv_b_{d}"]),
                           conv_act=True))
    return out


@pytest.mark.parametrize("dtype", ("fp32", "bf16"))
def test_convolution_with_dt_post_and_reverse_blocks(dtype):
    """Every option of the forward at once: each direction's dt through its
    bias, softplus and clamp, its width-3 convolution, and the reverse scan
    restarting at every 64-token block (chunks of 128, a ragged tail)."""
    w = W["tiny_fp32"].replace(Z=2, L=500, H=6, N=128, chunk=128, dtype=dtype, seed=421)
    inp = gen.with_dt_post(gen.make_inputs(w, mode="scan"), w)
    cv = gen.make_conv(w, 3)
    T = to_dev(inp, dtype)
    f, r = full_dirs(inp, T, cv)
    print("conv + dt post + rev_block 64", dtype, flush=True)
    y = ssd.bissd_forward(T["x"], f, r, T["D"], chunk=128, rev_block=64)
    torch.cuda.synchronize()
    e = maxrel(host(y), CV.forward(inp, oracle_convs(cv), rev_block=64))
    print(f"err={e:.2e}", flush=True)
    assert e <= TOL[dtype]


@pytest.mark.parametrize("Lb", (40, 100))
def test_block_update_with_dt_post_and_conv_state(Lb):
    """The block update with dt post-processing and the convolution together,
    continuing a cached state and a conv state, both committed (in place)."""
    w = W["block_update"].replace(Z=2, L=Lb, H=6, dtype="bf16", seed=433 + Lb)
    inp = gen.with_dt_post(gen.make_inputs(w, mode="scan"), w)
    cv = gen.make_conv(w, 4)
    cst = gen.make_conv_state(w, 4)
    S0 = gen.round_fp32(np.random.default_rng(9).standard_normal((2, 6, 64, 128)) * 0.05)
    T = to_dev(inp, "bf16")
    f, r = full_dirs(inp, T, cv)
    state = f32_dev(S0)
    cstate = gen.as_torch(cst, "bf16", T["x"].device)
    print("block + dt post + conv state", Lb, flush=True)
    y, so = ssd.bissd_block_update(state, T["x"], f, r, T["D"], chunk=128 if Lb > 64 else 64,
                                   state_out=state, conv_state=cstate, conv_state_out=cstate)
    torch.cuda.synchronize()
    ry, rso, rcs = CV.block_update(inp, oracle_convs(cv), S0, cst)
    assert maxrel(host(y), ry) <= TOL["bf16"]
    assert maxrel(host(so), rso) <= TOL["bf16"]
    assert np.array_equal(host(cstate), rcs)
