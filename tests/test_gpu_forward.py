"""GPU parity of the bidirectional scan (bissd_forward) against the fp64
oracle, element by element on the same seeded inputs.

Tolerance: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32) or 2e-2 (bf16) on
every checked tensor, in every check mode.  D x dominates y under the
workload distributions, so the modes "fwd" (D = 0, C_r = 0) and "rev"
(D = 0, C_f = 0) check each scan on its own.  Integer-valued cases and
causality zeros are checked bit for bit.
"""
import numpy as np
import pytest

from oracle import oracle as O
from synth import gen
from tests.gpu_util import TOL, dirs, gpu_forward, host, maxrel, select_heads, select_rows, to_dev

pytestmark = pytest.mark.gpu

W = gen.WORKLOADS
MODES = ("full", "scan", "fwd", "rev")


def check(inp, dtype, chunk, tol=None, **kw):
    g = gpu_forward(inp, dtype, chunk, **kw)
    r = O.forward(inp, **({"init_state": kw["init_state"]} if "init_state" in kw else {}))
    err = maxrel(g, r)
    assert err <= (tol or TOL[dtype]), err
    return err


@pytest.mark.parametrize("mode", MODES)
def test_tiny_fp32(mode):
    w = W["tiny_fp32"]
    inp = gen.make_inputs(w, mode=mode)
    print("tiny_fp32", mode, flush=True)
    check(inp, "fp32", w.chunk)


@pytest.mark.parametrize("mode", MODES)
def test_layer130m_L1k(mode):
    """Full 130M-class layer (Z=8, L=1024, 24 heads, N=128, chunk 256) on the
    GPU; the oracle checks batch rows 0, 3 and 7."""
    w = W["layer130m_L1k"]
    inp = gen.make_inputs(w, mode=mode)
    print("layer130m_L1k", mode, flush=True)
    g = gpu_forward(inp, "bf16", w.chunk)
    rows = [0, 3, 7]
    r = O.forward(select_rows(inp, rows))
    err = maxrel(g[rows], r)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("mode", MODES)
def test_two_head_tiles_fp32(mode):
    """fp32 at the layer130m_L1k shape (Z=8, L=1024, 24 heads, N=128, chunk
    256): here the chunk-state and output passes run two heads per workgroup
    (problems that fit one round of one-head workgroups run one); the oracle
    checks batch rows 0 and 5, in every check mode."""
    w = W["layer130m_L1k"].replace(dtype="fp32")
    inp = gen.make_inputs(w, mode=mode)
    print("layer130m_L1k fp32", mode, flush=True)
    g = gpu_forward(inp, "fp32", w.chunk)
    rows = [0, 5]
    r = O.forward(select_rows(inp, rows))
    err = maxrel(g[rows], r)
    assert err <= TOL["fp32"], err


@pytest.mark.parametrize("mode", ("full", "fwd", "rev"))
def test_long_L65k_sampled_heads(mode):
    """L=65536 (256 chunks): the GPU runs every head; the oracle checks heads
    0 and 17 over the whole sequence."""
    w = W["long_L65k"]
    inp = gen.make_inputs(w, mode=mode)
    print("long_L65k", mode, flush=True)
    g = gpu_forward(inp, "bf16", w.chunk)
    hs = [0, 17]
    r = O.forward(select_heads(inp, hs))
    err = maxrel(g[:, :, hs], r)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype", ("fp32", "bf16"))
@pytest.mark.parametrize("chunk", (64, 128, 256))
@pytest.mark.parametrize("L", (1, 63, 65, 255, 257, 1000))
def test_chunks_and_ragged_lengths(dtype, chunk, L):
    w = W["tiny_fp32"].replace(Z=2, L=L, H=4, N=128, chunk=chunk, dtype=dtype, seed=7 + L)
    for mode in ("fwd", "rev"):
        check(gen.make_inputs(w, mode=mode), dtype, chunk)


@pytest.mark.parametrize("H,G", [(4, 2), (6, 3), (3, 3), (8, 1)])
def test_groups(H, G):
    w = W["tiny_fp32"].replace(Z=2, L=300, H=H, G=G, N=64, chunk=128, dtype="bf16", seed=H * 10 + G)
    for mode in ("full", "fwd", "rev"):
        check(gen.make_inputs(w, mode=mode), "bf16", 128)


@pytest.mark.parametrize("dtype", ("fp32", "bf16"))
def test_init_and_final_state(dtype):
    w = W["tiny_fp32"].replace(Z=2, L=700, H=4, N=128, chunk=256, dtype=dtype, seed=31)
    inp = gen.make_inputs(w, mode="fwd")
    S0 = gen.round_fp32(np.random.default_rng(5).standard_normal((2, 4, 64, 128)) * 0.3)
    g, gfs = gpu_forward(inp, dtype, 256, init_state=S0, final=True)
    o = O.forward(inp, init_state=S0, final_state=True)
    assert maxrel(g, o["y"]) <= TOL[dtype]
    assert maxrel(gfs, o["final_state"]) <= TOL[dtype]


def test_weight_tied_directions_share_buffers():
    import torch
    import state_space_denoisers_amd as ssd
    from tests.gpu_util import to_dev, host
    w = W["tiny_fp32"].replace(Z=2, L=200, H=4, N=64, chunk=64, dtype="bf16", seed=41)
    inp = gen.make_inputs(w, mode="scan")
    for k in ("dt", "A", "B", "C"):
        inp[f"{k}_r"] = inp[f"{k}_f"]
    T = to_dev(inp, "bf16")
    f = (T["dt_f"], T["A_f"], T["B_f"], T["C_f"])
    y = ssd.bissd_forward(T["x"], f, f, T["D"], chunk=64)
    torch.cuda.synchronize()
    assert maxrel(host(y), O.forward(inp)) <= TOL["bf16"]


def closed_form_inputs(Z, L, H, N, seed, density=1.0):
    r = np.random.default_rng(seed)
    x = r.integers(-1, 2, (Z, L, H, 64)).astype(np.float64)
    if density < 1.0:
        x *= r.random(x.shape) < density
    e0 = np.zeros((Z, L, 1, N))
    e0[..., 0] = 1.0
    inp = {"x": x, "D": np.zeros(H)}
    for d in ("f", "r"):
        inp[f"dt_{d}"] = np.ones((Z, L, H))
        inp[f"A_{d}"] = np.zeros(H)
        inp[f"B_{d}"] = e0
        inp[f"C_{d}"] = e0
    return inp


@pytest.mark.parametrize("dtype,L,chunk", [("fp32", 1000, 64), ("fp32", 1000, 128),
                                           ("fp32", 1000, 256), ("bf16", 128, 64),
                                           ("bf16", 100, 256)])
def test_closed_form_prefix_sums_bit_exact(dtype, L, chunk):
    """A = 0, B = C = e_0, dt = 1: y is an exact running sum from each side;
    every chunk and block boundary must be indexed exactly."""
    inp = closed_form_inputs(2, L, 4, 128, seed=L + chunk)
    g = gpu_forward(inp, dtype, chunk)
    x = inp["x"]
    expect = np.cumsum(x, 1) + np.cumsum(x[:, ::-1], 1)[:, ::-1]
    assert np.array_equal(g, expect)


def test_closed_form_sparse_impulses_bf16_long():
    inp = closed_form_inputs(1, 3000, 4, 64, seed=3, density=0.01)
    g = gpu_forward(inp, "bf16", 256)
    x = inp["x"]
    expect = np.cumsum(x, 1) + np.cumsum(x[:, ::-1], 1)[:, ::-1]
    assert np.max(np.abs(expect)) <= 256
    assert np.array_equal(g, expect)


@pytest.mark.parametrize("s", [0, 63, 64, 200, 511])
def test_causality_exact_zeros(s):
    w = W["tiny_fp32"].replace(Z=1, L=512, H=4, N=128, chunk=128, dtype="bf16", seed=s)
    for mode in ("fwd", "rev"):
        inp = gen.make_inputs(w, mode=mode)
        inp["x"] = np.zeros_like(inp["x"])
        inp["x"][:, s] = 1.0
        g = gpu_forward(inp, "bf16", 128)
        if mode == "fwd":
            assert np.all(g[:, :s] == 0.0)
            assert np.any(g[:, s:] != 0.0)
        else:
            assert np.all(g[:, s + 1:] == 0.0)
            assert np.any(g[:, : s + 1] != 0.0)


def test_deterministic():
    w = W["layer130m_L1k"].replace(Z=2)
    inp = gen.make_inputs(w)
    a = gpu_forward(inp, "bf16", 256)
    b = gpu_forward(inp, "bf16", 256)
    assert np.array_equal(a, b)


def test_chunk_invariance_bf16():
    w = W["layer130m_L1k"].replace(Z=1, L=777, seed=5)
    inp = gen.make_inputs(w, mode="fwd")
    r = O.forward(inp)
    outs = [gpu_forward(inp, "bf16", q) for q in (64, 128, 256)]
    for g in outs:
        assert maxrel(g, r) <= TOL["bf16"]


@pytest.mark.parametrize("dtype", ("fp32", "bf16"))
def test_extreme_decays(dtype):
    """Per-token decays down to e^-48 (dt up to 3, |A| up to 16): the diagonal
    slab takes the exact per-element path; results stay finite and match."""
    w = W["tiny_fp32"].replace(Z=1, L=300, H=4, N=64, chunk=128, dtype=dtype, seed=77)
    r = np.random.default_rng(1)
    for mode in ("fwd", "rev", "full"):
        inp = gen.make_inputs(w, mode=mode)
        for d in ("f", "r"):
            inp[f"dt_{d}"] = gen.quantize(r.uniform(0.3, 3.0, inp[f"dt_{d}"].shape), dtype)
        g = gpu_forward(inp, dtype, 128)
        assert np.all(np.isfinite(g))
        assert maxrel(g, O.forward(inp)) <= TOL[dtype]


def test_every_decay_zero():
    """A = -1e30: every decay underflows to exactly 0, leaving the diagonal
    term of each direction (no NaN from 0 * inf anywhere)."""
    w = W["tiny_fp32"].replace(Z=2, L=200, H=4, N=64, chunk=64, dtype="fp32", seed=78)
    inp = gen.make_inputs(w, mode="scan")
    inp["A_f"] = np.full(4, -1e30)
    inp["A_r"] = np.full(4, -1e30)
    g = gpu_forward(inp, "fp32", 64)
    assert np.all(np.isfinite(g))
    assert maxrel(g, O.forward(inp)) <= TOL["fp32"]


@pytest.mark.parametrize("dtype,L", [("bf16", 1000), ("fp32", 300)])
def test_phases_compose(dtype, L):
    """The four phases enqueued one by one in the documented order (chunk
    states, Gram tiles, carry pass, output) give bissd_forward's y bit for
    bit, and the output phase alone repeated after them recomputes it."""
    import torch
    import state_space_denoisers_amd as ssd
    w = W["tiny_fp32"].replace(Z=2, L=L, H=4, N=128, chunk=256, dtype=dtype, seed=31)
    T = to_dev(gen.make_inputs(w), dtype)
    fwd, rev = dirs(T)
    full = host(ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=256))
    shape = ssd.shape_of(T["x"], T["B_f"], 256)
    nws = ssd.bissd_workspace_size(shape, 0)
    ws = torch.empty(nws, dtype=torch.uint8, device=T["x"].device)
    y = torch.full_like(T["x"], float("nan"))
    for p in (0, 3, 1, 2):
        ssd.bissd_forward_phase(p, T["x"], fwd, rev, T["D"], chunk=256, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), full)
    y.fill_(float("nan"))
    ssd.bissd_forward_phase(2, T["x"], fwd, rev, T["D"], chunk=256, y=y, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(host(y), full)


def flipped(inp: dict) -> dict:
    """The flip invariant's inputs: time reversed, with the two directions'
    parameters exchanged (x and dy flipped along time as well)."""
    out = {"x": inp["x"][:, ::-1].copy(), "D": inp["D"]}
    for a, b in (("f", "r"), ("r", "f")):
        for k in ("dt", "B", "C"):
            out[f"{k}_{a}"] = inp[f"{k}_{b}"][:, ::-1].copy()
        out[f"A_{a}"] = inp[f"A_{b}"]
    return out


@pytest.mark.parametrize("dtype,L,chunk", [("fp32", 1000, 256), ("bf16", 1000, 256),
                                           ("fp32", 333, 64)])
def test_flip_swaps_the_directions(dtype, L, chunk):
    """Reversing time and exchanging the two directions' parameters reverses
    y: the reverse scan is the forward scan of the flipped sequence.  The two
    GPU results agree with each other and with the oracle."""
    w = W["layer130m_L1k"].replace(Z=2, L=L, H=8, chunk=chunk, dtype=dtype, seed=90 + L)
    for mode in ("scan", "fwd"):
        inp = gen.make_inputs(w, mode=mode)
        print("flip", dtype, L, chunk, mode, flush=True)
        g = gpu_forward(inp, dtype, chunk)
        gf = gpu_forward(flipped(inp), dtype, chunk)
        assert maxrel(gf[:, ::-1], g) <= TOL[dtype]
        assert maxrel(gf, O.forward(flipped(inp))) <= TOL[dtype]


@pytest.mark.parametrize("mode", ("fwd", "rev"))
def test_long_L262k_sampled_heads(mode):
    """L=262,144 (1,024 chunks), the long end of the pages' context range:
    the GPU runs all 24 heads; the oracle checks heads 5 and 20 over the
    whole sequence."""
    w = W["long_L65k"].replace(L=262144, seed=1005)
    print("long_L262k", mode, "inputs", flush=True)
    inp = gen.make_inputs(w, mode=mode)
    print("long_L262k", mode, "gpu", flush=True)
    g = gpu_forward(inp, "bf16", w.chunk)
    hs = [5, 20]
    sub = select_heads(inp, hs)
    del inp
    print("long_L262k", mode, "oracle", flush=True)
    r = O.forward(sub)
    err = maxrel(g[:, :, hs], r)
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype,L,chunk,rb", [("fp32", 1000, 64, 64), ("fp32", 1000, 128, 64),
                                              ("fp32", 1000, 256, 128), ("fp32", 1000, 256, 512),
                                              ("fp32", 1000, 128, 256), ("bf16", 128, 128, 64),
                                              ("bf16", 128, 64, 64)])
def test_closed_form_segmented_reverse_bit_exact(dtype, L, chunk, rb):
    """A = 0, B = C = e_0, dt = 1 with the block-segmented reverse: the
    forward part is a running sum over the whole sequence and the reverse part
    a running sum from the end of each token's own block of rb tokens, bit for
    bit (every block boundary indexed exactly)."""
    import state_space_denoisers_amd as ssd
    inp = closed_form_inputs(2, L, 4, 128, seed=L + chunk + rb)
    T = to_dev(inp, dtype)
    y = ssd.bissd_forward(T["x"], *dirs(T), T["D"], chunk=chunk, rev_block=rb)
    g = host(y)
    x = inp["x"]
    yr = np.zeros_like(x)
    for k0 in range(0, L, rb):
        blk = x[:, k0:k0 + rb]
        yr[:, k0:k0 + rb] = np.cumsum(blk[:, ::-1], 1)[:, ::-1]
    expect = np.cumsum(x, 1) + yr
    assert np.array_equal(g, expect)


def test_caller_stream():
    """A call on a caller's stream that is not the current one allocates its
    output and workspace on that stream and gives the same y, bit for bit."""
    import torch
    import state_space_denoisers_amd as ssd
    w = W["layer130m_L1k"].replace(Z=2, L=700, H=8, seed=57)
    inp = gen.make_inputs(w)
    T = to_dev(inp, "bf16")
    y0 = ssd.bissd_forward(T["x"], *dirs(T), T["D"], chunk=256)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    ys = [ssd.bissd_forward(T["x"], *dirs(T), T["D"], chunk=256, stream=s) for _ in range(3)]
    s.synchronize()
    for y in ys:
        assert torch.equal(y, y0)
    assert maxrel(host(y0), O.forward(inp)) <= TOL["bf16"]
