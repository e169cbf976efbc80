"""Pins of the fp64 CPU oracle against things other than itself.

The pages print no numeric example of the scan, so every pin here is
mathematical: an independent dense formulation (materialised semiseparable
matrices + autograd), closed forms, a textbook filter routine, symmetries,
causality, cache consistency and finite differences.  Each is chosen so that a
plausible slip in ssd_oracle.c (wrong decay index, dropped diagonal, swapped
direction, wrong group, sign error in a gradient) fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.signal

from oracle import dense
from oracle import oracle as O

KEYS = ("x", "dt_f", "A_f", "B_f", "C_f", "dt_r", "A_r", "B_r", "C_r", "D")


def rand_inputs(Z, L, H, P, N, G, seed=0, dt_lo=0.01, dt_hi=0.3):
    r = np.random.default_rng(seed)
    inp = {"x": r.standard_normal((Z, L, H, P)), "D": r.standard_normal(H)}
    for d in ("f", "r"):
        inp[f"dt_{d}"] = r.uniform(dt_lo, dt_hi, (Z, L, H))
        inp[f"A_{d}"] = -np.exp(r.uniform(0, math.log(16), H))
        inp[f"B_{d}"] = r.standard_normal((Z, L, G, N)) / math.sqrt(N)
        inp[f"C_{d}"] = r.standard_normal((Z, L, G, N)) / math.sqrt(N)
    return inp


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    m = np.max(np.abs(b))
    return float(np.max(np.abs(a - b)) / (m if m > 0 else 1.0))


# ----------------------------------------------------------------- P1 dense

@pytest.mark.parametrize("shape", [(2, 37, 3, 5, 4, 1), (1, 130, 4, 8, 6, 2),
                                   (1, 64, 6, 3, 5, 3)])
def test_recurrence_matches_dense_semiseparable(shape):
    inp = rand_inputs(*shape, seed=1)
    o = O.forward(inp, parts=True)
    d = dense.forward(inp)
    assert rel(o["y_f"], d["y_f"]) < 1e-12
    assert rel(o["y_r"], d["y_r"]) < 1e-12
    assert rel(o["y"], d["y"]) < 1e-12


def test_recurrence_matches_dense_with_start_state():
    Z, L, H, P, N, G = 2, 50, 3, 4, 5, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=2)
    S0 = np.random.default_rng(3).standard_normal((Z, H, P, N))
    o = O.forward(inp, init_state=S0, parts=True, final_state=True)
    d = dense.forward(inp, init_state=S0)
    assert rel(o["y_f"], d["y_f"]) < 1e-12
    assert rel(o["y"], d["y"]) < 1e-12


# ----------------------------------------------------------- P2 closed form

@pytest.mark.parametrize("L", [1, 7, 130])
def test_closed_form_prefix_sums(L):
    """A = 0, B = C = e_0, dt = 1: the forward scan is a running sum, the
    reverse scan a running sum from the right, both exact in fp64."""
    Z, H, P, N, G = 2, 3, 4, 5, 1
    r = np.random.default_rng(L)
    inp = {"x": r.integers(-1, 2, (Z, L, H, P)).astype(np.float64),
           "D": np.array([0.0, 1.0, -2.0])}
    e0 = np.zeros((Z, L, G, N))
    e0[..., 0] = 1.0
    for d in ("f", "r"):
        inp[f"dt_{d}"] = np.ones((Z, L, H))
        inp[f"A_{d}"] = np.zeros(H)
        inp[f"B_{d}"] = e0
        inp[f"C_{d}"] = e0
    o = O.forward(inp, parts=True)
    x = inp["x"]
    cs = np.cumsum(x, axis=1)
    rcs = np.cumsum(x[:, ::-1], axis=1)[:, ::-1]
    assert np.array_equal(o["y_f"], cs)
    assert np.array_equal(o["y_r"], rcs)
    expect = x.sum(axis=1, keepdims=True) + x + inp["D"][None, None, :, None] * x
    assert np.array_equal(o["y"], expect)


# ------------------------------------------------------ P3 zero-decay limit

def test_every_decay_zero_leaves_the_diagonal_in_both_directions():
    Z, L, H, P, N, G = 2, 33, 3, 4, 6, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=4)
    inp["A_f"] = np.full(H, -1e30)
    inp["A_r"] = np.full(H, -1e30)
    o = O.forward(inp)
    cbf = np.einsum("zlgn,zlgn->zlg", inp["B_f"], inp["C_f"])[..., 0]
    cbr = np.einsum("zlgn,zlgn->zlg", inp["B_r"], inp["C_r"])[..., 0]
    coef = inp["dt_f"] * cbf[..., None] + inp["dt_r"] * cbr[..., None] + inp["D"]
    assert rel(o, coef[..., None] * inp["x"]) < 1e-14


# --------------------------------------------------------- P4 scipy filter

def test_scalar_case_is_a_first_order_iir_filter():
    L = 300
    r = np.random.default_rng(5)
    x = r.standard_normal(L)
    dtf, Af, dtr, Ar = 0.07, -2.5, 0.2, -0.9
    inp = {"x": x.reshape(1, L, 1, 1), "D": np.zeros(1),
           "dt_f": np.full((1, L, 1), dtf), "A_f": np.array([Af]),
           "dt_r": np.full((1, L, 1), dtr), "A_r": np.array([Ar]),
           "B_f": np.ones((1, L, 1, 1)), "C_f": np.ones((1, L, 1, 1)),
           "B_r": np.ones((1, L, 1, 1)), "C_r": np.ones((1, L, 1, 1))}
    o = O.forward(inp, parts=True)
    yf = scipy.signal.lfilter([dtf], [1.0, -math.exp(dtf * Af)], x)
    yr = scipy.signal.lfilter([dtr], [1.0, -math.exp(dtr * Ar)], x[::-1])[::-1]
    assert rel(o["y_f"].ravel(), yf) < 1e-13
    assert rel(o["y_r"].ravel(), yr) < 1e-13


# --------------------------------------------------------- P5 flip symmetry

def test_flip_swaps_the_two_directions():
    Z, L, H, P, N, G = 2, 45, 4, 3, 5, 2
    inp = rand_inputs(Z, L, H, P, N, G, seed=6)
    o = O.forward(inp, parts=True)
    fl = lambda a: a[:, ::-1].copy()  # noqa: E731
    sw = {"x": fl(inp["x"]), "D": inp["D"],
          "dt_f": fl(inp["dt_r"]), "A_f": inp["A_r"], "B_f": fl(inp["B_r"]), "C_f": fl(inp["C_r"]),
          "dt_r": fl(inp["dt_f"]), "A_r": inp["A_f"], "B_r": fl(inp["B_f"]), "C_r": fl(inp["C_f"])}
    s = O.forward(sw, parts=True)
    assert rel(s["y_f"], fl(o["y_r"])) < 1e-14
    assert rel(s["y_r"], fl(o["y_f"])) < 1e-14
    assert rel(s["y"], fl(o["y"])) < 1e-14


# ------------------------------------------------------------ P6 linearity

def test_linear_in_x():
    Z, L, H, P, N, G = 1, 40, 2, 3, 4, 1
    a = rand_inputs(Z, L, H, P, N, G, seed=7)
    b = dict(a)
    b["x"] = np.random.default_rng(8).standard_normal(a["x"].shape)
    c = dict(a)
    c["x"] = 0.75 * a["x"] - 1.5 * b["x"]
    ya, yb, yc = O.forward(a), O.forward(b), O.forward(c)
    assert rel(yc, 0.75 * ya - 1.5 * yb) < 1e-13


# ------------------------------------------------------------- P7 causality

@pytest.mark.parametrize("s", [0, 17, 63])
def test_impulse_respects_direction(s):
    Z, L, H, P, N, G = 1, 64, 2, 3, 4, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=9)
    inp["x"] = np.zeros_like(inp["x"])
    inp["x"][:, s] = 1.0
    o = O.forward(inp, parts=True)
    assert np.all(o["y_f"][:, :s] == 0.0)
    assert np.all(o["y_r"][:, s + 1:] == 0.0)
    assert np.all(o["y_f"][:, s:] != 0.0)
    assert np.all(o["y_r"][:, : s + 1] != 0.0)


# ----------------------------------------------------- P8 cache consistency

def test_block_update_reuses_the_prefix_state_exactly():
    """Scanning [prefix | block] forward equals continuing from the prefix's
    final state; the block's reverse scan sees the block only."""
    Z, Lp, Lb, H, P, N, G = 2, 70, 24, 3, 4, 5, 1
    full = rand_inputs(Z, Lp + Lb, H, P, N, G, seed=10)
    pre = {k: (v[:, :Lp] if v.ndim > 1 else v) for k, v in full.items()}
    blk = {k: (v[:, Lp:] if v.ndim > 1 else v) for k, v in full.items()}
    op = O.forward(pre, final_state=True)
    of = O.forward(full, parts=True, final_state=True)
    y, so = O.block_update(blk, op["final_state"])
    ob = O.forward(blk, parts=True)   # block-only scans (reverse part used)
    expect = of["y_f"][:, Lp:] + ob["y_r"] + blk["D"][None, None, :, None] * blk["x"]
    assert np.array_equal(y, expect)
    assert np.array_equal(so, of["final_state"])


def test_block_update_state_out_may_alias_state_in():
    Z, L, H, P, N, G = 1, 16, 2, 3, 4, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=11)
    S0 = np.random.default_rng(12).standard_normal((Z, H, P, N))
    y1, so1 = O.block_update(inp, S0.copy())
    d = dense.forward(inp, init_state=S0)
    assert rel(y1, d["y"]) < 1e-12


# ----------------------------------------------------- P10 backward pins

def _loss(inp, dy, S0=None):
    return float(np.sum(O.forward(inp, init_state=S0) * dy))


@pytest.mark.parametrize("shape", [(1, 20, 2, 3, 4, 1), (2, 33, 4, 3, 2, 2)])
def test_backward_matches_autograd_of_dense_form(shape):
    inp = rand_inputs(*shape, seed=13)
    dy = np.random.default_rng(14).standard_normal(inp["x"].shape)
    g = O.backward(inp, dy)
    ref = dense.gradients(inp, dy)
    for k in KEYS:
        assert rel(g["d" + k], ref["d" + k]) < 1e-11, k


def test_backward_with_start_state_matches_autograd():
    Z, L, H, P, N, G = 1, 150, 2, 3, 4, 1   # > 2 checkpoint segments
    inp = rand_inputs(Z, L, H, P, N, G, seed=15)
    S0 = np.random.default_rng(16).standard_normal((Z, H, P, N))
    dy = np.random.default_rng(17).standard_normal(inp["x"].shape)
    g = O.backward(inp, dy, init_state=S0)
    ref = dense.gradients(inp, dy, init_state=S0)
    for k in KEYS:
        assert rel(g["d" + k], ref["d" + k]) < 1e-11, k


def test_backward_finite_differences_tiny_fp32_shapes():
    """Central differences in fp64 on the tiny correctness shapes
    (L=128, 4 heads, P=64, N=64): a directional derivative per tensor."""
    Z, L, H, P, N, G = 1, 128, 4, 64, 64, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=18, dt_lo=1e-3, dt_hi=0.1)
    r = np.random.default_rng(19)
    dy = r.standard_normal(inp["x"].shape)
    g = O.backward(inp, dy)
    eps = 1e-6
    for k in KEYS:
        v = r.standard_normal(inp[k].shape)
        plus = dict(inp)
        minus = dict(inp)
        plus[k] = inp[k] + eps * v
        minus[k] = inp[k] - eps * v
        fd = (_loss(plus, dy) - _loss(minus, dy)) / (2 * eps)
        an = float(np.sum(g["d" + k] * v))
        assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (k, fd, an)


def test_backward_every_A_and_D_entry_by_finite_differences():
    Z, L, H, P, N, G = 2, 40, 3, 4, 5, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=20)
    dy = np.random.default_rng(21).standard_normal(inp["x"].shape)
    g = O.backward(inp, dy)
    eps = 1e-6
    for k in ("A_f", "A_r", "D"):
        for h in range(H):
            plus, minus = dict(inp), dict(inp)
            plus[k] = inp[k].copy()
            minus[k] = inp[k].copy()
            plus[k][h] += eps
            minus[k][h] -= eps
            fd = (_loss(plus, dy) - _loss(minus, dy)) / (2 * eps)
            assert abs(fd - g["d" + k][h]) <= 1e-7 * max(1.0, abs(fd)), (k, h)


def test_backward_dx_is_the_adjoint_of_the_dense_operator():
    Z, L, H, P, N, G = 2, 30, 3, 4, 5, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=22)
    dy = np.random.default_rng(23).standard_normal(inp["x"].shape)
    g = O.backward(inp, dy)
    for b in range(Z):
        for h in range(H):
            Mf, Mr = dense.matrices(inp, b, h)
            M = Mf + Mr + inp["D"][h] * np.eye(L)
            assert rel(g["dx"][b, :, h], M.T @ dy[b, :, h]) < 1e-12


# --------------------------------------------------- P11 permutations

def test_permuting_batch_rows_and_heads_permutes_outputs():
    Z, L, H, P, N, G = 3, 25, 4, 3, 4, 1
    inp = rand_inputs(Z, L, H, P, N, G, seed=24)
    y = O.forward(inp)
    pb = np.array([2, 0, 1])
    ph = np.array([3, 1, 0, 2])
    q = {}
    for k, v in inp.items():
        if k in ("A_f", "A_r", "D"):
            q[k] = v[ph]
        elif k.startswith(("B", "C")):
            q[k] = v[pb]
        elif k.startswith("dt"):
            q[k] = v[pb][:, :, ph]
        else:
            q[k] = v[pb][:, :, ph]
    yq = O.forward(q)
    assert np.array_equal(yq, y[pb][:, :, ph])


def test_thread_count_does_not_change_results():
    inp = rand_inputs(2, 50, 3, 4, 5, 1, seed=25)
    a = O.forward(inp, nthreads=1)
    b = O.forward(inp, nthreads=5)
    assert np.array_equal(a, b)
    dy = np.random.default_rng(26).standard_normal(inp["x"].shape)
    ga = O.backward(inp, dy, nthreads=1)
    gb = O.backward(inp, dy, nthreads=4)
    for k in ga:
        assert np.array_equal(ga[k], gb[k]), k


# ------------------------------------------- P12 block-segmented reverse

def _slice_tokens(inp, lo, hi):
    out = {}
    for k, v in inp.items():
        out[k] = v if k in ("A_f", "A_r", "D") else v[:, lo:hi]
    return out


@pytest.mark.parametrize("shape,rb", [((2, 37, 3, 5, 4, 1), 8), ((1, 130, 4, 8, 6, 2), 64),
                                      ((1, 64, 6, 3, 5, 3), 1), ((2, 40, 2, 3, 4, 1), 13)])
def test_segmented_reverse_matches_dense_block_mask(shape, rb):
    """The recurrence with restarts against the materialised reverse matrix
    with its cross-block entries removed."""
    inp = rand_inputs(*shape, seed=31)
    o = O.forward(inp, parts=True, rev_block=rb)
    d = dense.forward(inp, rev_block=rb)
    assert rel(o["y_f"], d["y_f"]) < 1e-12
    assert rel(o["y_r"], d["y_r"]) < 1e-12
    assert rel(o["y"], d["y"]) < 1e-12
    # the restarts change the result (the pin is not vacuous)
    assert rel(o["y_r"], O.forward(inp, parts=True)["y_r"]) > 1e-3


@pytest.mark.parametrize("L,rb", [(100, 16), (96, 32), (70, 70), (5, 2)])
def test_segmented_reverse_is_one_reverse_scan_per_block(L, rb):
    """Each block's reverse output equals a whole-sequence scan of that block
    alone, operation for operation; the forward direction is untouched."""
    inp = rand_inputs(2, L, 3, 4, 5, 1, seed=32)
    seg = O.forward(inp, parts=True, rev_block=rb)
    full = O.forward(inp, parts=True)
    assert np.array_equal(seg["y_f"], full["y_f"])
    for lo in range(0, L, rb):
        hi = min(lo + rb, L)
        blk = O.forward(_slice_tokens(inp, lo, hi), parts=True)
        assert np.array_equal(seg["y_r"][:, lo:hi], blk["y_r"]), lo


def test_reverse_block_longer_than_the_sequence_is_no_segmentation():
    inp = rand_inputs(1, 50, 2, 3, 4, 1, seed=33)
    dy = np.random.default_rng(34).standard_normal(inp["x"].shape)
    for rb in (50, 64, 1000):
        assert np.array_equal(O.forward(inp, rev_block=rb), O.forward(inp))
        ga, gb = O.backward(inp, dy, rev_block=rb), O.backward(inp, dy)
        for k in ga:
            assert np.array_equal(ga[k], gb[k]), (rb, k)


@pytest.mark.parametrize("shape,rb", [((1, 20, 2, 3, 4, 1), 6), ((2, 33, 4, 3, 2, 2), 8),
                                      ((1, 150, 2, 3, 4, 1), 64), ((1, 150, 2, 3, 4, 1), 37)])
def test_segmented_backward_matches_autograd_of_masked_dense_form(shape, rb):
    """L = 150 spans three checkpoint segments of the oracle's backward."""
    inp = rand_inputs(*shape, seed=35)
    S0 = np.random.default_rng(36).standard_normal((shape[0], shape[2], shape[3], shape[4]))
    dy = np.random.default_rng(37).standard_normal(inp["x"].shape)
    g = O.backward(inp, dy, init_state=S0, rev_block=rb)
    ref = dense.gradients(inp, dy, init_state=S0, rev_block=rb)
    for k in KEYS:
        assert rel(g["d" + k], ref["d" + k]) < 1e-11, k


def test_segmented_backward_reverse_gradients_come_block_by_block():
    """The reverse direction's parameter gradients of each block are those of
    that block alone (dA summed over blocks); the forward direction's are
    those of the unsegmented scan."""
    Z, L, H, P, N, G, rb = 2, 90, 3, 4, 5, 1, 32
    inp = rand_inputs(Z, L, H, P, N, G, seed=38)
    dy = np.random.default_rng(39).standard_normal(inp["x"].shape)
    seg = O.backward(inp, dy, rev_block=rb)
    full = O.backward(inp, dy)
    for k in ("ddt_f", "dA_f", "dB_f", "dC_f", "dD"):
        assert np.array_equal(seg[k], full[k]), k
    dA = np.zeros(H)
    for lo in range(0, L, rb):
        hi = min(lo + rb, L)
        blk = O.backward(_slice_tokens(inp, lo, hi), dy[:, lo:hi])
        for k in ("ddt_r", "dB_r", "dC_r"):
            assert rel(seg[k][:, lo:hi], blk[k]) < 1e-13, (k, lo)
        dA += blk["dA_r"]
    assert rel(seg["dA_r"], dA) < 1e-12


# ------------------------------------------------- P13 attention (hybrids)

from oracle import attention as AT


def _qkv(Z, L, H, D, seed):
    r = np.random.default_rng(seed)
    return (r.standard_normal((Z, L, H, D)), r.standard_normal((Z, L, H, D)),
            r.standard_normal((Z, L, H, D)))


def test_attention_zero_queries_average_the_visible_values():
    """Q = 0: every visible key scores the same, so each query gets the plain
    mean of the values it may see (full: all L; block-wise: blocks up to its own)."""
    Z, L, H, D = 2, 37, 3, 8
    _, k, v = _qkv(Z, L, H, D, 40)
    q = np.zeros_like(k)
    o = AT.forward(q, k, v)
    assert np.allclose(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), atol=1e-14)
    ob = AT.forward(q, k, v, block=8)
    for t in range(L):
        hi = (t // 8 + 1) * 8
        assert np.allclose(ob[:, t], v[:, :min(hi, L)].mean(axis=1), atol=1e-14), t


def test_attention_sharp_scores_select_one_value():
    """Keys equal to large multiples of orthonormal directions and each query
    along one of them: the softmax is one-hot (to fp64 precision) on that key."""
    Z, L, H, D = 1, 16, 2, 16
    r = np.random.default_rng(41)
    basis = np.linalg.qr(r.standard_normal((D, D)))[0]
    k = np.zeros((Z, L, H, D))
    v = r.standard_normal((Z, L, H, D))
    q = np.zeros((Z, L, H, D))
    perm = r.permutation(L)
    for h in range(H):
        k[0, :, h] = basis[:L] * 60.0
        q[0, :, h] = basis[perm] * 60.0
    o = AT.forward(q, k, v)
    for h in range(H):
        assert np.allclose(o[0, :, h], v[0, perm, h], atol=1e-12)


def test_attention_full_is_invariant_to_key_order_and_key_shift():
    """Full bidirectional attention: permuting keys with their values changes
    nothing, and adding one vector c to every key shifts all scores of a
    query by the same q.c, which the softmax removes."""
    Z, L, H, D = 2, 29, 2, 8
    q, k, v = _qkv(Z, L, H, D, 42)
    o = AT.forward(q, k, v)
    p = np.random.default_rng(43).permutation(L)
    assert np.allclose(AT.forward(q, k[:, p], v[:, p]), o, atol=1e-12)
    c = np.random.default_rng(44).standard_normal(D)
    assert np.allclose(AT.forward(q, k + c, v), o, atol=1e-12)


def test_attention_block_wise_is_full_attention_on_the_prefix():
    """A query of block i, block-wise, equals full attention over the tokens
    of blocks 0..i: the cache-consistency of block diffusion."""
    Z, L, H, D, blk = 1, 50, 2, 8, 16
    q, k, v = _qkv(Z, L, H, D, 45)
    o = AT.forward(q, k, v, block=blk)
    for i in range((L + blk - 1) // blk):
        hi = min((i + 1) * blk, L)
        full = AT.forward(q[:, :hi], k[:, :hi], v[:, :hi])
        assert np.allclose(o[:, i * blk:hi], full[:, i * blk:hi], rtol=0, atol=1e-13), i


def test_attention_single_token_and_scale():
    Z, L, H, D = 1, 1, 2, 4
    q, k, v = _qkv(Z, L, H, D, 46)
    assert np.allclose(AT.forward(q, k, v), v, atol=1e-15)
    # scale multiplies the scores: scale s on q is the same as s on the scores
    q, k, v = _qkv(1, 9, 1, 4, 47)
    assert np.allclose(AT.forward(q, k, v, scale=0.3), AT.forward(0.3 * q, k, v, scale=1.0), atol=1e-13)


def _attn_torch(q, k, v, block, scale):
    """The same layer through torch's own softmax, differentiated by autograd."""
    import torch
    Z, L, H, D = q.shape
    vis = torch.as_tensor(AT.visible(L, block))
    s = scale * torch.einsum("zthd,zshd->zhts", q, k)
    s = s.masked_fill(~vis, float("-inf"))
    return torch.einsum("zhts,zshd->zthd", torch.softmax(s, dim=-1), v)


@pytest.mark.parametrize("block", [0, 8, 16])
def test_attention_backward_matches_autograd(block):
    import torch
    Z, L, H, D = 2, 33, 2, 8
    q, k, v = _qkv(Z, L, H, D, 50)
    do = np.random.default_rng(51).standard_normal((Z, L, H, D))
    g = AT.backward(q, k, v, do, block=block)
    T = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v)]
    o = _attn_torch(*T, block, 1.0 / math.sqrt(D))
    assert np.allclose(o.detach().numpy(), AT.forward(q, k, v, block=block), atol=1e-13)
    (o * torch.tensor(do)).sum().backward()
    for name, t in zip(("dq", "dk", "dv"), T):
        assert rel(g[name], t.grad.numpy()) < 1e-12, name


def test_attention_backward_finite_differences():
    Z, L, H, D = 1, 20, 1, 8
    q, k, v = _qkv(Z, L, H, D, 52)
    do = np.random.default_rng(53).standard_normal((Z, L, H, D))
    g = AT.backward(q, k, v, do, block=8)
    r = np.random.default_rng(54)
    eps = 1e-6
    for name, idx in (("dq", 0), ("dk", 1), ("dv", 2)):
        d = r.standard_normal((Z, L, H, D))
        args_p = [q, k, v]
        args_m = [q, k, v]
        args_p[idx] = args_p[idx] + eps * d
        args_m[idx] = args_m[idx] - eps * d
        fd = (np.sum(AT.forward(*args_p, block=8) * do) - np.sum(AT.forward(*args_m, block=8) * do)) / (2 * eps)
        assert abs(fd - np.sum(g[name] * d)) <= 1e-7 * max(1.0, abs(fd)), name


# ------------------------------------------- P14 dt post-processing

from oracle import dt_act as DTA


def _with_dt_act(inp, seed, lo=1e-3, hi=0.1):
    """Pre-activation dt ~ N(0, 1) with per-head biases around -4 (the
    synthetic dt recipe's shift) and the recipe's clamp."""
    r = np.random.default_rng(seed)
    out = dict(inp)
    Z, L, H = inp["dt_f"].shape
    for d in ("f", "r"):
        out[f"dt_{d}"] = r.standard_normal((Z, L, H))
        out[f"dt_bias_{d}"] = -4.0 + 0.5 * r.standard_normal(H)
        out[f"dt_min_{d}"], out[f"dt_max_{d}"] = lo, hi
    return out


def test_dt_post_processing_reduces_to_the_plain_scan():
    """Feeding softplus^{-1}(dt) - bias with no clamp reproduces the scan
    of dt itself."""
    inp = rand_inputs(2, 40, 3, 4, 5, 1, seed=60)
    q = dict(inp)
    r = np.random.default_rng(61)
    for d in ("f", "r"):
        b = r.standard_normal(3)
        q[f"dt_bias_{d}"] = b
        q[f"dt_{d}"] = np.log(np.expm1(inp[f"dt_{d}"])) - b[None, None, :]
    assert rel(O.forward(q), O.forward(inp)) < 1e-12


def test_dt_post_processing_clamps():
    inp = _with_dt_act(rand_inputs(1, 30, 2, 3, 4, 1, seed=62), 63)
    eff = DTA.effective(inp)
    for d in ("f", "r"):
        assert eff[f"dt_{d}"].min() >= 1e-3 and eff[f"dt_{d}"].max() <= 0.1
        assert np.any(eff[f"dt_{d}"] == 1e-3) or np.any(eff[f"dt_{d}"] == 0.1)


@pytest.mark.parametrize("rb", [0, 8])
def test_dt_post_processing_backward_matches_autograd(rb):
    """Chain rule through softplus and clamp (and dbias) against autograd of
    the dense form with torch's softplus and clamp."""
    inp = _with_dt_act(rand_inputs(2, 24, 3, 3, 4, 1, seed=64), 65)
    dy = np.random.default_rng(66).standard_normal(inp["x"].shape)
    g = O.backward(inp, dy, rev_block=rb)
    ref = dense.gradients(inp, dy, rev_block=rb)
    for k in list(KEYS) + ["dt_bias_f", "dt_bias_r"]:
        assert rel(g["d" + k], ref["d" + k]) < 1e-11, k
    assert np.any(g["ddt_f"] == 0.0)  # clamped tokens pass no gradient


def test_dt_post_processing_at_the_exact_clamp_bounds():
    """The clamp range chosen as softplus(-7) and softplus(-2) (fp64), and
    pre-activations placed exactly on those points (raw -7.5 and -2.5 with
    bias 0.5, sums exact in fp64): the step is the bound itself and the
    gradient passes (ends included); just beyond either point the step is
    held at the bound and no gradient passes."""
    lo, hi = float(np.logaddexp(0.0, -7.0)), float(np.logaddexp(0.0, -2.0))
    eps = 2.0 ** -30
    raw = np.array([-7.5, -2.5, -7.5 - eps, -2.5 + eps, -5.0]).reshape(1, 5, 1)
    bias = np.array([0.5])
    dt = DTA.forward(raw, bias, lo, hi).ravel()
    assert dt[0] == lo and dt[1] == hi
    assert dt[2] == lo and dt[3] == hi
    assert lo < dt[4] < hi
    ddt = np.full((1, 5, 1), 3.0)
    draw, dbias = DTA.backward(raw, bias, lo, hi, ddt)
    z = raw.ravel() + 0.5
    sig = 1.0 / (1.0 + np.exp(-z))
    assert draw.ravel()[0] == 3.0 * sig[0] and draw.ravel()[1] == 3.0 * sig[1]
    assert draw.ravel()[2] == 0.0 and draw.ravel()[3] == 0.0
    assert draw.ravel()[4] == 3.0 * sig[4]
    assert dbias[0] == draw.sum()


def test_dt_post_processing_forward_and_backward_take_one_decision():
    """Over pre-activations spread across both bounds, the gradient passes
    exactly where the clamped step equals the unclamped softplus."""
    r = np.random.default_rng(67)
    raw = r.uniform(-9.0, 0.0, (2, 500, 3))
    bias = r.standard_normal(3)
    lo, hi = 1e-3, 0.1
    dt = DTA.forward(raw, bias, lo, hi)
    draw, _ = DTA.backward(raw, bias, lo, hi, np.ones_like(raw))
    free = dt == np.logaddexp(0.0, raw + bias[None, None, :])
    assert np.array_equal(free, draw != 0.0)
    assert 0 < free.sum() < free.size


def test_synthetic_pre_activations_keep_clear_of_the_clamp_edges():
    """The test inputs hold no pre-activation within the band around either
    point where the clamp engages (there the in-range decision depends on the
    precision softplus is formed in), in either dtype."""
    from synth import gen as G
    for dtype in ("fp32", "bf16"):
        w = G.WORKLOADS["tiny_fp32"].replace(Z=4, L=1000, H=6, dtype=dtype)
        inp = G.with_dt_post(G.make_inputs(w), w)
        for d in ("f", "r"):
            z = inp[f"dt_{d}"] + inp[f"dt_bias_{d}"][None, None, :]
            assert np.array_equal(G.quantize(inp[f"dt_{d}"], dtype), inp[f"dt_{d}"])
            for edge in (1e-3, 0.1):
                ze = np.log(np.expm1(edge))
                assert np.min(np.abs(z - ze)) >= G.CLAMP_EDGE_BAND
    # a value placed on an edge is moved off it, to a representable value
    raw = np.full((1, 1, 1), np.log(np.expm1(0.1)) - 0.25)
    moved = G.off_clamp_edges(G.round_fp32(raw), np.array([0.25]), 1e-3, 0.1, "fp32")
    assert abs(moved[0, 0, 0] + 0.25 - np.log(np.expm1(0.1))) >= 2 * G.CLAMP_EDGE_BAND


# ---------------------------------------------------------------- the conv

from oracle import conv as CV  # noqa: E402


def _conv_params(H, P, K, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((H, P, K)) * 0.5, r.standard_normal((H, P)) * 0.1


@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_is_numpy_convolve_per_channel(K):
    """Forward: the full discrete convolution with the taps reversed,
    truncated to the sequence (numpy.convolve); reverse: the same of the
    flipped sequence, flipped back.  No bias or activation."""
    r = np.random.default_rng(70 + K)
    x = r.standard_normal((2, 37, 3, 4))
    w, _ = _conv_params(3, 4, K, 71)
    cf = CV.conv(x, w, None, "f", act=False)
    cr = CV.conv(x, w, None, "r", act=False)
    for z in range(2):
        for h in range(3):
            for p in range(4):
                v = w[h, p, ::-1]
                assert np.allclose(cf[z, :, h, p], np.convolve(x[z, :, h, p], v)[:37], rtol=0, atol=1e-13)
                assert np.allclose(cr[z, :, h, p], np.convolve(x[z, ::-1, h, p], v)[:37][::-1], rtol=0, atol=1e-13)


def test_conv_activation_is_silu():
    from scipy.special import expit
    r = np.random.default_rng(72)
    x = r.standard_normal((1, 20, 2, 3))
    w, b = _conv_params(2, 3, 4, 73)
    pre = CV.conv(x, w, b, "f", act=False)
    assert np.allclose(CV.conv(x, w, b, "f"), pre * expit(pre), rtol=1e-14, atol=0)


def test_conv_identity_taps_leave_the_plain_scan():
    """Width 1 with tap 1, no bias, no activation: both directions read x."""
    inp = rand_inputs(2, 50, 3, 4, 5, 1, seed=74)
    one = (np.ones((3, 4, 1)), None, False)
    assert rel(CV.forward(inp, {"f": one, "r": one}), O.forward(inp)) < 1e-13


@pytest.mark.parametrize("K", [2, 4])
def test_conv_state_continues_the_prefix_and_the_reverse_stays_in_the_block(K):
    r = np.random.default_rng(75)
    x = r.standard_normal((2, 30, 2, 3))
    w, b = _conv_params(2, 3, K, 76)
    full_f = CV.conv(x, w, b, "f")
    blk_f = CV.conv(x[:, 20:], w, b, "f", state=x[:, 20 - (K - 1):20])
    assert np.array_equal(full_f[:, 20:], blk_f)
    assert np.array_equal(CV.next_state(x[:, 20:], x[:, 20 - (K - 1):20], K), x[:, 30 - (K - 1):])
    # a block shorter than the state: the state shifts by the block
    st = x[:, :K - 1]
    assert np.array_equal(CV.next_state(x[:, K - 1:K], st, K), x[:, 1:K])
    # reverse of the block alone == reverse with the sequence ending at the block
    assert np.array_equal(CV.conv(x[:, 20:], w, b, "r"), CV.conv(x, w, b, "r")[:, 20:])
    # block-segmented reverse: each block alone
    seg = CV.conv(x, w, b, "r", rev_block=8)
    for k0 in range(0, 30, 8):
        assert np.array_equal(seg[:, k0:k0 + 8], CV.conv(x[:, k0:k0 + 8], w, b, "r"))


def test_conv_block_update_is_the_full_scan_restricted_to_the_block():
    """Cache consistency with the convolution: the forward part of the scan
    over [prefix | block] restricted to the block equals the block update
    continuing the prefix's final state and conv state; the reverse part
    equals the scan of the block alone."""
    Lp, Lb, K = 40, 16, 4
    inp = rand_inputs(2, Lp + Lb, 3, 4, 5, 1, seed=77)
    wf, bf = _conv_params(3, 4, K, 78)
    wr, br = _conv_params(3, 4, K, 79)
    convs = {"f": (wf, bf, True), "r": (wr, br, True)}
    pre = {k: (v[:, :Lp] if v.ndim > 1 else v) for k, v in inp.items()}
    blk = {k: (v[:, Lp:] if v.ndim > 1 else v) for k, v in inp.items()}
    # forward-only and reverse-only views (D = 0 and the other C = 0)
    fwd_only = lambda q: {**q, "C_r": np.zeros_like(q["C_r"]), "D": np.zeros_like(q["D"])}  # noqa: E731
    rev_only = lambda q: {**q, "C_f": np.zeros_like(q["C_f"]), "D": np.zeros_like(q["D"])}  # noqa: E731
    xcf_pre = CV.conv(pre["x"], wf, bf, "f")
    S = O.forward({**fwd_only(pre), "x": xcf_pre}, final_state=True)["final_state"]
    cst = pre["x"][:, Lp - (K - 1):]
    yb, so, cso = CV.block_update(fwd_only(blk), convs, S, conv_state=cst)
    assert rel(yb, CV.forward(fwd_only(inp), convs)[:, Lp:]) < 1e-12
    yr, _, _ = CV.block_update(rev_only(blk), convs, S, conv_state=cst)
    assert rel(yr, CV.forward(rev_only(blk), convs)) < 1e-12
    full_S = O.forward({**fwd_only(inp), "x": CV.conv(inp["x"], wf, bf, "f")}, final_state=True)["final_state"]
    assert rel(so, full_S) < 1e-12
    assert np.array_equal(cso, inp["x"][:, -(K - 1):])
