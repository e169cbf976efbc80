"""GPU parity of the hybrids' attention layer (bissd_attention_forward)
against the fp64 oracle (oracle/attention.py), element by element on the same
seeded inputs: full bidirectional and block-wise masks, ragged lengths that
leave partial query and key tiles, one-token sequences, and the training /
inference layer shape of the 130M-class hybrids (12 heads of 64).
Tolerance: max|gpu - oracle| / max|oracle| <= 1e-4 (fp32), 2e-2 (bf16).
"""
import numpy as np
import pytest
import torch

from oracle import attention as AT
from synth import gen
from tests.gpu_util import TOL, device, host, maxrel

pytestmark = pytest.mark.gpu


def run(Z, L, H, dtype, block=0, scale=0.0, seed=7):
    import state_space_denoisers_amd as ssd
    inp = gen.make_attention_inputs(Z, L, H, dtype, seed)
    T = {k: gen.as_torch(v, dtype, device()) for k, v in inp.items()}
    o = ssd.bissd_attention_forward(T["q"], T["k"], T["v"], block=block, scale=scale)
    torch.cuda.synchronize()
    ref = AT.forward(inp["q"], inp["k"], inp["v"], block=block, scale=scale if scale > 0 else None)
    e = maxrel(host(o), ref)
    print(f"attn {dtype} Z={Z} L={L} H={H} block={block} err={e:.1e}", flush=True)
    return e


@pytest.mark.parametrize("L", [1, 63, 64, 65, 200, 513])
@pytest.mark.parametrize("block", [0, 64, 128])
def test_fp32_lengths_and_masks(L, block):
    assert run(2, L, 3, "fp32", block) <= TOL["fp32"]


@pytest.mark.parametrize("block", [0, 128])
def test_bf16_hybrid_layer(block):
    """12 heads of 64 at L = 1024 (the 130M-class hybrids), two batch rows."""
    assert run(2, 1024, 12, "bf16", block) <= TOL["bf16"]


def test_bf16_ragged_long():
    assert run(1, 2500, 4, "bf16", 0) <= TOL["bf16"]


def test_explicit_scale():
    assert run(1, 300, 2, "fp32", 0, scale=0.37) <= TOL["fp32"]


def test_block_wise_matches_full_attention_on_each_prefix():
    """The block-wise output of a block equals full attention over the
    sequence cut after that block (computed by the same kernel): the keys
    past the block are really invisible."""
    import state_space_denoisers_amd as ssd
    Z, L, H, blk = 1, 320, 2, 64
    inp = gen.make_attention_inputs(Z, L, H, "fp32", 9)
    T = {k: gen.as_torch(v, "fp32", device()) for k, v in inp.items()}
    ob = host(ssd.bissd_attention_forward(T["q"], T["k"], T["v"], block=blk))
    for i in range(L // blk):
        hi = (i + 1) * blk
        part = {k: v[:, :hi].contiguous() for k, v in T.items()}
        of = host(ssd.bissd_attention_forward(part["q"], part["k"], part["v"]))
        assert np.array_equal(ob[:, i * blk:hi], of[:, i * blk:hi]), i


def run_bwd(Z, L, H, dtype, block=0, seed=11):
    import state_space_denoisers_amd as ssd
    inp = gen.make_attention_inputs(Z, L, H, dtype, seed)
    dout = gen.make_attention_inputs(Z, L, H, dtype, seed + 1)["q"]
    T = {k: gen.as_torch(v, dtype, device()) for k, v in inp.items()}
    G = gen.as_torch(dout, dtype, device())
    lse = torch.empty((Z, H, L), dtype=torch.float32, device=device())
    o = ssd.bissd_attention_forward(T["q"], T["k"], T["v"], block=block, lse=lse)
    g = ssd.bissd_attention_backward(T["q"], T["k"], T["v"], o, G, lse, block=block)
    torch.cuda.synchronize()
    ref = AT.backward(inp["q"], inp["k"], inp["v"], dout, block=block)
    errs = {n: maxrel(host(g[n]), ref[n]) for n in ("dq", "dk", "dv")}
    print(f"attn bwd {dtype} Z={Z} L={L} H={H} block={block} " +
          " ".join(f"{n}={e:.1e}" for n, e in errs.items()), flush=True)
    return errs


@pytest.mark.parametrize("L", [1, 63, 65, 200, 513])
@pytest.mark.parametrize("block", [0, 64, 128])
def test_backward_fp32(L, block):
    errs = run_bwd(2, L, 3, "fp32", block)
    assert max(errs.values()) <= TOL["fp32"], errs


@pytest.mark.parametrize("block", [0, 256])
def test_backward_bf16_hybrid_layer(block):
    errs = run_bwd(2, 1024, 12, "bf16", block)
    assert max(errs.values()) <= TOL["bf16"], errs


def test_backward_deterministic():
    import state_space_denoisers_amd as ssd
    Z, L, H = 1, 700, 4
    inp = gen.make_attention_inputs(Z, L, H, "bf16", 13)
    T = {k: gen.as_torch(v, "bf16", device()) for k, v in inp.items()}
    lse = torch.empty((Z, H, L), dtype=torch.float32, device=device())
    o = ssd.bissd_attention_forward(T["q"], T["k"], T["v"], lse=lse)
    a = ssd.bissd_attention_backward(T["q"], T["k"], T["v"], o, T["v"], lse)
    b = ssd.bissd_attention_backward(T["q"], T["k"], T["v"], o, T["v"], lse)
    for n in a:
        assert torch.equal(a[n], b[n]), n
