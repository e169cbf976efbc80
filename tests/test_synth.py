"""The seeded input generator: determinism, rounding and distributions."""
import numpy as np
import torch

from synth import gen


def test_round_bf16_matches_torch_round_to_nearest_even():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000) * 10.0 ** r.integers(-6, 6, 100000),
                        [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e-3]])
    a32 = a.astype(np.float32)
    ours = gen.round_bf16(a32.astype(np.float64))
    ref = torch.from_numpy(a32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_round_bf16_ties_go_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: even mantissa is 1.0
    assert gen.round_bf16(1.0 + 2.0 ** -8) == 1.0
    # 1 + 3 * 2^-8 lies halfway between 1 + 2^-7 and 1 + 2^-6: goes to 1 + 2^-6
    assert gen.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6


def test_inputs_are_deterministic_and_representable():
    w = gen.WORKLOADS["tiny_fp32"]
    a = gen.make_inputs(w)
    b = gen.make_inputs(w)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
        assert np.array_equal(a[k], a[k].astype(np.float32).astype(np.float64)), k
    wb = w.replace(dtype="bf16")
    c = gen.make_inputs(wb)
    for k in ("x", "dt_f", "B_r", "C_f"):
        assert np.array_equal(c[k], gen.round_bf16(c[k])), k


def test_distributions():
    w = gen.WORKLOADS["layer130m_L1k"].replace(Z=2)
    inp = gen.make_inputs(w)
    for d in ("f", "r"):
        dt = inp[f"dt_{d}"]
        assert dt.min() >= gen.round_bf16(1e-3) and dt.max() <= gen.round_bf16(0.1)
        assert 0.01 < np.median(dt) < 0.03
        A = inp[f"A_{d}"]
        assert A.min() >= -16.0 and A.max() <= -1.0
        assert abs(inp[f"B_{d}"].std() * np.sqrt(w.N) - 1.0) < 0.02
    assert abs(inp["x"].std() - 1.0) < 0.01
    assert not np.array_equal(inp["dt_f"], inp["dt_r"])


def test_check_modes_zero_the_right_tensors():
    w = gen.WORKLOADS["tiny_fp32"]
    f = gen.make_inputs(w, mode="fwd")
    assert not f["C_r"].any() and not f["D"].any() and f["C_f"].any()
    r = gen.make_inputs(w, mode="rev")
    assert not r["C_f"].any() and r["C_r"].any()


def test_block_workload_mask_positions():
    w = gen.WORKLOADS["block_update"]
    inp = gen.make_inputs(w)
    m = inp["mask_vec"]
    for b in range(w.Z):
        hits = [np.array_equal(inp["x"][b, t], m) for t in range(w.L)]
        assert sum(hits) == w.mask_count
    assert 0.07 < m.std() < 0.13
