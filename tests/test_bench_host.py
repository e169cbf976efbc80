"""Host-side checks of bench.py's bookkeeping (no GPU): the one-GPU guard,
and the algorithmic byte and flop counts its roofline lines divide by,
against independent hand derivations or brute force."""
import os
import subprocess
import sys

import bench
from synth import gen

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_algorithmic_bytes_of_the_layer_workload():
    # bf16: x and y 1536 values each, dt 24 per direction, B and C 128 per
    # direction: 2 * 3072 + 2 * 48 + 4 * 256 bytes per token
    w = gen.WORKLOADS["layer130m_L1k"]
    assert bench.per_token_bytes(w) == 7264
    assert bench.per_token_bytes(w) * w.tokens == 59506688


def test_training_bytes_add_the_backward_streams():
    w = gen.WORKLOADS["train_L2k"]
    fwd = bench.per_token_bytes(w)
    # the backward reads x, dy (bf16), dt and B/C again and writes dx (fp32),
    # ddt (fp32, both directions) and dB/dC (fp32, both directions)
    bwd = 2 * 1536 * 2 + 2 * 24 * 2 + 4 * 128 * 2 + 1536 * 4 + 2 * 24 * 4 + 4 * 128 * 4
    assert bench.train_bytes_per_token(w) == fwd + bwd


def test_output_kernel_flops_count_causal_pairs():
    # per head and direction: 2 P flops for each of the Q (Q + 1) / 2 causal
    # (t, s) pairs of a chunk, spread over Q tokens, plus the carry-in
    # product 2 N P per token
    w = gen.WORKLOADS["layer130m_L1k"]
    Q, P, N, H = w.chunk, w.P, w.N, w.H
    pairs = sum(t + 1 for t in range(Q))
    per_token = 2 * H * (2 * P * pairs / Q + 2 * N * P)
    assert bench.k3_flops_per_token(w) == per_token
    assert bench.k3_flops_per_token(w) * w.tokens == 12910067712


def test_attention_pairs_by_brute_force():
    for L, block in ((200, 0), (200, 64), (256, 64), (130, 128)):
        pairs = sum(1 for t in range(L) for s in range(L) if block == 0 or s // block <= t // block)
        assert bench.attention_flops(2, L, 3, block) == 4 * 2 * 3 * 64 * pairs
