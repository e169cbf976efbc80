#!/usr/bin/env python3
"""Throughput of the bidirectional SSD (Mamba-2) scan on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one bissd_forward call (chunk states -> carry pass -> fused
bidirectional output) over the 130M-class layer workload: batch 8, L=1024,
24 heads x head dim 64, d_state 128, one B/C group, chunk 256, bf16 inputs
with fp32 accumulation, synthetic seeded inputs already resident in HBM.
Untimed calls for --settle seconds (default 0.5: a GPU that has been idle
runs its first milliseconds of work below its sustained clocks), W untimed
warm-up steps, then exactly K timed steps between two device
synchronisations; `value` is tokens per second over the timed region.

The same run also measures, live with HIP events on the launch stream, the
average duration of each forward kernel (each launch's own dispatch start
and end, in complete forward calls enqueued through bissd_forward_phase), the
long-context L=65536 scan, the training step (forward + backward, batch 16,
L=2048), the block update with a cached 262,144-token prefix state, the
generation loop, a latency sweep and the hybrids' attention layer; and times
the fp64 CPU oracle on a bounded sample of the same workload.  One JSON line
is printed.

Profiling helpers (for rocprofv3 runs):
    python bench.py --profile-phase {0,1,2,3,all,conv,train,backward,block,attention} [--workload W]
        [--iters R] [--settle S]   (S seconds of a bf16 matrix product first)
    python bench.py --copy-calibrate
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "bidir SSD scan tokens/s at L=1K/65K; achieved HBM GB/s and MFMA %"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
PHASE_NAMES = {0: "k1_chunk_state", 3: "k_gram", 1: "k2_state_pass", 2: "k3_chunk_out"}
PHASE_ORDER = (0, 3, 1, 2)   # the order bissd_forward runs them in
KERNEL_SOURCES = ("state_space_denoisers_amd/csrc/bissd_fwd.hip",
                  "state_space_denoisers_amd/csrc/bissd_conv.hip",
                  "state_space_denoisers_amd/csrc/bissd_device.hpp",
                  "state_space_denoisers_amd/csrc/bissd_internal.hpp")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ inputs

def device_inputs(w, mode="full"):
    import torch
    from synth import gen
    inp = gen.make_inputs(w, mode=mode)
    dev = torch.device("cuda", 0)
    T = {k: gen.as_torch(inp[k], w.dtype, dev) for k in
         ("x", "dt_f", "B_f", "C_f", "dt_r", "B_r", "C_r")}
    for k in ("A_f", "A_r", "D"):
        T[k] = gen.as_torch(inp[k], "fp32", dev)
    return inp, T


def dirs(T):
    return ((T["dt_f"], T["A_f"], T["B_f"], T["C_f"]),
            (T["dt_r"], T["A_r"], T["B_r"], T["C_r"]))


class Forward:
    """Preallocated forward call on one workload (rev_block > 0: the
    block-segmented reverse of full-block training)."""

    def __init__(self, w, rev_block=0):
        import torch
        import state_space_denoisers_amd as ssd
        from state_space_denoisers_amd import _abi
        self.ssd, self.w, self.rb = ssd, w, rev_block
        self.inp, self.T = device_inputs(w)
        self.fwd, self.rev = dirs(self.T)
        self.y = torch.empty_like(self.T["x"])
        shape = ssd.shape_of(self.T["x"], self.T["B_f"], w.chunk, rev_block)
        n = ssd.bissd_workspace_size(shape, _abi.OP_FORWARD)
        self.ws = torch.empty(n, dtype=torch.uint8, device=self.y.device)

    def __call__(self):
        self.ssd.bissd_forward(self.T["x"], self.fwd, self.rev, self.T["D"], chunk=self.w.chunk,
                               rev_block=self.rb, y=self.y, workspace=self.ws)

    def phase(self, p):
        self.ssd.bissd_forward_phase(p, self.T["x"], self.fwd, self.rev, self.T["D"],
                                     chunk=self.w.chunk, rev_block=self.rb, y=self.y,
                                     workspace=self.ws)


# ----------------------------------------------------------------- timing

def event_time_ms(fn, reps):
    """Average ms per call of fn over reps calls, HIP events on the current
    stream (the stream every library launch goes to)."""
    import torch
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for _ in range(reps):
        fn()
    b.record(s)
    b.synchronize()
    return a.elapsed_time(b) / reps


def gram_in_chunk_state_kernel(w) -> bool:
    """The chunk-state kernel forms the Gram tiles itself (and phase 3
    launches nothing) when every B/C group has a head tile per (row-block,
    column-block) pair: the rule documented with bissd_forward_phase."""
    hpg = w.H // w.G
    ht = 2 if hpg % 2 == 0 else 1
    nrb = w.chunk // 64
    return hpg // ht >= nrb * (nrb + 1) // 2


def phase_times_us(f: Forward, reps):
    """Average duration of each forward kernel inside complete forward calls
    (the kernels in the call's order, each after the same predecessors):
    before each kernel's launch a library timer slot is armed, so that launch
    records its own dispatch start and end in a pair of HIP events on its
    stream (bissd_timer_arm / bissd_timer_read), with no marker between the
    kernels; the durations are averaged over reps calls."""
    import torch
    ssd = f.ssd
    f()
    torch.cuda.synchronize()
    order = [p for p in PHASE_ORDER if not (p == 3 and gram_in_chunk_state_kernel(f.w))]
    names = dict(PHASE_NAMES)
    if 3 not in order:
        names[0] = "k1_chunk_state+gram"
    reps = min(reps, ssd.TIMER_SLOTS // len(order))
    for r in range(reps):
        for i, p in enumerate(order):
            ssd.bissd_timer_arm(r * len(order) + i)
            f.phase(p)
    ssd.bissd_timer_arm(-1)
    torch.cuda.synchronize()
    out = {}
    for i, p in enumerate(order):
        out[names[p]] = 1e3 * sum(ssd.bissd_timer_read(r * len(order) + i) for r in range(reps)) / reps
    return out


def state_pass_line(w, ph):
    """The carry pass (the memory-bound scan phase): its live average
    duration and its HBM bytes per launch from the committed counter runs
    (FETCH_SIZE + WRITE_SIZE, calibrated; null when they were taken on
    other kernel sources), against the 8 TB/s peak."""
    us = ph.get(PHASE_NAMES[1])
    if us is None:
        return None
    traffic = stored_traffic(PHASE_NAMES[1], w.name)
    out = {"kernel": PHASE_NAMES[1], "avg_launch_us": round(us, 2), "traffic": traffic,
           "unit": "GB/s", "peak": HBM_PEAK_GBS}
    if traffic:
        gbs = traffic / (us * 1e-6) / 1e9
        out.update({"achieved_by_counters": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)})
    return out


def per_token_bytes(w):
    """Algorithmic HBM bytes per token of the whole path: read x, dt and
    B/C of both directions once, write y once."""
    e = 2 if w.dtype == "bf16" else 4
    return 2 * w.H * w.P * e + 2 * w.H * e + 4 * w.G * w.N * e


def k3_flops_per_token(w):
    """Matrix-core work of the fused output kernel per token (both
    directions), on the method's causal work: per head the intra-chunk
    product of the decay-weighted C.B^T with x over the causal pairs of a
    chunk (Q (Q + 1) / 2 pairs per Q tokens, 2 P flops each) and the
    carry-in contraction C S^T (2 N P)."""
    intra = (w.chunk + 1) * w.P          # 2 P flops x (Q + 1) / 2 pairs per token
    inter = 2 * w.N * w.P
    return 2 * w.H * (intra + inter)


def gram_tiles_per_chunk(w):
    """16x64 Gram tiles one slot keeps per chunk (row tile tt needs column
    blocks 0..tt/4 on the causal side, tt/4..end on the other)."""
    qt, nrb = w.chunk // 16, w.chunk // 64
    return sum(tt // 4 + 1 for tt in range(qt)), nrb


def phase_bytes_per_token(w, phase):
    e = 2 if w.dtype == "bf16" else 4
    state_bytes = 2 * w.H * w.P * w.N * 4 / w.chunk   # both directions
    if phase == 0:
        return w.H * w.P * e + 2 * w.H * e + 2 * w.G * w.N * e + state_bytes
    if phase == 1:
        return 2 * state_bytes
    if phase == 3:
        tiles, _ = gram_tiles_per_chunk(w)
        return 2 * 2 * w.G * w.N * e + 2 * w.G * tiles * 16 * 64 * 4 / w.chunk
    return per_token_bytes(w)


def stored_traffic(kernel, workload):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "counters.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
        rec = d["kernels"][f"{kernel}@{workload}"]
        if rec.get("source_sha") != source_sha():
            return None
        return float(rec["fetch_bytes"] + rec["write_bytes"])
    except Exception:
        return None


# ------------------------------------------------------------ cpu baseline

def cpu_baseline(w, budget_s=12.0):
    from oracle import oracle as O
    from synth import gen
    inp = gen.make_inputs(w)
    n = int(os.environ.get("OMP_NUM_THREADS", "0") or 0) or O.thread_count(0)
    n = min(n, O.thread_count(0))
    reps, t0 = 0, time.perf_counter()
    while True:
        O.forward(inp, nthreads=n)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or el * (reps + 1) / reps > 30.0:
            break
    # one thread on one batch row of the same workload
    w1 = w.replace(Z=1)
    inp1 = gen.make_inputs(w1)
    t1 = time.perf_counter()
    O.forward(inp1, nthreads=1)
    el1 = time.perf_counter() - t1
    return {"value": reps * w.tokens / el, "unit": "tokens/s", "cores": n, "kind": "oracle",
            "sample": f"{reps} x the full {w.name} batch ({w.Z}x{w.L} tokens, 24 heads, both "
                      f"directions, fp64 sequential recurrence), {el:.1f} s wall",
            "value_1_thread": w1.tokens / el1,
            "sample_1_thread": f"one {w1.L}-token row of the same workload on 1 thread, {el1:.2f} s"}


# ------------------------------------------------------------ extra cases

def bench_long(steps):
    from synth import gen
    import torch
    w = gen.WORKLOADS["long_L65k"]
    f = Forward(w)
    for _ in range(2):
        f()
    torch.cuda.synchronize()
    settle(f, LEG_SETTLE_S)
    ms = event_time_ms(f, steps)
    ph = phase_times_us(f, max(3, steps // 2))
    return {"workload": w.name, "tokens_per_s": w.tokens / (ms * 1e-3), "ms_per_call": ms,
            "hbm_algorithmic_GBs": per_token_bytes(w) * w.tokens / (ms * 1e-3) / 1e9,
            "kernels_us": ph}


class ConvForward:
    """bissd_forward with the mixer's convolution on both directions (width
    K, bias, SiLU; taps and biases from gen.make_conv) on workload w."""

    def __init__(self, w, K=4):
        import torch
        import state_space_denoisers_amd as ssd
        from state_space_denoisers_amd import _abi
        from synth import gen
        self.ssd, self.w, self.K = ssd, w, K
        self.f = Forward(w)
        dev = self.f.y.device
        cv = gen.make_conv(w, K)
        self.convs = [ssd.Dir(*p, conv_w=gen.as_torch(cv[f"conv_w_{d}"], "fp32", dev),
                              conv_b=gen.as_torch(cv[f"conv_b_{d}"], "fp32", dev), conv_act=True)
                      for d, p in (("f", self.f.fwd), ("r", self.f.rev))]
        shape = ssd.shape_of(self.f.T["x"], self.f.T["B_f"], w.chunk, 0, K)
        self.ws = torch.empty(ssd.bissd_workspace_size(shape, _abi.OP_FORWARD), dtype=torch.uint8,
                              device=dev)

    def __call__(self):
        f = self.f
        self.ssd.bissd_forward(f.T["x"], self.convs[0], self.convs[1], f.T["D"], chunk=self.w.chunk,
                               y=f.y, workspace=self.ws)

    def x_bytes(self):
        x = self.f.T["x"]
        return x.numel() * x.element_size()


def bench_conv(steps, K=4):
    """The 130M-class layer forward with the mixer's convolution on both
    directions (width K, bias, SiLU): the convolution pass over x, then the
    scan on each direction's convolved x (the tokens/s of the whole call,
    against the same call without the convolution).  The convolution kernel
    is the call's first launch; its duration comes from a library timer on
    that dispatch, and its algorithmic bytes are x read once and the two
    directions' convolved x written (3 x-sized tensors)."""
    import torch
    from synth import gen
    w = gen.WORKLOADS["layer130m_L1k"]
    cf = ConvForward(w, K)
    ssd = cf.ssd
    for _ in range(2):
        cf()
    torch.cuda.synchronize()
    settle(cf, LEG_SETTLE_S)
    ms = event_time_ms(cf, steps)
    reps = min(steps, ssd.TIMER_SLOTS)
    for r in range(reps):
        ssd.bissd_timer_arm(r)
        cf()
    torch.cuda.synchronize()
    conv_us = 1e3 * sum(ssd.bissd_timer_read(r) for r in range(reps)) / reps
    settle(cf.f, LEG_SETTLE_S)
    ms0 = event_time_ms(cf.f, steps)
    alg = 3 * cf.x_bytes()
    return {"workload": w.name + f"_conv{K}", "tokens_per_s": w.tokens / (ms * 1e-3), "us_per_call": 1e3 * ms,
            "us_per_call_without_conv": 1e3 * ms0, "conv_kernel_us": round(conv_us, 2),
            "conv_algorithmic_bytes": alg, "conv_achieved_GBs": round(alg / (conv_us * 1e-6) / 1e9, 1),
            "conv_frac_hbm": round(alg / (conv_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}


def bench_block(reps):
    """Block update on Z=4 rows of a 64-token active block (16 mask-token
    positions per row) continuing from the forward state of a 262,144-token
    prefix.  The prefix is drawn on the device and its state computed by
    bissd_forward (final_state)."""
    import torch
    import state_space_denoisers_amd as ssd
    from synth import gen
    w = gen.WORKLOADS["block_update"]
    dev = torch.device("cuda", 0)
    inp, T = device_inputs(w)
    fwd, rev = dirs(T)
    pre = gen.prefix_on_device(w, w.prefix_len, dev)
    state = torch.empty((w.Z, w.H, w.P, w.N), dtype=torch.float32, device=dev)
    pf = (pre["dt_f"], T["A_f"], pre["B_f"], pre["C_f"])
    ssd.bissd_forward(pre["x"], pf, pf, T["D"], chunk=256, final_state=state)
    torch.cuda.synchronize()
    del pre
    y = torch.empty_like(T["x"])
    s_out = torch.empty_like(state)
    from state_space_denoisers_amd import _abi
    shape = ssd.shape_of(T["x"], T["B_f"], w.chunk)
    ws = torch.empty(max(256, ssd.bissd_workspace_size(shape, _abi.OP_BLOCK)),
                     dtype=torch.uint8, device=dev)

    def upd(commit):
        ssd.bissd_block_update(state, T["x"], fwd, rev, T["D"], chunk=w.chunk, y_blk=y,
                               state_out=s_out if commit else None, commit=commit, workspace=ws)

    out = {"workload": w.name, "prefix_tokens": w.prefix_len, "block_tokens": w.L, "batch": w.Z}
    # algorithmic bytes of one update: cached state read, x / y, dt and B / C
    # of both directions (and the state written back with commit)
    e = 2 if w.dtype == "bf16" else 4
    st_b = w.Z * w.H * w.P * w.N * 4
    blk_b = w.Z * w.L * (2 * w.H * w.P * e + 2 * w.H * e + 4 * w.G * w.N * e)
    per_graph = 50
    for commit in (False, True):
        for _ in range(5):
            upd(commit)
        torch.cuda.synchronize()
        settle(lambda: upd(commit), LEG_SETTLE_S)
        ms = event_time_ms(lambda: upd(commit), reps)
        key = "commit" if commit else "no_commit"
        # eager calls from Python: bounded by host submission for a call this small
        out[f"us_per_update_{key}"] = 1e3 * ms
        # device time: a captured HIP graph of 50 back-to-back updates
        g = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            upd(commit)
            torch.cuda.synchronize()
            with torch.cuda.graph(g, stream=s):
                for _ in range(per_graph):
                    upd(commit)
        torch.cuda.current_stream().wait_stream(s)
        g.replay()
        torch.cuda.synchronize()
        out[f"us_per_update_{key}_graph"] = 1e3 * event_time_ms(g.replay, max(5, reps // per_graph)) / per_graph
        nbytes = st_b * (2 if commit else 1) + blk_b
        out[f"algorithmic_bytes_{key}"] = nbytes
        out[f"effective_GBs_{key}_graph"] = nbytes / (out[f"us_per_update_{key}_graph"] * 1e-6) / 1e9
        del g
    return out


class Train:
    """Preallocated training step of the scan on one workload: the forward
    that keeps its chunk states, carry-ins, decays and Gram tiles for the
    backward (BISSD_SAVE), then the backward that reads them -- y, then every
    gradient of sum(dy * y).  ``backward_recompute`` is the backward that
    forms everything itself (no saving forward needed)."""

    def __init__(self, w, rev_block=0):
        import torch
        import state_space_denoisers_amd as ssd
        from state_space_denoisers_amd import _abi
        from synth import gen
        self.ssd, self.w, self.rb = ssd, w, rev_block
        self.f = Forward(w, rev_block)
        dev = self.f.y.device
        inp = gen.make_inputs(w, with_dy=True)
        self.dy = gen.as_torch(inp["dy"], w.dtype, dev)
        shape = ssd.shape_of(self.f.T["x"], self.f.T["B_f"], w.chunk, rev_block)
        n = ssd.bissd_workspace_size(shape, _abi.OP_BACKWARD)
        self.ws = torch.empty(n, dtype=torch.uint8, device=dev)
        self.grads = ssd.bissd_backward(self.f.T["x"], self.f.fwd, self.f.rev, self.f.T["D"],
                                        self.dy, chunk=w.chunk, rev_block=rev_block,
                                        workspace=self.ws)

    def forward(self):
        self.ssd.bissd_forward(self.f.T["x"], self.f.fwd, self.f.rev, self.f.T["D"],
                               chunk=self.w.chunk, rev_block=self.rb, y=self.f.y,
                               workspace=self.ws, save=True)

    def backward(self):
        """The saved backward: valid right after forward()."""
        self.ssd.bissd_backward(self.f.T["x"], self.f.fwd, self.f.rev, self.f.T["D"], self.dy,
                                chunk=self.w.chunk, rev_block=self.rb, grads=self.grads,
                                saved=self.ws)

    def backward_recompute(self):
        self.ssd.bissd_backward(self.f.T["x"], self.f.fwd, self.f.rev, self.f.T["D"], self.dy,
                                chunk=self.w.chunk, rev_block=self.rb, grads=self.grads,
                                workspace=self.ws)

    def __call__(self):
        self.forward()
        self.backward()


def train_bytes_per_token(w):
    """Algorithmic HBM bytes per token of forward + backward: the forward's
    reads and y write, then the backward reads x, dy, dt and B/C of both
    directions and writes dx, ddt, dB and dC (fp32 gradients)."""
    e = 2 if w.dtype == "bf16" else 4
    bwd = (2 * w.H * w.P * e + 2 * w.H * e + 4 * w.G * w.N * e
           + w.H * w.P * 4 + 2 * w.H * 4 + 4 * w.G * w.N * 4)
    return per_token_bytes(w) + bwd


def bench_train(steps, rev_block=0):
    """Forward + backward of the training workload; rev_block > 0 times the
    full-block objective (reverse restarting at every block of that many
    tokens)."""
    import torch
    from synth import gen
    w = gen.WORKLOADS["train_L2k"]
    t = Train(w, rev_block)
    for _ in range(3):
        t()
    torch.cuda.synchronize()
    settle(t, LEG_SETTLE_S)
    # the saved backward needs the saving forward before it, so its time is
    # the step's less the forward's
    ms_f = event_time_ms(t.forward, steps)
    ms = event_time_ms(t, steps)
    ms_r = event_time_ms(t.backward_recompute, steps)
    name = w.name + (f"_rev{rev_block}" if rev_block else "")
    return {"workload": name, "batch": w.Z, "seq_len": w.L, "rev_block": rev_block,
            "tokens_per_s": w.tokens / (ms * 1e-3),
            "ms_per_step": ms, "ms_forward": ms_f, "ms_backward": ms - ms_f,
            "ms_backward_recompute": ms_r, "ms_forward_plain": event_time_ms(t.f, steps),
            "hbm_algorithmic_GBs": train_bytes_per_token(w) * w.tokens / (ms * 1e-3) / 1e9}


def attention_flops(Z, L, H, block=0, D=64):
    """Matrix-core flops of one attention call: Q K^T and P V over the
    visible (query, key) pairs, 2 flops per multiply-add each."""
    if block <= 0:
        pairs = L * L
    else:
        pairs = sum(min(L, (t // block + 1) * block) for t in range(L))
    return 4 * Z * H * D * pairs


def bench_attention(reps, Z=8, L=1024, H=12, block=0):
    """The hybrids' attention layer at the 130M-class shape (12 heads of 64),
    bf16, full bidirectional (block 0) or block-wise."""
    import torch
    import state_space_denoisers_amd as ssd
    from synth import gen
    dev = torch.device("cuda", 0)
    inp = gen.make_attention_inputs(Z, L, H, "bf16", 2001)
    T = {k: gen.as_torch(v, "bf16", dev) for k, v in inp.items()}
    o = torch.empty_like(T["q"])
    fn = lambda: ssd.bissd_attention_forward(T["q"], T["k"], T["v"], block=block, o=o)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    settle(fn, LEG_SETTLE_S)
    ms = event_time_ms(fn, reps)
    fl = attention_flops(Z, L, H, block)
    return {"workload": f"attention_L{L // 1024}k" + (f"_block{block}" if block else ""),
            "batch": Z, "seq_len": L, "heads": H, "headdim": 64, "block": block,
            "us_per_call": ms * 1e3, "tokens_per_s": Z * L / (ms * 1e-3),
            "achieved_TFLOPs": fl / (ms * 1e-3) / 1e12,
            "frac_bf16_peak": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def bench_attention_backward(reps, Z=8, L=1024, H=12, block=0):
    """Backward of the attention layer (dq, dk, dv from the forward's o and
    lse); TFLOP/s over the algorithmic 5 products (Q K^T recomputed, dP,
    dV, dK, dQ; 10 L^2 D per head) on the visible pairs."""
    import torch
    import state_space_denoisers_amd as ssd
    from synth import gen
    dev = torch.device("cuda", 0)
    inp = gen.make_attention_inputs(Z, L, H, "bf16", 2002)
    T = {k: gen.as_torch(v, "bf16", dev) for k, v in inp.items()}
    dout = gen.as_torch(gen.make_attention_inputs(Z, L, H, "bf16", 2003)["q"], "bf16", dev)
    lse = torch.empty((Z, H, L), dtype=torch.float32, device=dev)
    o = ssd.bissd_attention_forward(T["q"], T["k"], T["v"], block=block, lse=lse)
    fn = lambda: ssd.bissd_attention_backward(T["q"], T["k"], T["v"], o, dout, lse, block=block)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    settle(fn, LEG_SETTLE_S)
    ms = event_time_ms(fn, reps)
    fl = attention_flops(Z, L, H, block) * 10 // 4
    return {"workload": f"attention_bwd_L{L // 1024}k" + (f"_block{block}" if block else ""),
            "batch": Z, "seq_len": L, "heads": H, "headdim": 64, "block": block,
            "us_per_call": ms * 1e3, "achieved_TFLOPs": fl / (ms * 1e-3) / 1e12,
            "frac_bf16_peak": fl / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS}


def bench_latency_sweep(lengths=(1024, 4096, 16384, 65536, 262144)):
    """Forward latency of one sequence (Z = 1, the layer shape) against its
    length, and the least-squares fit t(L) = a L^2 + b L + c the pages use to
    split latency into quadratic, linear and constant terms.  Inputs drawn on
    the device (same distributions), directions weight-tied."""
    import numpy as np
    import torch
    import state_space_denoisers_amd as ssd
    from state_space_denoisers_amd import _abi
    from synth import gen
    dev = torch.device("cuda", 0)
    base = gen.WORKLOADS["layer130m_L1k"].replace(Z=1)
    small = gen.make_inputs(base.replace(L=64))
    A = gen.as_torch(small["A_f"], "fp32", dev)
    D = gen.as_torch(small["D"], "fp32", dev)
    pts = []
    for L in lengths:
        T = gen.prefix_on_device(base, L, dev, seed=base.seed + L)
        p = (T["dt_f"], A, T["B_f"], T["C_f"])
        y = torch.empty_like(T["x"])
        shape = ssd.shape_of(T["x"], T["B_f"], base.chunk)
        ws = torch.empty(ssd.bissd_workspace_size(shape, _abi.OP_FORWARD), dtype=torch.uint8, device=dev)
        fn = lambda: ssd.bissd_forward(T["x"], p, p, D, chunk=base.chunk, y=y, workspace=ws)
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        reps = max(5, min(200, int(2e6 // L)))
        settle(fn, LEG_SETTLE_S)
        pts.append((L, event_time_ms(fn, reps)))
        del T, y, ws
    Ls = np.array([q[0] for q in pts], dtype=np.float64)
    ts = np.array([q[1] for q in pts], dtype=np.float64)
    coef, *_ = np.linalg.lstsq(np.stack([Ls ** 2, Ls, np.ones_like(Ls)], 1), ts, rcond=None)
    return {"workload": "latency_sweep", "batch": 1, "heads": base.H, "dstate": base.N,
            "points": [{"seq_len": int(L), "ms": round(t, 4), "tokens_per_s": L / (t * 1e-3)}
                       for L, t in pts],
            "fit_ms": {"a_per_L2": coef[0], "b_per_L": coef[1], "c": coef[2]},
            "share_at_max_L": {"quadratic": coef[0] * Ls[-1] ** 2 / ts[-1],
                               "linear": coef[1] * Ls[-1] / ts[-1], "constant": coef[2] / ts[-1]}}


def bench_generation(steps_per_block=8, blocks=2, prefix=65536):
    """Block-wise generation after a long prefix, two ways, same kernels:
    (a) a full-sequence bidirectional model re-scans prefix + every block so
    far at each denoising step (bissd_forward over the whole sequence);
    (b) the partially bidirectional model continues the cached prefix state
    (bissd_block_update per step, committing the state after each block's
    last step).  Batch 4, blocks of 64 tokens, bf16, 24 heads, N = 128.
    The prefix's own encode is done once for (b) and not timed.  Both give
    the active block the same output (the full scan's reverse over the last
    block sees only that block), which is checked."""
    import torch
    import state_space_denoisers_amd as ssd
    from synth import gen
    w = gen.WORKLOADS["block_update"]
    dev = torch.device("cuda", 0)
    Lb = w.L
    Lmax = prefix + blocks * Lb
    seq = gen.prefix_on_device(w, Lmax, dev, seed=w.seed + 17)
    A = gen.as_torch(gen.make_inputs(w)["A_f"], "fp32", dev)
    D = gen.as_torch(gen.make_inputs(w)["D"], "fp32", dev)

    def cut(lo, hi):
        return {k: v[:, lo:hi].contiguous() for k, v in seq.items()}

    full = [cut(0, prefix + (k + 1) * Lb) for k in range(blocks)]
    blk = [cut(prefix + k * Lb, prefix + (k + 1) * Lb) for k in range(blocks)]
    p = lambda T: (T["dt_f"], A, T["B_f"], T["C_f"])  # weight-tied directions
    y_full = [torch.empty_like(f["x"]) for f in full]
    from state_space_denoisers_amd import _abi
    ws_full = [torch.empty(ssd.bissd_workspace_size(ssd.shape_of(f["x"], f["B_f"], 256),
                                                    _abi.OP_FORWARD), dtype=torch.uint8, device=dev)
               for f in full]
    ws_blk = torch.empty(max(256, ssd.bissd_workspace_size(ssd.shape_of(blk[0]["x"], blk[0]["B_f"], 64),
                                                            _abi.OP_BLOCK)), dtype=torch.uint8, device=dev)
    y_blk = [torch.empty_like(b["x"]) for b in blk]
    state0 = torch.empty((w.Z, w.H, w.P, w.N), dtype=torch.float32, device=dev)
    pre = cut(0, prefix)
    ssd.bissd_forward(pre["x"], p(pre), p(pre), D, chunk=256, final_state=state0)
    del pre
    state = torch.empty_like(state0)

    def run_full():
        for k in range(blocks):
            for _ in range(steps_per_block):
                ssd.bissd_forward(full[k]["x"], p(full[k]), p(full[k]), D, chunk=256,
                                  y=y_full[k], workspace=ws_full[k])

    def run_cached():
        state.copy_(state0)
        for k in range(blocks):
            for s in range(steps_per_block):
                last = s == steps_per_block - 1
                ssd.bissd_block_update(state, blk[k]["x"], p(blk[k]), p(blk[k]), D, chunk=64,
                                       y_blk=y_blk[k], state_out=state if last else None,
                                       commit=last, workspace=ws_blk)

    for fn in (run_full, run_cached):
        fn()
    torch.cuda.synchronize()
    settle(run_cached, LEG_SETTLE_S)
    ms_full = event_time_ms(run_full, 3)
    ms_cached = event_time_ms(run_cached, 10)
    nstep = blocks * steps_per_block
    agree = 0.0
    for k in range(blocks):
        ref = y_full[k][:, prefix + k * Lb:].float()
        agree = max(agree, float((y_blk[k].float() - ref).abs().max() / ref.abs().max()))
    return {"workload": f"generation_L{prefix // 1024}k", "prefix_tokens": prefix,
            "block_tokens": Lb, "batch": w.Z, "blocks": blocks,
            "steps_per_block": steps_per_block,
            "ms_per_step_full_rescan": ms_full / nstep, "ms_per_step_block_update": ms_cached / nstep,
            "speedup": ms_full / ms_cached, "active_block_y_maxrel_full_vs_cached": agree}


# ------------------------------------------------------------- profiling

LEG_SETTLE_S = 0.2  # untimed calls before each further leg's timing


def settle(fn, seconds):
    """Untimed calls of fn for at least `seconds`: a GPU that has been idle
    runs its first milliseconds of work below its sustained clocks."""
    import torch
    t = time.perf_counter()
    while time.perf_counter() - t < seconds:
        for _ in range(20):
            fn()
        torch.cuda.synchronize()


def settle_with_gemm(seconds):
    """The same for profiling runs, with a plain bf16 matrix product (a kernel
    of another library, left out of the committed summaries)."""
    import torch
    a = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    b = torch.randn(4096, 4096, dtype=torch.bfloat16, device="cuda")
    settle(lambda: torch.mm(a, b), seconds)


def profile_phase(args):
    """Kernel launches for rocprofv3.  With --settle S, the profiled call
    itself runs for S seconds first (the block update: a matrix product),
    so the profile sees the GPU at its sustained clocks; those calls are part
    of the statistics."""
    import torch
    from synth import gen
    if args.profile_phase == "attention":
        # the hybrids' attention layer: forward (with lse) then backward,
        # Z = 8, L = 4096, 12 heads of 64, bf16, full bidirectional
        import state_space_denoisers_amd as ssd
        dev = torch.device("cuda", 0)
        Z, L, H = 8, 4096, 12
        inp = gen.make_attention_inputs(Z, L, H, "bf16", 2002)
        T = {k: gen.as_torch(v, "bf16", dev) for k, v in inp.items()}
        dout = gen.as_torch(gen.make_attention_inputs(Z, L, H, "bf16", 2003)["q"], "bf16", dev)
        lse = torch.empty((Z, H, L), dtype=torch.float32, device=dev)
        o = torch.empty_like(T["q"])
        def fb():
            ssd.bissd_attention_forward(T["q"], T["k"], T["v"], o=o, lse=lse)
            ssd.bissd_attention_backward(T["q"], T["k"], T["v"], o, dout, lse)
        settle(fb, args.settle)
        torch.cuda.synchronize()
        print(f"profiling attention forward + backward Z={Z} L={L} H={H} x{args.iters}", flush=True)
        for _ in range(args.iters):
            fb()
        torch.cuda.synchronize()
        print("done", flush=True)
        return
    w = gen.WORKLOADS[args.workload]
    if args.profile_phase == "block":
        import state_space_denoisers_amd as ssd
        inp, T = device_inputs(w)
        fwd, rev = dirs(T)
        state = torch.zeros((w.Z, w.H, w.P, w.N), dtype=torch.float32, device=T["x"].device)
        if args.settle > 0:
            settle_with_gemm(args.settle)
        torch.cuda.synchronize()
        print(f"profiling block update on {w.name} x{args.iters}", flush=True)
        for _ in range(args.iters):
            ssd.bissd_block_update(state, T["x"], fwd, rev, T["D"], commit=True)
        torch.cuda.synchronize()
        print("done", flush=True)
        return
    if args.profile_phase == "conv":
        cf = ConvForward(w)
        cf()
        settle(cf, args.settle)
        torch.cuda.synchronize()
        print(f"profiling forward with the width-4 convolution on {w.name} x{args.iters}", flush=True)
        for _ in range(args.iters):
            cf()
        torch.cuda.synchronize()
        print("done", flush=True)
        return
    if args.profile_phase in ("train", "backward"):
        # train: the training step (saving forward, saved backward);
        # backward: the backward that forms everything itself
        t = Train(w)
        fn = t if args.profile_phase == "train" else t.backward_recompute
        settle(fn, args.settle)
        torch.cuda.synchronize()
        print(f"profiling {args.profile_phase} on {w.name} x{args.iters}", flush=True)
        for _ in range(args.iters):
            fn()
        torch.cuda.synchronize()
        print("done", flush=True)
        return
    f = Forward(w)
    f()
    if args.profile_phase == "all":
        settle(f, args.settle)
    torch.cuda.synchronize()
    print(f"profiling {args.profile_phase} on {w.name} x{args.iters}", flush=True)
    for _ in range(args.iters):
        if args.profile_phase == "all":
            f()
        else:
            f.phase(int(args.profile_phase))
    torch.cuda.synchronize()
    print("done", flush=True)


def copy_calibrate():
    """A plain device copy of known size, for scaling HBM byte counters."""
    import torch
    n = 1 << 28  # 256 MiB
    a = torch.ones(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copy_calibrate bytes_read={n} bytes_written={n} launches=5", flush=True)


# ------------------------------------------------------------------ main

def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--profile-phase", choices=["0", "1", "2", "3", "all", "conv", "train", "backward",
                                                "block", "attention"])
    ap.add_argument("--workload", default="layer130m_L1k")
    ap.add_argument("--iters", type=int, default=20)
    ap.add_argument("--copy-calibrate", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--settle", type=float, default=None,
                    help="seconds of untimed work before the warm-up steps (default 0.5; 0 for --profile-phase)")
    args = ap.parse_args()
    if args.settle is None:
        args.settle = 0.0 if args.profile_phase is not None else 0.5

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: there is no multi-GPU path (the design notes say "
              "how the scan would shard); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.copy_calibrate:
        return copy_calibrate()
    if args.profile_phase is not None:
        return profile_phase(args)

    from synth import gen
    w = gen.WORKLOADS["layer130m_L1k"]
    log(f"bench: {w.name} Z={w.Z} L={w.L} H={w.H} P={w.P} N={w.N} chunk={w.chunk} {w.dtype}")
    f = Forward(w)
    settle(f, args.settle)
    for _ in range(args.warmup):
        f()
    torch.cuda.synchronize()
    s = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(s)
    for _ in range(args.steps):
        f()
    ev1.record(s)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = 1e3 * wall / args.steps
    ev_ms = ev0.elapsed_time(ev1) / args.steps
    tokens = w.tokens
    log(f"bench: {ms_step * 1e3:.1f} us/step wall, {ev_ms * 1e3:.1f} us/step events")

    ph = phase_times_us(f, max(20, args.steps // 4))
    log(f"bench: kernels {ph}")
    dom = max(ph, key=ph.get)
    pidx = {v: k for k, v in PHASE_NAMES.items()}[dom.split("+")[0]]
    dur_s = ph[dom] * 1e-6
    alg_bytes = phase_bytes_per_token(w, pidx) * tokens
    achieved = alg_bytes / dur_s / 1e9
    roof = {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": stored_traffic(dom, w.name),
            "algorithmic_bytes_per_launch": alg_bytes, "avg_launch_us": round(ph[dom], 2)}
    mfma = None
    if pidx == 2 or PHASE_NAMES[2] in ph:
        fl = k3_flops_per_token(w) * tokens
        mfma = {"kernel": PHASE_NAMES[2], "achieved_TFLOPs": round(fl / (ph[PHASE_NAMES[2]] * 1e-6) / 1e12, 1),
                "peak_TFLOPs": BF16_PEAK_TFLOPS,
                "frac": round(fl / (ph[PHASE_NAMES[2]] * 1e-6) / 1e12 / BF16_PEAK_TFLOPS, 4),
                "flops_per_launch": fl}

    # five further trials of the same workload (event-timed on the launch
    # stream), for their median and spread next to the timed region above
    trials = [event_time_ms(f, max(20, args.steps // 4)) * 1e3 for _ in range(5)]
    extra = {"settle_s": args.settle,
             "kernels_us": {k: round(v, 2) for k, v in ph.items()},
             "trials_us_per_step": {"values": [round(t, 2) for t in trials],
                                    "median": round(float(sorted(trials)[2]), 2)},
             "path_hbm_algorithmic_GBs": round(per_token_bytes(w) * tokens / (ev_ms * 1e-3) / 1e9, 1),
             "k3_mfma": mfma,
             "state_pass": state_pass_line(w, ph)}
    if not args.no_extra:
        try:
            extra["long_L65k"] = bench_long(max(5, args.steps // 20))
            log(f"bench: long {extra['long_L65k']['tokens_per_s']:.3e} tokens/s")
        except Exception as exc:  # report, do not hide
            extra["long_L65k"] = {"error": repr(exc)}
        try:
            extra["train_L2k"] = bench_train(max(5, args.steps // 20))
            log(f"bench: train {extra['train_L2k']}")
        except Exception as exc:
            extra["train_L2k"] = {"error": repr(exc)}
        try:
            extra["train_L2k_rev64"] = bench_train(max(5, args.steps // 20), rev_block=64)
            log(f"bench: train rev64 {extra['train_L2k_rev64']}")
        except Exception as exc:
            extra["train_L2k_rev64"] = {"error": repr(exc)}
        try:
            extra["layer130m_L1k_conv4"] = bench_conv(max(20, args.steps // 4))
            log(f"bench: conv {extra['layer130m_L1k_conv4']}")
        except Exception as exc:
            extra["layer130m_L1k_conv4"] = {"error": repr(exc)}
        try:
            extra["block_update"] = bench_block(max(50, args.steps))
            log(f"bench: block {extra['block_update']}")
        except Exception as exc:
            extra["block_update"] = {"error": repr(exc)}
        for L, blk in ((1024, 0), (4096, 0), (4096, 256)):
            key = f"attention_L{L // 1024}k" + (f"_block{blk}" if blk else "")
            try:
                extra[key] = bench_attention(max(20, args.steps // 4), L=L, block=blk)
                log(f"bench: {key} {extra[key]}")
            except Exception as exc:
                extra[key] = {"error": repr(exc)}
        try:
            extra["attention_bwd_L4k"] = bench_attention_backward(max(10, args.steps // 10), L=4096)
            log(f"bench: attention_bwd_L4k {extra['attention_bwd_L4k']}")
        except Exception as exc:
            extra["attention_bwd_L4k"] = {"error": repr(exc)}
        try:
            extra["latency_sweep"] = bench_latency_sweep()
            log(f"bench: latency sweep {extra['latency_sweep']}")
        except Exception as exc:
            extra["latency_sweep"] = {"error": repr(exc)}
        try:
            extra["generation_L64k"] = bench_generation()
            log(f"bench: generation {extra['generation_L64k']}")
        except Exception as exc:
            extra["generation_L64k"] = {"error": repr(exc)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w)
        log(f"bench: cpu baseline {cpu}")

    out = {"metric": METRIC, "value": tokens / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1,
           "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic",
           "config": {"workload": w.name, "batch": w.Z, "seq_len": w.L, "heads": w.H,
                      "headdim": w.P, "dstate": w.N, "ngroups": w.G, "chunk": w.chunk,
                      "parallelism": "none (1 GPU)"},
           "roofline": roof, "cpu_baseline": cpu, "extra": extra,
           "kernel_source_sha": source_sha()}
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
