"""GPU tests of the library's kernel timers (bissd_timer_arm / bissd_timer_read):
an armed slot is taken by exactly the next kernel launch, records that
dispatch's own duration, and leaves the output of the call unchanged."""
import pytest
import torch

import state_space_denoisers_amd as ssd
from synth import gen
from tests.gpu_util import device, dirs, to_dev

pytestmark = pytest.mark.gpu


def _layer():
    w = gen.WORKLOADS["layer130m_L1k"]
    inp = gen.make_inputs(w)
    T = to_dev(inp, "bf16")
    return w, T


def test_timer_takes_the_next_launch_only():
    w, T = _layer()
    fwd, rev = dirs(T)
    y0 = ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=w.chunk)
    torch.cuda.synchronize()
    print("timer: full forward, slot 7", flush=True)
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    ssd.bissd_timer_arm(7)
    y1 = ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=w.chunk)
    b.record(s)
    torch.cuda.synchronize()
    whole = a.elapsed_time(b)
    k1 = ssd.bissd_timer_read(7)
    # the first kernel of the call took the slot: shorter than the whole call
    assert 0.0 < k1 < whole, (k1, whole)
    assert torch.equal(y0, y1)
    # the slot was disarmed: a second call leaves it as it was
    ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=w.chunk)
    torch.cuda.synchronize()
    assert ssd.bissd_timer_read(7) == k1


def test_timer_durations_add_up_to_the_call():
    """Each forward kernel timed on its own dispatch (phases enqueued in the
    call's order): their sum is no more than the span of the calls and not
    much less (the kernels run back to back)."""
    w, T = _layer()
    fwd, rev = dirs(T)
    shape = ssd.shape_of(T["x"], T["B_f"], w.chunk)
    from state_space_denoisers_amd import _abi
    ws = torch.empty(ssd.bissd_workspace_size(shape, _abi.OP_FORWARD), dtype=torch.uint8,
                     device=device())
    y = torch.empty_like(T["x"])

    def phase(p):
        ssd.bissd_forward_phase(p, T["x"], fwd, rev, T["D"], chunk=w.chunk, y=y, workspace=ws)
    ssd.bissd_forward(T["x"], fwd, rev, T["D"], chunk=w.chunk, y=y, workspace=ws)
    torch.cuda.synchronize()
    print("timer: phases 0 1 2 timed", flush=True)
    reps, order = 20, (0, 1, 2)
    s = torch.cuda.current_stream()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(s)
    for r in range(reps):
        for i, p in enumerate(order):
            ssd.bissd_timer_arm(100 + 3 * r + i)
            phase(p)
    b.record(s)
    ssd.bissd_timer_arm(-1)
    torch.cuda.synchronize()
    span = a.elapsed_time(b)
    total = sum(ssd.bissd_timer_read(100 + k) for k in range(3 * reps))
    assert 0.0 < total <= span, (total, span)
    assert all(ssd.bissd_timer_read(100 + k) > 0.0 for k in range(3 * reps))
