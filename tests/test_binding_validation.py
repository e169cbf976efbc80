"""The Python binding rejects bad tensors before any call into the library.

The C library sizes every buffer from x's dtype and the shapes of x and B, so
a tensor of another dtype, shape or device would be read or written past its
end.  These tests run on the CPU: the library is replaced by a stub whose
every entry point fails the test if it is reached, and each case must raise
in the binding.  A call whose tensors are all well formed but live in host
memory must be rejected as well (the last check).
"""
import pytest
import torch

import state_space_denoisers_amd as ssd
from state_space_denoisers_amd import _abi

Z, L, H, P, N, G = 2, 40, 4, 64, 64, 2


class _NoCalls:
    """Library stand-in: workspace sizes are answered, everything else fails."""

    def bissd_workspace_size(self, shape, op):
        return 1024

    def bissd_attention_workspace_size(self, shape):
        return 1024

    def __getattr__(self, name):
        def fail(*a, **k):
            raise AssertionError(f"{name} was called despite invalid arguments")
        return fail


@pytest.fixture(autouse=True)
def no_library(monkeypatch):
    monkeypatch.setattr(_abi, "load", lambda *a, **k: _NoCalls())


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def scan_args(dtype=torch.bfloat16):
    x = t(Z, L, H, P, dtype=dtype)
    def d():
        return ssd.Dir(t(Z, L, H, dtype=dtype), t(H, dtype=torch.float32),
                       t(Z, L, G, N, dtype=dtype), t(Z, L, G, N, dtype=dtype))
    return x, d(), d(), t(H, dtype=torch.float32)


def state(dtype=torch.float32):
    return t(Z, H, P, N, dtype=dtype)


# each case: (what is wrong, exception type, a function of the valid
# arguments that returns the kwargs of the bad forward call)
def _replace_dir(d, **kw):
    return d._replace(**kw)


FORWARD_CASES = [
    ("x not 4-D", ValueError, lambda x, f, r, D: dict(x=x[0])),
    ("x fp16", TypeError, lambda x, f, r, D: dict(x=x.half())),
    ("dt dtype differs from x", TypeError,
     lambda x, f, r, D: dict(fwd=_replace_dir(f, dt=f.dt.float()))),
    ("dt shape", ValueError, lambda x, f, r, D: dict(rev=_replace_dir(r, dt=t(Z, L, H + 1)))),
    ("A bf16", TypeError, lambda x, f, r, D: dict(fwd=_replace_dir(f, A=f.A.bfloat16()))),
    ("A shape", ValueError, lambda x, f, r, D: dict(rev=_replace_dir(r, A=t(H + 1, dtype=torch.float32)))),
    ("B fp32 with bf16 x", TypeError, lambda x, f, r, D: dict(fwd=_replace_dir(f, B=f.B.float()))),
    ("C shape differs from B", ValueError,
     lambda x, f, r, D: dict(fwd=_replace_dir(f, C=t(Z, L, G, 2 * N)))),
    ("rev B of other length", ValueError, lambda x, f, r, D: dict(rev=_replace_dir(r, B=t(Z, L + 1, G, N)))),
    ("groups do not divide heads", ValueError,
     lambda x, f, r, D: dict(fwd=_replace_dir(f, B=t(Z, L, 3, N), C=t(Z, L, 3, N)))),
    ("dt_bias bf16", TypeError,
     lambda x, f, r, D: dict(fwd=_replace_dir(f, dt_bias=t(H)))),
    ("dt_bias shape", ValueError,
     lambda x, f, r, D: dict(fwd=_replace_dir(f, dt_bias=t(2 * H, dtype=torch.float32)))),
    ("D bf16", TypeError, lambda x, f, r, D: dict(D=D.bfloat16())),
    ("D shape", ValueError, lambda x, f, r, D: dict(D=t(1, dtype=torch.float32))),
    ("init_state shape", ValueError, lambda x, f, r, D: dict(init_state=t(Z, H, P, N + 1, dtype=torch.float32))),
    ("init_state bf16", TypeError, lambda x, f, r, D: dict(init_state=state(torch.bfloat16))),
    ("final_state shape", ValueError, lambda x, f, r, D: dict(final_state=t(Z, H, N, P, dtype=torch.float32))),
    ("y dtype", TypeError, lambda x, f, r, D: dict(y=x.float())),
    ("y shape", ValueError, lambda x, f, r, D: dict(y=x[:, :-1])),
    ("y not contiguous", ValueError, lambda x, f, r, D: dict(y=x.transpose(0, 1).contiguous().transpose(0, 1))),
    ("everything in host memory", ValueError, lambda x, f, r, D: dict()),
]


@pytest.mark.parametrize("what,exc,bad", FORWARD_CASES, ids=[c[0] for c in FORWARD_CASES])
def test_forward_rejects(what, exc, bad):
    x, f, r, D = scan_args()
    kw = dict(x=x, fwd=f, rev=r, D=D)
    kw.update(bad(x, f, r, D))
    args = (kw.pop("x"), kw.pop("fwd"), kw.pop("rev"), kw.pop("D"))
    with pytest.raises(exc):
        ssd.bissd_forward(*args, chunk=64, **kw)


def test_forward_phase_rejects_a_short_state():
    x, f, r, D = scan_args()
    with pytest.raises(ValueError):
        ssd.bissd_forward_phase(0, x, f, r, D, chunk=64, y=torch.empty_like(x),
                                workspace=t(64, dtype=torch.uint8),
                                init_state=t(Z, H, P, N - 1, dtype=torch.float32))


@pytest.mark.parametrize("what", ["state_in shape", "state_in bf16", "state_out shape", "y_blk dtype",
                                  "dt shape", "host memory"])
def test_block_update_rejects(what):
    x, f, r, D = scan_args()
    kw = dict(state_in=state(), y_blk=None, state_out=None)
    if what == "state_in shape":
        kw["state_in"] = t(Z, H, P, 2 * N, dtype=torch.float32)
    elif what == "state_in bf16":
        kw["state_in"] = state(torch.bfloat16)
    elif what == "state_out shape":
        kw["state_out"] = t(Z, H + 1, P, N, dtype=torch.float32)
    elif what == "y_blk dtype":
        kw["y_blk"] = x.float()
    elif what == "dt shape":
        f = f._replace(dt=t(Z, L + 1, H))
    with pytest.raises((ValueError, TypeError)):
        ssd.bissd_block_update(kw.pop("state_in"), x, f, r, D, chunk=64, **kw)


@pytest.mark.parametrize("what", ["dy dtype", "dy shape", "dy missing", "dx shape", "dB_f fp16",
                                  "dA_r shape", "unknown buffer", "bias grad without bias",
                                  "host memory"])
def test_backward_rejects(what):
    x, f, r, D = scan_args()
    dy = torch.zeros_like(x)
    grads = {}
    if what == "dy dtype":
        dy = dy.float()
    elif what == "dy shape":
        dy = dy[:, 1:]
    elif what == "dy missing":
        dy = None
    elif what == "dx shape":
        grads["dx"] = t(Z, L, H, P + 1, dtype=torch.float32)
    elif what == "dB_f fp16":
        grads["dB_f"] = t(Z, L, G, N, dtype=torch.float16)
    elif what == "dA_r shape":
        grads["dA_r"] = t(2 * H, dtype=torch.float32)
    elif what == "unknown buffer":
        grads["dq"] = t(H, dtype=torch.float32)
    elif what == "bias grad without bias":
        grads["ddt_bias_f"] = t(H, dtype=torch.float32)
    with pytest.raises((ValueError, TypeError)):
        ssd.bissd_backward(x, f, r, D, dy, chunk=64, grads=grads)


@pytest.mark.parametrize("what", ["k shape", "v dtype", "o dtype", "lse shape", "lse bf16",
                                  "host memory"])
def test_attention_forward_rejects(what):
    q = t(Z, L, H, 64)
    k, v, o, lse = torch.zeros_like(q), torch.zeros_like(q), None, None
    if what == "k shape":
        k = t(Z, L + 1, H, 64)
    elif what == "v dtype":
        v = v.float()
    elif what == "o dtype":
        o = q.float()
    elif what == "lse shape":
        lse = t(Z, L, H, dtype=torch.float32)
    elif what == "lse bf16":
        lse = t(Z, H, L)
    with pytest.raises((ValueError, TypeError)):
        ssd.bissd_attention_forward(q, k, v, o=o, lse=lse)


@pytest.mark.parametrize("what", ["dout dtype", "o shape", "lse missing", "host memory"])
def test_attention_backward_rejects(what):
    q = t(Z, L, H, 64)
    k, v, o, dout = torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q), torch.zeros_like(q)
    lse = t(Z, H, L, dtype=torch.float32)
    if what == "dout dtype":
        dout = dout.float()
    elif what == "o shape":
        o = o[:, :-1]
    elif what == "lse missing":
        lse = None
    with pytest.raises((ValueError, TypeError)):
        ssd.bissd_attention_backward(q, k, v, o, dout, lse)


def test_a_well_formed_call_reaches_only_the_device_check():
    """Every shape and dtype right, tensors in host memory: the message names
    the device, so no earlier check fired on valid arguments."""
    x, f, r, D = scan_args()
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.bissd_forward(x, f, r, D, chunk=64, init_state=state(), final_state=state())
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.bissd_backward(x, f, r, D, torch.zeros_like(x), chunk=64, init_state=state())
    with pytest.raises(ValueError, match="GPU tensor"):
        ssd.bissd_block_update(state(), x, f, r, D, chunk=64)
