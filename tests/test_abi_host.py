"""The C ABI on the host: the library loads, exports every symbol the header
declares, and rejects bad arguments before anything reaches a device.

Pointers here are fake host addresses: validation only compares and
alignment-checks them, it never dereferences them.
"""
import ctypes as C
import os
import re

import pytest

from state_space_denoisers_amd import _abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_abi.LIB_PATH):
        from state_space_denoisers_amd import build
        build.build()
    return _abi.load()


def header_functions():
    text = open(os.path.join(ROOT, "include", "bissd.h")).read()
    return sorted(set(re.findall(r"^\w[\w\s\*]*?\b(bissd_\w+)\s*\(", text, re.M)))


def test_header_and_binding_agree():
    assert sorted(_abi.EXPORTS) == header_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in header_functions():
        assert hasattr(lib, name), name
    assert lib.bissd_version() == 4
    assert lib.bissd_last_hip_error() == 0


def test_no_torch_types_in_the_header():
    text = open(os.path.join(ROOT, "include", "bissd.h")).read()
    for banned in ("torch", "at::", "Tensor", "c10"):
        assert banned not in text, banned
    assert 'extern "C"' in text


def shape(**kw):
    d = dict(batch=2, seqlen=300, nheads=8, headdim=64, dstate=128, ngroups=1, chunk=256,
             dtype=_abi.BISSD_BF16, rev_block=0)
    d.update(kw)
    return _abi.Shape(**d)


A = 1 << 20  # fake, 16-byte aligned addresses far apart


def addr(i):
    return C.c_void_p(A * (i + 1))


def dirs(base):
    return _abi.Dir(addr(base), addr(base + 1), addr(base + 2), addr(base + 3))


def call_forward(lib, s, **over):
    args = dict(x=addr(0), fwd=dirs(1), rev=dirs(5), D=addr(9), init=None, y=addr(10),
                final=None, ws=addr(12), nws=1 << 40, stream=None)
    args.update(over)
    return lib.bissd_forward(C.byref(s) if s is not None else None, args["x"], args["fwd"],
                             args["rev"], args["D"], args["init"], args["y"], args["final"],
                             args["ws"], C.c_size_t(args["nws"]), args["stream"])


def test_workspace_size(lib):
    s = shape()
    n = lib.bissd_workspace_size(C.byref(s), _abi.OP_FORWARD)
    nc = (300 + 255) // 256
    assert n >= 2 * 2 * nc * 8 * 64 * 128 * 4
    assert lib.bissd_workspace_size(C.byref(shape(headdim=32)), 0) == 0
    assert lib.bissd_workspace_size(None, 0) == 0
    # linear in L (constant-size state per chunk)
    n1 = lib.bissd_workspace_size(C.byref(shape(seqlen=256 * 8)), 0)
    n2 = lib.bissd_workspace_size(C.byref(shape(seqlen=256 * 16)), 0)
    assert 1.9 < n2 / n1 < 2.1


@pytest.mark.parametrize("over,code", [
    (dict(batch=0), -2), (dict(seqlen=0), -2), (dict(nheads=6, ngroups=4), -2),
    (dict(headdim=32), -3), (dict(dstate=96), -3), (dict(chunk=100), -3),
    (dict(dtype=7), -3), (dict(rev_block=-64), -2), (dict(rev_block=32), -3),
    (dict(rev_block=192), -3), (dict(rev_block=384), -3), (dict(rev_block=96, chunk=128), -3),
])
def test_bad_shapes(lib, over, code):
    assert call_forward(lib, shape(**over)) == code


@pytest.mark.parametrize("rb,chunk", [(64, 256), (128, 256), (256, 256), (512, 256), (1024, 256),
                                      (64, 64), (192, 64), (128, 128)])
def test_supported_reverse_blocks(lib, rb, chunk):
    """Multiples of the 64-token tile that split a chunk evenly or span whole
    chunks pass validation (the call then fails only on the fake workspace)."""
    assert call_forward(lib, shape(rev_block=rb, chunk=chunk), nws=16) == -5


def test_block_update_takes_no_reverse_block(lib):
    s = shape(seqlen=64, chunk=64, rev_block=64)
    rc = lib.bissd_block_update(C.byref(s), addr(20), addr(0), dirs(1), dirs(5), addr(9),
                                addr(10), None, None, None, addr(12), C.c_size_t(1 << 40), None)
    assert rc == -3
    assert lib.bissd_workspace_size(C.byref(s), _abi.OP_BLOCK) == 0


def test_null_and_alignment(lib):
    s = shape()
    assert call_forward(lib, None) == -1
    assert call_forward(lib, s, x=None) == -1
    assert call_forward(lib, s, y=None) == -1
    bad = _abi.Dir(addr(1), None, addr(3), addr(4))
    assert call_forward(lib, s, fwd=bad) == -1
    assert call_forward(lib, s, x=C.c_void_p(A + 8)) == -4
    assert call_forward(lib, s, ws=None) == -5
    assert call_forward(lib, s, nws=16) == -5


def test_aliasing_is_rejected(lib):
    s = shape()
    assert call_forward(lib, s, y=addr(0)) == -7          # y over x
    assert call_forward(lib, s, ws=addr(10)) == -7        # workspace over y
    assert call_forward(lib, s, final=addr(9)) == -7      # final_state over D


def test_block_update_validation(lib):
    s = shape(seqlen=300, chunk=256)
    rc = lib.bissd_block_update(C.byref(s), addr(20), addr(0), dirs(1), dirs(5), addr(9),
                                addr(10), None, None, None, addr(12), C.c_size_t(1 << 40), None)
    assert rc == -2  # block longer than chunk
    s = shape(seqlen=64, chunk=64)
    rc = lib.bissd_block_update(C.byref(s), None, addr(0), dirs(1), dirs(5), addr(9),
                                addr(10), None, None, None, addr(12), C.c_size_t(1 << 40), None)
    assert rc == -1
    # state_out partially overlapping state_in
    rc = lib.bissd_block_update(C.byref(s), addr(20), addr(0), dirs(1), dirs(5), addr(9),
                                addr(10), C.c_void_p(A * 21 + 4096), None, None, addr(12),
                                C.c_size_t(1 << 40), None)
    assert rc == -7


def test_forward_phase_range(lib):
    """Phases 0..3 exist (3 = Gram tiles); any other index is rejected before
    the shape or a pointer is looked at."""
    s = shape()
    for bad in (-1, 4, 100):
        rc = lib.bissd_forward_phase(C.byref(s), addr(0), dirs(1), dirs(5), addr(9), None,
                                     addr(10), None, addr(12), C.c_size_t(1 << 40), None, bad)
        assert rc == -3, bad
    # a valid phase index still validates the arguments
    rc = lib.bissd_forward_phase(C.byref(s), None, dirs(1), dirs(5), addr(9), None, addr(10),
                                 None, addr(12), C.c_size_t(1 << 40), None, 3)
    assert rc == -1


def test_workspace_holds_gram_tiles(lib):
    """The forward workspace holds both slots' chunk Gram tiles in the compute
    dtype (2 x batch x chunks x groups x chunk^2 elements) besides the states;
    a block update of at most 64 tokens needs none."""
    s = shape(seqlen=1024, ngroups=2, nheads=8)  # bf16
    n = lib.bissd_workspace_size(C.byref(s), _abi.OP_FORWARD)
    states = 2 * 2 * 2 * 4 * 8 * 64 * 128 * 2
    gram = 2 * 2 * 4 * 2 * 256 * 256 * 2
    assert n >= states + gram
    n32 = lib.bissd_workspace_size(C.byref(shape(seqlen=1024, ngroups=2, nheads=8,
                                                 dtype=_abi.BISSD_F32)), _abi.OP_FORWARD)
    assert n32 >= 2 * states + 2 * gram
    small = lib.bissd_workspace_size(C.byref(shape(seqlen=64, chunk=64)), _abi.OP_BLOCK)
    big = lib.bissd_workspace_size(C.byref(shape(seqlen=65, chunk=128)), _abi.OP_BLOCK)
    assert big - small >= 2 * 2 * 128 * 128 * 2


def test_status_strings(lib):
    for code in _abi.STATUS:
        assert lib.bissd_status_string(code)
    assert b"unknown" in lib.bissd_status_string(99)


def call_backward(lib, s, **over):
    args = dict(x=addr(0), fwd=dirs(1), rev=dirs(5), D=addr(9), init=None, dy=addr(10),
                dx=addr(11), gf=_abi.Grad(addr(12), addr(13), addr(14), addr(15)),
                gr=_abi.Grad(addr(16), addr(17), addr(18), addr(19)), dD=addr(20),
                ws=addr(21), nws=1 << 40)
    args.update(over)
    return lib.bissd_backward(C.byref(s), args["x"], args["fwd"], args["rev"], args["D"],
                              args["init"], args["dy"], args["dx"], args["gf"], args["gr"],
                              args["dD"], args["ws"], C.c_size_t(args["nws"]), None)


def test_backward_validation(lib):
    """Every rejected backward call returns before anything is enqueued
    (these pointers are fake; a call that passed validation would launch)."""
    s = shape(seqlen=100)  # every tensor fits in the 1 MiB spacing
    assert lib.bissd_workspace_size(C.byref(s), _abi.OP_BACKWARD) > \
        lib.bissd_workspace_size(C.byref(s), _abi.OP_FORWARD)
    assert call_backward(lib, s, dy=None) == -1
    assert call_backward(lib, s, gr=_abi.Grad(addr(16), None, addr(18), addr(19))) == -1
    assert call_backward(lib, s, dx=C.c_void_p(A * 12 + 8)) == -4
    assert call_backward(lib, s, nws=64) == -5
    assert call_backward(lib, s, dx=addr(0)) == -7                     # dx over x
    assert call_backward(lib, s, dD=addr(10)) == -7                    # dD over dy
    assert call_backward(lib, s, gf=_abi.Grad(addr(12), addr(13), addr(14), addr(14))) == -7
    assert call_backward(lib, s, ws=addr(11)) == -7                    # workspace over dx
    assert call_backward(lib, shape(seqlen=100, headdim=32)) == -3


def attn_shape(**kw):
    d = dict(batch=2, seqlen=300, nheads=12, headdim=64, block=0, dtype=_abi.BISSD_BF16,
             reserved=0)
    d.update(kw)
    return _abi.AttnShape(**d)


def call_attention(lib, s, scale=0.0, **over):
    args = dict(q=addr(0), k=addr(1), v=addr(2), o=addr(3), lse=None, stream=None)
    args.update(over)
    return lib.bissd_attention_forward(C.byref(s) if s is not None else None, args["q"],
                                       args["k"], args["v"], C.c_float(scale), args["o"],
                                       args["lse"], args["stream"])


@pytest.mark.parametrize("over,scale,code", [
    (dict(headdim=128), 0.0, -3), (dict(block=32), 0.0, -3), (dict(block=-64), 0.0, -2),
    (dict(seqlen=0), 0.0, -2), (dict(dtype=5), 0.0, -3), (dict(reserved=1), 0.0, -2),
    (dict(), -1.0, -2), (dict(), float("nan"), -2),
])
def test_attention_validation(lib, over, scale, code):
    assert call_attention(lib, attn_shape(**over), scale) == code


def test_attention_pointers(lib):
    s = attn_shape()
    assert call_attention(lib, None) == -1
    assert call_attention(lib, s, q=None) == -1
    assert call_attention(lib, s, o=C.c_void_p(A + 8)) == -4
    assert call_attention(lib, s, o=addr(1)) == -7   # o over k


def test_attention_backward_validation(lib):
    s = attn_shape()
    n = lib.bissd_attention_workspace_size(C.byref(s))
    assert n >= 2 * 12 * 300 * 4
    assert lib.bissd_attention_workspace_size(C.byref(attn_shape(headdim=32))) == 0

    def bwd(**over):
        args = dict(q=addr(0), k=addr(1), v=addr(2), o=addr(3), do=addr(4), lse=addr(5),
                    dq=addr(6), dk=addr(7), dv=addr(8), ws=addr(9), nws=1 << 30)
        args.update(over)
        return lib.bissd_attention_backward(C.byref(s), args["q"], args["k"], args["v"],
                                            args["o"], args["do"], args["lse"], C.c_float(0.0),
                                            args["dq"], args["dk"], args["dv"], args["ws"],
                                            C.c_size_t(args["nws"]), None)
    assert bwd(lse=None) == -1
    assert bwd(nws=16) == -5
    assert bwd(dq=C.c_void_p(A * 7 + 8)) == -4
    assert bwd(dk=addr(6)) == -7      # dk over dq
    assert bwd(ws=addr(0)) == -7      # workspace over q


def test_dt_post_processing_validation(lib):
    s = shape()
    bad = _abi.Dir(addr(1), addr(2), addr(3), addr(4), addr(20), 0.2, 0.1)   # dt_min > dt_max
    assert call_forward(lib, s, fwd=bad) == -2
    bad = _abi.Dir(addr(1), addr(2), addr(3), addr(4), addr(20), -1.0, 0.1)  # dt_min < 0
    assert call_forward(lib, s, fwd=bad) == -2
    bad = _abi.Dir(addr(1), addr(2), addr(3), addr(4), C.c_void_p(A * 21 + 4), 0.0, 1.0)
    assert call_forward(lib, s, rev=bad) == -4
    ok = _abi.Dir(addr(1), addr(2), addr(3), addr(4), addr(20), 0.0, float("inf"))
    assert call_forward(lib, s, fwd=ok, nws=16) == -5   # passes validation up to the workspace



def test_noalloc_rejects_before_any_device_call(lib):
    """bissd_forward_noalloc checks the shape and the size of its workspace
    against the scratch array before it touches the device: a bad shape and
    a shape too large for the array are rejected here, with no GPU."""
    args = (addr(0), dirs(1), dirs(5), addr(9), None, addr(10), None, None)
    big = shape(batch=2, seqlen=65536, nheads=4)
    assert lib.bissd_workspace_size(C.byref(big), _abi.OP_FORWARD) > _abi.NOALLOC_SCRATCH_BYTES
    assert lib.bissd_forward_noalloc(C.byref(big), *args) == -8
    assert lib.bissd_forward_noalloc(C.byref(shape(headdim=32)), *args) == -3
    assert lib.bissd_forward_noalloc(C.byref(shape(batch=0)), *args) == -2
    assert lib.bissd_forward_noalloc(None, *args) == -1
    assert b"BISSD_NOALLOC_SCRATCH_BYTES" in lib.bissd_status_string(-8)
    hdr = open(os.path.join(ROOT, "include", "bissd.h")).read()
    assert f"({_abi.NOALLOC_SCRATCH_BYTES >> 20}u << 20)" in hdr


def conv_dir(base, w=None, b=None, act=0, reserved=0):
    d = dirs(base)
    d.conv_w = w
    d.conv_b = b
    d.conv_act = act
    d.reserved = reserved
    return d


def test_convolution_validation(lib):
    """The mixer's convolution fields are checked before anything is
    enqueued: taps need a width in the shape, a bias or an activation needs
    taps, the width is at most 4, reserved fields are zero, pointers are
    16-byte aligned, and the backward rejects a direction with taps."""
    ok_w = addr(30)
    assert call_forward(lib, shape(conv_width=4), fwd=conv_dir(1, ok_w), nws=16) == -5
    assert call_forward(lib, shape(conv_width=0), fwd=conv_dir(1, ok_w)) == -2
    assert call_forward(lib, shape(conv_width=5)) == -3
    assert call_forward(lib, shape(conv_width=-1)) == -2
    assert call_forward(lib, shape(flags=2)) == -2
    assert call_forward(lib, shape(conv_width=4), rev=conv_dir(5, None, addr(31))) == -2
    assert call_forward(lib, shape(conv_width=4), rev=conv_dir(5, None, None, act=1)) == -2
    assert call_forward(lib, shape(conv_width=4), rev=conv_dir(5, ok_w, act=2)) == -2
    assert call_forward(lib, shape(conv_width=4), rev=conv_dir(5, ok_w, reserved=1)) == -2
    assert call_forward(lib, shape(conv_width=4), fwd=conv_dir(1, C.c_void_p(A * 30 + 4))) == -4
    # the forward workspace holds both directions' convolved x
    s0, s4 = shape(), shape(conv_width=4)
    n0 = lib.bissd_workspace_size(C.byref(s0), _abi.OP_FORWARD)
    n4 = lib.bissd_workspace_size(C.byref(s4), _abi.OP_FORWARD)
    assert n4 - n0 >= 2 * 2 * 300 * 8 * 64 * 2
    # a 64-token block forms it in LDS; a longer one in the workspace
    b0 = lib.bissd_workspace_size(C.byref(shape(seqlen=64, chunk=64, conv_width=4)), _abi.OP_BLOCK)
    assert b0 == lib.bissd_workspace_size(C.byref(shape(seqlen=64, chunk=64)), _abi.OP_BLOCK)
    b1 = lib.bissd_workspace_size(C.byref(shape(seqlen=100, chunk=128, conv_width=4)), _abi.OP_BLOCK)
    assert b1 > lib.bissd_workspace_size(C.byref(shape(seqlen=100, chunk=128)), _abi.OP_BLOCK)
    # the backward takes no convolution
    assert call_backward(lib, shape(conv_width=4), fwd=conv_dir(1, ok_w)) == -3


def test_block_update_conv_state_aliasing(lib):
    s = shape(seqlen=64, chunk=64, conv_width=4)
    f = conv_dir(1, addr(30))

    def blk(cin, cout):
        return lib.bissd_block_update(C.byref(s), addr(20), addr(0), f, dirs(5), addr(9),
                                      addr(10), None, cin, cout, addr(12), C.c_size_t(1 << 40), None)
    assert blk(addr(40), addr(10)) == -7           # conv_state_out over y
    assert blk(addr(40), C.c_void_p(A * 41 + 16)) == -7   # partially over conv_state_in
    assert blk(addr(40), addr(0)) == -7            # over x
    assert blk(C.c_void_p(A * 40 + 4), None) == -4   # misaligned


def test_timer_validation(lib):
    # no device call: out-of-range slots, a NULL result pointer, a slot that
    # has never been armed, and disarming
    assert lib.bissd_timer_arm(-2) == -2
    assert lib.bissd_timer_arm(4096) == -2
    assert lib.bissd_timer_arm(-1) == 0
    ms = C.c_float(0.0)
    assert lib.bissd_timer_read(-1, C.byref(ms)) == -2
    assert lib.bissd_timer_read(4096, C.byref(ms)) == -2
    assert lib.bissd_timer_read(4095, None) == -1
    assert lib.bissd_timer_read(4095, C.byref(ms)) == -1


def test_save_flag_validation(lib):
    """BISSD_SAVE: the saving forward's workspace is the backward's (so one
    buffer serves both calls), and the flag is refused where there is no
    backward to keep values for (a convolution, a block update, the static
    scratch array) or next to an unknown flag bit."""
    plain, saving = shape(), shape(flags=_abi.SAVE)
    nf = lib.bissd_workspace_size(C.byref(plain), _abi.OP_FORWARD)
    nb = lib.bissd_workspace_size(C.byref(plain), _abi.OP_BACKWARD)
    assert nb > nf > 0
    assert lib.bissd_workspace_size(C.byref(saving), _abi.OP_FORWARD) == nb
    assert lib.bissd_workspace_size(C.byref(saving), _abi.OP_BACKWARD) == nb
    # a forward-sized workspace is too small for a saving forward
    assert call_forward(lib, saving, nws=nf) == -5
    assert call_forward(lib, shape(flags=_abi.SAVE | 2)) == -2
    assert call_forward(lib, shape(flags=_abi.SAVE, conv_width=4)) == -3
    assert lib.bissd_workspace_size(C.byref(shape(flags=_abi.SAVE, conv_width=4)), _abi.OP_FORWARD) == 0
    blk = shape(seqlen=64, chunk=64, flags=_abi.SAVE)
    rc = lib.bissd_block_update(C.byref(blk), addr(20), addr(0), dirs(1), dirs(5), addr(9),
                                addr(10), None, None, None, addr(12), C.c_size_t(1 << 40), None)
    assert rc == -3
    args = (addr(0), dirs(1), dirs(5), addr(9), None, addr(10), None, None)
    assert lib.bissd_forward_noalloc(C.byref(shape(seqlen=64, chunk=64, flags=_abi.SAVE)), *args) == -3
    # the backward takes the flag like the forward
    assert call_backward(lib, shape(flags=_abi.SAVE), nws=16) == -5
