"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects invalid arguments before launching anything.

Every call here fails validation (or is a documented no-op such as batch 0
without outputs), so no HIP kernel is launched and no device memory is
touched; the pointers are fake addresses that are never dereferenced.
"""
import ctypes
import os
import re

import pytest

import state_space_model_amd as ssd
from state_space_model_amd import ConvDesc, ScanDesc, StepDesc, lib

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "ssd.h")

OK, INVALID, SHAPE, DTYPE, ALIGN, UNSUP, WS, HIP = range(8)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = declared_functions()
    assert set(names) == set(ssd.EXPORTED), names
    for n in names:
        assert hasattr(lib, n), n
        assert ctypes.cast(getattr(lib, n), ctypes.c_void_p).value


def test_abi_version_and_status_strings():
    assert ssd.abi_version() == 5
    for code in range(8):
        s = lib.ssd_status_string(code).decode()
        assert s.startswith(ssd.STATUS_NAMES[code])
    assert lib.ssd_status_string(99).decode() == "unknown ssd_status"


def desc(**kw):
    d = dict(batch=1, seqlen=512, nheads=4, headdim=16, dstate=16, ngroups=1, chunk=64,
             io_dtype=0, dt_softplus=1, dt_min=1e-4, dt_max=0.5)
    d.update(kw)
    return ScanDesc(**d)


BASE = 0x7F0000000000  # fake, 256-byte aligned device addresses, never dereferenced


def fake_args(d: ScanDesc, ws_bytes=None, **over):
    es = 2 if d.io_dtype == 1 else 4
    sizes = dict(x=d.batch * d.seqlen * d.nheads * d.headdim * es,
                 dt=d.batch * d.seqlen * d.nheads * 4, dt_bias=d.nheads * 4, A=d.nheads * 4,
                 B=d.batch * d.seqlen * d.ngroups * d.dstate * es,
                 C=d.batch * d.seqlen * d.ngroups * d.dstate * es, D=d.nheads * 4,
                 h0=d.batch * d.nheads * d.headdim * d.dstate * 4,
                 y=d.batch * d.seqlen * d.nheads * d.headdim * es,
                 fin=d.batch * d.nheads * d.headdim * d.dstate * 4, ws=1 << 30)
    ptr, addr = {}, BASE
    for k, v in sizes.items():
        ptr[k] = addr
        addr += (max(v, 1) + 4095) // 4096 * 4096
    ptr.update(over)
    need = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    wsb = need if ws_bytes is None else ws_bytes
    P = ctypes.c_void_p
    return (ctypes.byref(d), P(ptr["x"]), P(ptr["dt"]), P(ptr["dt_bias"]), P(ptr["A"]),
            P(ptr["B"]), P(ptr["C"]), P(ptr["D"]), P(ptr["h0"]), P(ptr["y"]), P(ptr["fin"]),
            P(ptr["ws"]), ctypes.c_size_t(wsb), P(0))


def scan_status(d, **kw):
    return lib.ssd_chunk_scan(*fake_args(d, **kw))


def test_workspace_query():
    d = desc()
    n = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    nc = 512 // 64
    assert n >= 4 * 1 * 4 * nc * (16 * 16 + 1)
    assert n % 256 == 0
    # ragged sequence: the last partial chunk still needs a state
    d2 = desc(seqlen=513)
    assert lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d2)) > n
    assert lib.ssd_chunk_scan_workspace_bytes(None) == 0
    assert lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(desc(headdim=24))) == 0


def _r256(v):
    return (v + 255) // 256 * 256


@pytest.mark.parametrize("kw,chain", [
    (dict(io_dtype=1, batch=8, nheads=64, headdim=64, dstate=128, chunk=256), True),
    (dict(io_dtype=1, batch=4, nheads=64, headdim=64, dstate=128, chunk=128), True),
    (dict(io_dtype=1, batch=16, nheads=16, headdim=32, dstate=64, chunk=64), True),
    (dict(io_dtype=1, batch=1, nheads=255, headdim=64, dstate=128, chunk=256), False),  # too few chains
    (dict(io_dtype=0, batch=8, nheads=64, headdim=64, dstate=128, chunk=256), False),   # float32 io
    (dict(io_dtype=1, batch=8, nheads=64, headdim=64, dstate=128, chunk=512), False),   # L > 256
    (dict(io_dtype=1, batch=8, nheads=64, headdim=128, dstate=128, chunk=256), False),  # P = 128
    (dict(io_dtype=1, batch=8, nheads=64, headdim=64, dstate=32, chunk=256), False),    # N = 32
])
def test_schedule_and_workspace(kw, chain):
    """The schedule choice and the exact workspace size of each schedule."""
    d = desc(seqlen=1000, **kw)
    sched = lib.ssd_chunk_scan_schedule(ctypes.byref(d))
    assert sched == (ssd.SSD_SCHEDULE_CHAIN if chain else ssd.SSD_SCHEDULE_PHASED)
    Bt, H, P, N, L, G = d.batch, d.nheads, d.headdim, d.dstate, d.chunk, d.ngroups
    nc = (d.seqlen + L - 1) // L
    cb = _r256((2 if d.io_dtype == 1 else 4) * Bt * nc * G * L * L)   # bf16 scan: C B^T in bf16
    if chain:
        want = cb + _r256(2 * Bt * nc * G * N * L)
    else:
        want = _r256(4 * Bt * H * nc * P * N) + _r256(4 * Bt * H * nc) + cb
        if d.io_dtype == 1:
            want += _r256(2 * Bt * H * nc * P * N)
            # the chain's head shapes at L <= 256 keep the B^T pre-pass copy
            if P in (32, 64) and N in (64, 128) and L <= 256:
                want += _r256(2 * Bt * nc * G * N * L)
    assert lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d)) == want


def test_schedule_query_rejects_invalid_descriptors():
    assert lib.ssd_chunk_scan_schedule(None) == -INVALID
    assert lib.ssd_chunk_scan_schedule(ctypes.byref(desc(headdim=24))) == -UNSUP
    assert lib.ssd_chunk_scan_schedule(ctypes.byref(desc(io_dtype=5))) == -DTYPE


@pytest.mark.parametrize("kw,code", [
    (dict(io_dtype=2), DTYPE),
    (dict(batch=-1), SHAPE),
    (dict(seqlen=-5), SHAPE),
    (dict(nheads=0), SHAPE),
    (dict(headdim=0), SHAPE),
    (dict(chunk=0), SHAPE),
    (dict(nheads=6, ngroups=4), SHAPE),
    (dict(dt_min=0.6, dt_max=0.5), INVALID),
    (dict(dt_min=float("nan")), INVALID),
    (dict(headdim=24), UNSUP),
    (dict(dstate=48), UNSUP),
    (dict(chunk=48), UNSUP),
    (dict(chunk=1024), UNSUP),
    (dict(headdim=128, chunk=512), UNSUP),
    (dict(io_dtype=1, dstate=16), UNSUP),
])
def test_scan_descriptor_errors(kw, code):
    assert scan_status(desc(**kw)) == code


def test_scan_pointer_errors():
    d = desc()
    assert lib.ssd_chunk_scan(None, *fake_args(d)[1:]) == INVALID
    assert scan_status(d, x=0) == INVALID
    assert scan_status(d, dt=0) == INVALID
    assert scan_status(d, A=0) == INVALID
    assert scan_status(d, y=0) == INVALID
    assert scan_status(d, x=BASE + 8) == ALIGN
    assert scan_status(d, fin=BASE + 4) == ALIGN
    args = fake_args(d)
    assert scan_status(d, dt=args[2].value + 2) == ALIGN     # scalars: 4-byte alignment
    assert scan_status(d, A=args[4].value + 4, ws=0) == WS   # 4-byte offset is fine for A
    assert scan_status(d, ws=0) == WS
    assert scan_status(d, ws_bytes=1024) == WS
    # outputs overlapping inputs, the workspace or each other
    args = fake_args(d)
    x_addr = args[1].value
    assert scan_status(d, y=x_addr) == INVALID
    assert scan_status(d, fin=args[4].value) == INVALID      # final state over A
    assert scan_status(d, y=args[11].value + 4096) == INVALID  # y inside the workspace
    assert scan_status(d, fin=args[9].value + 256) == INVALID  # final state inside y


def test_scan_timed_needs_enough_events():
    d = desc()
    evs = (ctypes.c_void_p * 2)()
    assert lib.ssd_chunk_scan_timed(*fake_args(d), evs, 2) == INVALID
    evs = (ctypes.c_void_p * 5)()  # enough slots, but NULL events
    assert lib.ssd_chunk_scan_timed(*fake_args(d), evs, 5) == INVALID


def test_empty_batch_is_a_noop():
    # batch 0: nothing to compute, nothing launched
    assert scan_status(desc(batch=0)) == OK
    # empty sequence without a requested final state: nothing launched
    d = desc(seqlen=0)
    assert scan_status(d, fin=0) == OK


def step_desc(**kw):
    d = dict(batch=2, nheads=4, headdim=16, dstate=16, ngroups=1, io_dtype=0, dt_softplus=1,
             dt_min=1e-4, dt_max=0.5)
    d.update(kw)
    return StepDesc(**d)


def step_status(d, **over):
    ptr = dict(state=BASE, x=BASE + (1 << 24), dt=BASE + (2 << 24), bias=BASE + (3 << 24),
               A=BASE + (4 << 24), B=BASE + (5 << 24), C=BASE + (6 << 24), D=BASE + (7 << 24),
               y=BASE + (8 << 24))
    ptr.update(over)
    P = ctypes.c_void_p
    return lib.ssd_step(ctypes.byref(d), P(ptr["state"]), P(ptr["x"]), P(ptr["dt"]),
                        P(ptr["bias"]), P(ptr["A"]), P(ptr["B"]), P(ptr["C"]), P(ptr["D"]),
                        P(ptr["y"]), P(0))


def test_step_errors():
    assert lib.ssd_step(None, *([None] * 10)) == INVALID
    assert step_status(step_desc(io_dtype=3)) == DTYPE
    assert step_status(step_desc(nheads=3, ngroups=2)) == SHAPE
    assert step_status(step_desc(headdim=8)) == UNSUP
    assert step_status(step_desc(dt_min=1.0, dt_max=0.1)) == INVALID
    assert step_status(step_desc(), state=0) == INVALID
    assert step_status(step_desc(), x=BASE + (1 << 24) + 2) == ALIGN
    assert step_status(step_desc(), dt=BASE + (2 << 24) + 2) == ALIGN
    assert step_status(step_desc(), y=BASE) == INVALID          # y over the state
    assert step_status(step_desc(), x=BASE + 64) == INVALID     # x inside the state
    assert step_status(step_desc(batch=0)) == OK                # nothing to do


def conv_desc(**kw):
    d = dict(batch=2, seqlen=64, channels=40, width=4, io_dtype=0, silu=1)
    d.update(kw)
    return ConvDesc(**d)


def conv_status(d, **over):
    ptr = dict(x=BASE, w=BASE + (1 << 24), bias=BASE + (2 << 24), si=BASE + (3 << 24),
               y=BASE + (4 << 24), so=BASE + (5 << 24))
    ptr.update(over)
    P = ctypes.c_void_p
    return lib.ssd_conv1d(ctypes.byref(d), P(ptr["x"]), P(ptr["w"]), P(ptr["bias"]),
                          P(ptr["si"]), P(ptr["y"]), P(ptr["so"]), P(0))


def conv_step_status(d, **over):
    ptr = dict(state=BASE, x=BASE + (1 << 24), w=BASE + (2 << 24), bias=BASE + (3 << 24),
               y=BASE + (4 << 24))
    ptr.update(over)
    P = ctypes.c_void_p
    return lib.ssd_conv1d_step(ctypes.byref(d), P(ptr["state"]), P(ptr["x"]), P(ptr["w"]),
                               P(ptr["bias"]), P(ptr["y"]), P(0))


def test_conv_errors():
    assert lib.ssd_conv1d(None, *([None] * 7)) == INVALID
    assert conv_status(conv_desc(io_dtype=2)) == DTYPE
    assert conv_status(conv_desc(channels=0)) == SHAPE
    assert conv_status(conv_desc(seqlen=-1)) == SHAPE
    assert conv_status(conv_desc(width=0)) == SHAPE
    assert conv_status(conv_desc(width=1)) == UNSUP
    assert conv_status(conv_desc(width=5)) == UNSUP
    assert conv_status(conv_desc(), w=0) == INVALID
    assert conv_status(conv_desc(), x=0) == INVALID
    assert conv_status(conv_desc(), y=0) == INVALID
    assert conv_status(conv_desc(), x=BASE + 4) == ALIGN
    assert conv_status(conv_desc(), so=BASE + (5 << 24) + 8) == ALIGN
    assert conv_status(conv_desc(), w=BASE + (1 << 24) + 2) == ALIGN
    assert conv_status(conv_desc(), y=BASE + 1024) == INVALID       # y inside x
    assert conv_status(conv_desc(), so=BASE + (1 << 24)) == INVALID  # window over the weights
    assert conv_status(conv_desc(), so=BASE + (3 << 24) + 16) == INVALID  # partly over state_in
    assert conv_status(conv_desc(), so=BASE + (4 << 24)) == INVALID  # window over y
    # nothing to do: no launch
    assert conv_status(conv_desc(batch=0)) == OK
    assert conv_status(conv_desc(seqlen=0), so=0) == OK


def test_conv_step_errors():
    d = conv_desc(seqlen=123456)   # the step does not read seqlen
    assert lib.ssd_conv1d_step(None, *([None] * 6)) == INVALID
    assert conv_step_status(conv_desc(io_dtype=7)) == DTYPE
    assert conv_step_status(conv_desc(width=6)) == UNSUP
    assert conv_step_status(d, state=0) == INVALID
    assert conv_step_status(d, bias=BASE + (3 << 24) + 1) == ALIGN
    assert conv_step_status(d, y=BASE + 16) == INVALID            # y over the window
    assert conv_step_status(d, x=BASE + 32) == INVALID            # x inside the window
    assert conv_step_status(conv_desc(batch=0)) == OK


def bwd_status(d, ws_bytes=None, **over):
    ptr = {k: BASE + (i << 26) for i, k in enumerate(
        ["x", "dt", "bias", "A", "B", "C", "D", "h0", "dy", "df", "dx", "ddt", "dA", "dB", "dC",
         "dD", "dbias", "dh0", "ws"])}
    ptr.update(over)
    P = ctypes.c_void_p
    need = lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(d))
    return lib.ssd_chunk_scan_backward(
        ctypes.byref(d), *[P(ptr[k]) for k in ["x", "dt", "bias", "A", "B", "C", "D", "h0", "dy",
                                               "df", "dx", "ddt", "dA", "dB", "dC", "dD", "dbias",
                                               "dh0", "ws"]],
        ctypes.c_size_t(need if ws_bytes is None else ws_bytes), P(0))


def test_backward_workspace_and_errors():
    d = desc()
    need = lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(d))
    assert need > lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d))
    assert need % 256 == 0
    # chunks of at most 256 tokens (one token per thread of a 256-thread workgroup)
    assert lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(desc(dstate=128, chunk=512, headdim=32))) == 0
    assert lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(desc(chunk=288))) == 0
    assert lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(desc(chunk=256))) > 0
    assert lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(desc(io_dtype=1, headdim=16, dstate=32))) > 0
    assert bwd_status(desc(dstate=128, chunk=512, headdim=32)) == UNSUP
    assert bwd_status(desc(io_dtype=5)) == DTYPE
    assert bwd_status(d, dy=0) == INVALID
    assert bwd_status(d, dx=0) == INVALID
    assert bwd_status(d, dA=0) == INVALID
    assert bwd_status(d, dy=BASE + (8 << 26) + 4) == ALIGN
    assert bwd_status(d, ddt=BASE + (11 << 26) + 2) == ALIGN
    assert bwd_status(d, ws=0) == WS
    assert bwd_status(d, ws_bytes=1024) == WS
    assert bwd_status(d, dx=BASE) == INVALID                 # gradient over x
    assert bwd_status(d, dB=BASE + (10 << 26)) == INVALID    # two gradients overlap
    assert bwd_status(d, dh0=BASE + (18 << 26) + 4096) == INVALID  # inside the workspace


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(1, 64, 4, 16)
    B = torch.zeros(1, 64, 1, 16)
    with pytest.raises(ValueError, match="device tensor"):
        ssd.ssd_chunk_scan(x, torch.zeros(1, 64, 4), torch.zeros(4), B, B, chunk=64)


def ablation_status(d, variant, **kw):
    a = fake_args(d, **kw)
    return lib.ssd_chunk_scan_ablation(a[0], variant, *a[1:])


@pytest.mark.parametrize("kw,variant,code", [
    (dict(io_dtype=1, headdim=64, dstate=128, chunk=256), 7, INVALID),      # unknown variant
    (dict(io_dtype=1, headdim=64, dstate=128, chunk=256), -1, INVALID),
    (dict(io_dtype=1, headdim=32, dstate=128, chunk=256), 1, UNSUP),        # not the 64 x 128 head
    (dict(io_dtype=1, headdim=64, dstate=64, chunk=256), 2, UNSUP),
    (dict(io_dtype=1, headdim=64, dstate=128, chunk=512), 1, UNSUP),        # chunk > 256
    (dict(io_dtype=0, headdim=64, dstate=128, chunk=256), 2, UNSUP),        # loaded mask: bf16 only
    (dict(io_dtype=1, headdim=24, dstate=128, chunk=256), 1, UNSUP),        # the descriptor's own error
])
def test_ablation_rejects_before_launch(kw, variant, code):
    assert ablation_status(desc(**kw), variant) == code


def test_ablation_shares_the_scan_validation():
    d = desc(io_dtype=1, headdim=64, dstate=128, chunk=256)
    assert ablation_status(d, 1, x=0) == INVALID                  # NULL x
    assert ablation_status(d, 2, x=BASE + 8) == ALIGN             # misaligned x
    assert ablation_status(d, 1, ws_bytes=16) == WS               # workspace too small
    # batch 0 writes nothing and is valid for every variant
    assert ablation_status(desc(io_dtype=1, headdim=64, dstate=128, chunk=256, batch=0), 2) == OK


def noalloc_status(d, **over):
    a = fake_args(d, **over)
    # the same arguments without the workspace pointer and size
    return lib.ssd_chunk_scan_noalloc(*a[:11], a[13])


def test_noalloc_rejects_problems_beyond_its_scratch():
    """Sizes beyond the static scratch are refused on the host, before the
    scratch's address is looked up or anything is launched."""
    big = desc(io_dtype=1, batch=16, seqlen=16384, nheads=64, headdim=64, dstate=128, chunk=256)
    need = lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(big))
    assert need > ssd.SSD_NOALLOC_MAX_WORKSPACE
    assert noalloc_status(big) == WS
    # the 2.7B-shaped 4096-token layer and the 8 x 16384 batched prefill fit
    for fits in (desc(io_dtype=1, batch=1, seqlen=4096, nheads=80, headdim=64, dstate=128,
                      chunk=256),
                 desc(io_dtype=1, batch=8, seqlen=16384, nheads=64, headdim=64, dstate=128,
                      chunk=256)):
        assert lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(fits)) <= ssd.SSD_NOALLOC_MAX_WORKSPACE
    # descriptor errors come first
    assert noalloc_status(desc(headdim=24)) == UNSUP
    assert noalloc_status(desc(io_dtype=3)) == DTYPE
    assert lib.ssd_chunk_scan_noalloc(None, *fake_args(desc())[1:11], None) == INVALID
    # batch 0: nothing to do, no scratch needed
    assert noalloc_status(desc(batch=0)) == OK
