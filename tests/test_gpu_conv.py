"""GPU parity of the depthwise causal convolution (ssd_conv1d, ssd_conv1d_step)
against the CPU oracle.

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching", O(1) cache section (a depthwise convolution over a sliding window of
the k-1 previous inputs per channel, cached with shape (B, D_conv, k-1); the
decode body updates that window) and Setup (k = 4; D_conv of the 130M and 2.7B
checkpoint shapes).

Bars: the outgoing window holds copies of inputs and must equal the oracle's
exactly.  y: max over (b, channel) slices of ||y - ref||_inf / ||ref||_inf at
most 1e-4 for float32 and 2e-2 for bfloat16; for bfloat16 also, element by
element, |y - ref| <= 2^-8 |ref| + 1e-6 (the only error beyond float32
arithmetic is the final rounding to bfloat16, at most half a unit of the last
of its 8 significant bits).  A sequence split anywhere, or run token by token
through ssd_conv1d_step, gives bitwise the same outputs as one call.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import TOL, announce, need_gpu
from oracle.metrics import slice_rel_err
from ssd_inputs import CONV_WORKLOADS, ConvWorkload, make_conv_inputs

pytestmark = pytest.mark.gpu


def conv_y_err(got, ref) -> float:
    return slice_rel_err(got, ref, 2, (1,))


def check_y(y, ref, io):
    err = conv_y_err(y, ref)
    assert err <= TOL[io], err
    if io == "bf16":
        g = y.detach().to("cpu", torch.float64).numpy()
        bad = np.abs(g - ref) > np.abs(ref) * 2.0 ** -8 + 1e-6
        assert not bad.any(), (int(bad.sum()), np.argwhere(bad)[:4])


def check_state(st, ref):
    g = st.detach().to("cpu", torch.float64).numpy()
    assert g.shape == ref.shape
    assert np.array_equal(g, ref), np.abs(g - ref).max()


def run(ssd, inp, w: ConvWorkload, with_state=True, with_bias=True, silu=None):
    silu = w.silu if silu is None else silu
    d = {k: v.to("cuda") for k, v in inp.items()}
    y, st = ssd.ssd_conv1d(d["x"], d["weight"], d["bias"] if with_bias else None,
                           state=d.get("state") if with_state else None, silu=silu)
    torch.cuda.synchronize()
    ref_y, ref_st = oracle.conv1d(inp["x"], inp["weight"], inp["bias"] if with_bias else None,
                                  inp.get("state") if with_state else None, silu=silu)
    return y, st, ref_y, ref_st


CASES = [
    # (Bt, T, D, k, io, state, bias, silu)
    (1, 5, 3, 4, "f32", True, True, False),
    (2, 17, 8, 4, "f32", True, False, True),
    (1, 33, 40, 4, "f32", False, True, True),
    (3, 16, 13, 3, "f32", True, True, True),
    (1, 2, 12, 4, "f32", True, True, False),
    (2, 1, 4, 2, "f32", True, True, True),
    (1, 70, 1, 4, "f32", True, True, True),
    (1, 5, 3, 4, "bf16", True, True, False),
    (2, 17, 16, 4, "bf16", True, False, True),
    (1, 49, 40, 4, "bf16", False, True, True),
    (3, 16, 13, 3, "bf16", True, True, True),
    (1, 2, 24, 4, "bf16", True, True, True),
    (2, 31, 8, 2, "bf16", True, True, False),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "_".join(map(str, c)))
def test_conv_tiny_shapes(case):
    need_gpu()
    import state_space_model_amd as ssd
    Bt, T, D, K, io, with_state, with_bias, silu = case
    w = ConvWorkload("tiny", Bt, T, D, K, io, silu, 3000 + CASES.index(case))
    inp = make_conv_inputs(w, with_state=True)
    announce(f"conv tiny {case}")
    y, st, ref_y, ref_st = run(ssd, inp, w, with_state, with_bias, silu)
    check_y(y, ref_y, io)
    check_state(st, ref_st)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_empty_sequence_hands_the_window_on(io):
    need_gpu()
    import state_space_model_amd as ssd
    w = ConvWorkload("empty", 2, 0, 24, 4, io, True, 3100)
    inp = make_conv_inputs(w, with_state=True)
    announce(f"conv empty sequence {io}")
    y, st, _, ref_st = run(ssd, inp, w)
    assert y.shape == (2, 0, 24)
    check_state(st, ref_st)
    _, st0, _, ref0 = run(ssd, inp, w, with_state=False)
    check_state(st0, ref0)
    assert not ref0.any()


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_conv_split_and_in_place_window_are_bitwise_equal(io):
    """A sequence cut into parts (each seeded with the previous window, updated
    in place) gives the same bits as one call; so do 8 single-token steps."""
    need_gpu()
    import state_space_model_amd as ssd
    w = ConvWorkload("split", 2, 64, 48, 4, io, True, 3200)
    inp = make_conv_inputs(w, with_state=True)
    d = {k: v.to("cuda") for k, v in inp.items()}
    announce(f"conv split {io}")
    y_full, st_full = ssd.ssd_conv1d(d["x"], d["weight"], d["bias"], state=d["state"])
    win = d["state"].clone()
    ptr = win.data_ptr()
    parts = []
    for lo, hi in ((0, 5), (5, 23), (23, 24), (24, 56)):
        y, _ = ssd.ssd_conv1d(d["x"][:, lo:hi].contiguous(), d["weight"], d["bias"], state=win,
                              state_out=win)
        parts.append(y)
    for t in range(56, 64):
        parts.append(ssd.ssd_conv1d_step(win, d["x"][:, t].contiguous(), d["weight"],
                                         d["bias"])[:, None])
    torch.cuda.synchronize()
    assert win.data_ptr() == ptr
    assert torch.equal(torch.cat(parts, 1), y_full)
    assert torch.equal(win, st_full)
    ref_y, ref_st = oracle.conv1d(inp["x"], inp["weight"], inp["bias"], inp["state"], silu=True)
    check_y(y_full, ref_y, io)
    check_state(st_full, ref_st)


@pytest.mark.parametrize("case", [(1, 4, 3, "f32"), (5, 13, 4, "f32"), (3, 40, 4, "bf16"),
                                  (2, 7, 2, "bf16"), (4, 64, 3, "bf16")],
                         ids=lambda c: "_".join(map(str, c)))
def test_conv_step_against_oracle(case):
    need_gpu()
    import state_space_model_amd as ssd
    Bt, D, K, io = case
    w = ConvWorkload("step", Bt, 6, D, K, io, True, 3300 + D)
    inp = make_conv_inputs(w, with_state=True)
    d = {k: v.to("cuda") for k, v in inp.items()}
    announce(f"conv step {case}")
    win = d["state"].clone()
    ref_win = inp["state"].double().numpy()
    for t in range(6):
        y = ssd.ssd_conv1d_step(win, d["x"][:, t].contiguous(), d["weight"], d["bias"])
        torch.cuda.synchronize()
        ref_y, ref_win = oracle.conv1d_step(ref_win, inp["x"][:, t], inp["weight"], inp["bias"],
                                            silu=True)
        check_y(y[:, None], ref_y[:, None], io)
        check_state(win, ref_win)


@pytest.mark.parametrize("name", ["conv_m130_f32", "conv_m2p7_bf16"])
def test_conv_full_size(name):
    """The 130M and 2.7B shapes (4096 tokens, D_conv 1792 / 5376), every
    output against the oracle, in the launch configuration the benchmark
    times; a repeated call is bitwise identical."""
    need_gpu()
    import state_space_model_amd as ssd
    w = CONV_WORKLOADS[name]
    inp = make_conv_inputs(w, with_state=True)
    announce(f"conv full {name}")
    y, st, ref_y, ref_st = run(ssd, inp, w)
    check_y(y, ref_y, w.io_dtype)
    check_state(st, ref_st)
    y2, st2, _, _ = run(ssd, inp, w)
    assert torch.equal(y, y2) and torch.equal(st, st2)


@pytest.mark.parametrize("batch", [1, 16, 64])
def test_conv_decode_shape(batch):
    """The 2.7B decode shape (D_conv 5376, bfloat16 window): 4 steps."""
    need_gpu()
    import state_space_model_amd as ssd
    w = CONV_WORKLOADS["conv_m2p7_decode"].with_(batch=batch, seqlen=4)
    inp = make_conv_inputs(w, with_state=True)
    d = {k: v.to("cuda") for k, v in inp.items()}
    announce(f"conv decode b{batch}")
    win = d["state"].clone()
    ys = [ssd.ssd_conv1d_step(win, d["x"][:, t].contiguous(), d["weight"], d["bias"])[:, None]
          for t in range(4)]
    torch.cuda.synchronize()
    ref_y, ref_st = oracle.conv1d(inp["x"], inp["weight"], inp["bias"], inp["state"], silu=True)
    check_y(torch.cat(ys, 1), ref_y, "bf16")
    check_state(win, ref_st)
