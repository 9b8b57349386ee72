"""Pins that tie a depthwise causal convolution to facts other than itself.

Each pin takes an implementation `impl` with the signature of oracle.conv1d
(x [Bt,T,D], w [D,k], bias, state [Bt,D,k-1], silu=...) returning float64
(y, state_out), and returns the worst relative error it saw.  They are applied
to the C oracle (test_conv_oracle.py) and to broken copies of a plain loop to
show that a plausible slip fails at least one of them.

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching", O(1) cache section (a depthwise convolution over a sliding window of
the k-1 previous inputs, cached per channel with shape (B, D_conv, k-1)) and
Setup (k = 4).
"""
from __future__ import annotations

import numpy as np
import torch
from scipy.special import expit

import golden_io


def _rel(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    if a.shape != b.shape:
        return float("inf")
    if a.size == 0:
        return 0.0
    den = max(float(np.abs(b).max()), 1e-300)
    return float(np.abs(a - b).max() / den)


def _rand(rng, Bt, T, D, K, state=True, bias=True):
    f32 = np.float32
    x = rng.standard_normal((Bt, T, D)).astype(f32)
    w = rng.uniform(-0.5, 0.5, (D, K)).astype(f32)
    b = rng.uniform(-0.5, 0.5, D).astype(f32) if bias else None
    s = rng.standard_normal((Bt, D, K - 1)) if state else None
    return x, w, b, s


def pin_hand_example(impl) -> float:
    """The dyadic example of tests/golden/hand_conv.txt, worked by hand."""
    g = golden_io.load("hand_conv.txt")
    Bt, T, D, K = (int(v) for v in g["shape"])
    w = g["w"].reshape(D, K).astype(np.float32)
    bias = g["bias"].astype(np.float32)
    state = g["state"].reshape(Bt, D, K - 1)
    y, st = impl(g["x"].reshape(Bt, T, D).astype(np.float32), w, bias, state, silu=False)
    worst = max(_rel(y, g["y"].reshape(Bt, T, D)), _rel(st, g["state_out"].reshape(Bt, D, K - 1)))
    y, st = impl(g["short_x"].reshape(Bt, 2, D).astype(np.float32), w, bias, state, silu=False)
    return max(worst, _rel(y, g["short_y"].reshape(Bt, 2, D)),
               _rel(st, g["short_state_out"].reshape(Bt, D, K - 1)))


def pin_numpy_convolve(impl) -> float:
    """Per channel the layer is a truncated full convolution (numpy.convolve)
    of the window-prefixed input with the reversed kernel, plus the bias."""
    rng = np.random.default_rng(10)
    worst = 0.0
    for Bt, T, D, K in ((2, 11, 3, 4), (1, 7, 5, 2), (1, 3, 2, 4), (2, 6, 1, 3)):
        x, w, b, s = _rand(rng, Bt, T, D, K)
        y, st = impl(x, w, b, s, silu=False)
        ref = np.empty((Bt, T, D))
        ref_st = np.empty((Bt, D, K - 1))
        for bb in range(Bt):
            for c in range(D):
                xp = np.concatenate([s[bb, c], x[bb, :, c].astype(np.float64)])
                full = np.convolve(xp, w[c, ::-1].astype(np.float64))
                ref[bb, :, c] = full[K - 1:K - 1 + T] + b[c]
                ref_st[bb, c] = xp[T:]
        worst = max(worst, _rel(y, ref), _rel(st, ref_st))
    return worst


def pin_torch_conv1d(impl) -> float:
    """A grouped convolution with one group per channel and k-1 leading
    padding frames (torch.nn.functional.conv1d in float64, the window spliced
    in front of the sequence) gives the same outputs, SiLU included."""
    rng = np.random.default_rng(20)
    worst = 0.0
    for Bt, T, D, K, silu in ((2, 13, 4, 4, False), (1, 9, 6, 4, True), (3, 5, 2, 3, True)):
        x, w, b, s = _rand(rng, Bt, T, D, K)
        y, st = impl(x, w, b, s, silu=silu)
        seq = torch.cat([torch.from_numpy(s), torch.from_numpy(x.astype(np.float64)).transpose(1, 2)], 2)
        ref = torch.nn.functional.conv1d(seq, torch.from_numpy(w.astype(np.float64))[:, None, :],
                                         torch.from_numpy(b.astype(np.float64)), groups=D)
        if silu:
            ref = torch.nn.functional.silu(ref)
        worst = max(worst, _rel(y, ref.transpose(1, 2).numpy()), _rel(st, seq[:, :, T:].numpy()))
    return worst


def pin_impulse_response(impl) -> float:
    """A unit impulse at token t0 of one channel, from a zero window and no
    bias, writes that channel's kernel reversed into y[t0..t0+k-1] and
    nothing anywhere else: this fixes the orientation of the window."""
    K, D, T, t0 = 4, 3, 9, 2
    w = np.arange(1, D * K + 1, dtype=np.float32).reshape(D, K)
    worst = 0.0
    for c in range(D):
        x = np.zeros((1, T, D), np.float32)
        x[0, t0, c] = 1.0
        y, st = impl(x, w, None, None, silu=False)
        ref = np.zeros((1, T, D))
        ref[0, t0:t0 + K, c] = w[c, ::-1]
        worst = max(worst, _rel(y, ref), _rel(st, np.zeros((1, D, K - 1))))
    return worst


def pin_closed_forms(impl) -> float:
    """k = 1 is y = w x + b with an empty window; a constant input after a
    window of the same constant gives (sum w) v + b at every token; SiLU
    equals z * logistic(z) (scipy.special.expit) and is 0 at z = 0."""
    rng = np.random.default_rng(30)
    worst = 0.0
    x, w, b, _ = _rand(rng, 2, 6, 5, 1, state=False)
    y, st = impl(x, w, b, None, silu=False)
    worst = max(worst, _rel(y, x.astype(np.float64) * w[:, 0] + b), 0.0 if st.size == 0 else 1.0)
    v = 0.75
    x = np.full((1, 7, 3), v, np.float32)
    w = rng.uniform(-1, 1, (3, 4)).astype(np.float32)
    b = rng.uniform(-1, 1, 3).astype(np.float32)
    y, st = impl(x, w, b, np.full((1, 3, 3), v), silu=False)
    ref = np.broadcast_to(w.astype(np.float64).sum(1) * v + b, (1, 7, 3))
    worst = max(worst, _rel(y, ref), _rel(st, np.full((1, 3, 3), v)))
    # SiLU at chosen pre-activations: k = 1, w = 1, bias 0 gives z = x
    z = np.array([[[-30.0, -4.0, -1.0, -0.25, 0.0, 0.5, 2.0, 30.0]]], np.float32)
    y, _ = impl(z, np.ones((z.shape[2], 1), np.float32), None, None, silu=True)
    ref = z.astype(np.float64) * expit(z.astype(np.float64))
    worst = max(worst, _rel(y, ref), float(abs(y[0, 0, 4])))
    return worst


def pin_continuation(impl) -> float:
    """O(1) cache: the sequence split anywhere (also into single tokens), the
    window of one part seeding the next, equals one pass over the whole."""
    rng = np.random.default_rng(40)
    x, w, b, s = _rand(rng, 2, 12, 3, 4)
    full_y, full_s = impl(x, w, b, s, silu=True)
    worst = 0.0
    for cuts in ((5,), (1, 2), (3, 4, 9), tuple(range(1, 12))):
        st, ys, lo = s, [], 0
        for hi in cuts + (12,):
            y, st = impl(x[:, lo:hi], w, b, st, silu=True)
            ys.append(y)
            lo = hi
        worst = max(worst, _rel(np.concatenate(ys, 1), full_y), _rel(st, full_s))
    return worst


def pin_empty_sequence(impl) -> float:
    """T = 0 returns no outputs and hands the window back unchanged."""
    rng = np.random.default_rng(50)
    _, w, b, s = _rand(rng, 2, 1, 3, 4)
    y, st = impl(np.zeros((2, 0, 3), np.float32), w, b, s, silu=True)
    return max(0.0 if y.shape == (2, 0, 3) else 1.0, _rel(st, s))


CONV_PINS = {
    "hand_example": pin_hand_example,
    "numpy_convolve": pin_numpy_convolve,
    "torch_conv1d": pin_torch_conv1d,
    "impulse_response": pin_impulse_response,
    "closed_forms": pin_closed_forms,
    "continuation": pin_continuation,
    "empty_sequence": pin_empty_sequence,
}

# fp64 arithmetic against fp64 references: the only differences are rounding
CONV_PIN_TOL = 1e-12
