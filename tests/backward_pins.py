"""Pins that tie an implementation of the scan's gradients to facts other than
itself.

Each pin takes `impl` with the signature of oracle.scan_backward (numpy inputs,
keyword dy / dfinal, returns a dict of float64 gradients) and returns the
worst relative error it saw.  They are applied to the C oracle
(test_backward_oracle.py) and to broken copies of a plain adjoint loop.

Sources: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching", Background (Eq. 2: the recurrence being differentiated) and
Implementation (softplus and clip on Delta).  The gradients themselves are
fixed by the mathematics: central finite differences of the forward
recurrence, and reverse-mode differentiation of an independent float64
torch recurrence (torch.autograd).
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
from ssd_inputs import as_f32_numpy, make_inputs, make_tiny

GRAD_OF = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD",
           "dt_bias": "ddt_bias", "h0": "dh0"}

CASES = [
    # (Bt, T, H, P, N, G, softplus, dt_max)
    (1, 9, 2, 3, 4, 1, True, 0.5),
    (2, 13, 4, 2, 3, 2, True, 0.5),
    (1, 70, 2, 2, 2, 1, False, 10.0),     # longer than one oracle segment of 64 tokens
    (1, 11, 3, 2, 2, 3, True, 0.06),      # a low dt_max: many clipped steps (zero gradient)
]


def case_inputs(i, seed_base=700):
    Bt, T, H, P, N, G, sp, hi = CASES[i]
    w = make_tiny(Bt, T, H, P, N, G, 32, "f32", seed=seed_base + i)
    inp = {k: as_f32_numpy(v) for k, v in make_inputs(w, with_initial_state=True).items()}
    inp["h0"] = inp["h0"].astype(np.float64)
    if not sp:
        # Delta = dt + dt_bias directly: keep it positive
        inp["dt"] = np.abs(inp["dt"]).astype(np.float32) * np.float32(0.4) + np.float32(0.01)
        inp["dt_bias"] = np.abs(inp["dt_bias"]).astype(np.float32) * np.float32(0.01)
    rng = np.random.default_rng(seed_base + 50 + i)
    dy = rng.standard_normal(inp["x"].shape)
    dfinal = rng.standard_normal(inp["h0"].shape)
    return inp, dy, dfinal, dict(dt_softplus=sp, dt_min=1e-4, dt_max=hi)


def call(impl, inp, dy, dfinal, kw):
    return impl(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["dt_bias"],
                inp["h0"], dy=dy, dfinal=dfinal, **kw)


def loss(inp, dy, dfinal, kw):
    y, f = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                       inp["dt_bias"], inp["h0"], **kw)
    return float((dy * y).sum() + (dfinal * f).sum())


def pin_finite_differences(impl) -> float:
    """Central differences of the fp64 forward recurrence, element by element
    (six elements of every input per case; the step is the exact float32
    difference of the perturbed inputs)."""
    worst = 0.0
    for i in range(len(CASES)):
        inp, dy, dfinal, kw = case_inputs(i)
        g = call(impl, inp, dy, dfinal, kw)
        rng = np.random.default_rng(900 + i)
        for name, gname in GRAD_OF.items():
            arr = inp[name]
            scale = max(float(np.abs(g[gname]).max()), 1e-12)
            for _ in range(6):
                idx = tuple(int(rng.integers(0, s)) for s in arr.shape)
                v = float(arr[idx])
                eps = 1e-4 * max(1.0, abs(v))
                up, dn = arr.copy(), arr.copy()
                up[idx] = v + eps
                dn[idx] = v - eps
                step = float(up[idx]) - float(dn[idx])
                fd = (loss({**inp, name: up}, dy, dfinal, kw) -
                      loss({**inp, name: dn}, dy, dfinal, kw)) / step
                worst = max(worst, abs(fd - float(g[gname][idx])) / scale)
    return worst


def torch_recurrence_grads(inp, dy, dfinal, kw):
    """Reverse-mode gradients of a float64 torch recurrence written token by
    token (Background, Eq. 2; softplus and clip on Delta)."""
    t = {k: torch.tensor(np.asarray(v, np.float64), requires_grad=True) for k, v in inp.items()}
    Bt, T, H, P = t["x"].shape
    G, N = t["B"].shape[2], t["B"].shape[3]
    hpg = H // G
    lo, hi = float(np.float32(kw["dt_min"])), float(np.float32(kw["dt_max"]))
    z = t["dt"] + t["dt_bias"][None, None, :]
    d = torch.nn.functional.softplus(z) if kw["dt_softplus"] else z
    d = torch.clamp(d, lo, hi)
    gi = torch.arange(H) // hpg
    Bh = t["B"][:, :, gi, :]                      # [Bt,T,H,N]
    Ch = t["C"][:, :, gi, :]
    h = t["h0"]
    ys = []
    for s in range(T):
        ab = torch.exp(d[:, s] * t["A"][None, :])                       # [Bt,H]
        h = ab[..., None, None] * h + (d[:, s][..., None] * t["x"][:, s])[..., None] * Bh[:, s][:, :, None, :]
        ys.append(torch.einsum("bhpn,bhn->bhp", h, Ch[:, s]) + t["D"][None, :, None] * t["x"][:, s])
    y = torch.stack(ys, 1)
    L = (torch.from_numpy(dy) * y).sum() + (torch.from_numpy(dfinal) * h).sum()
    L.backward()
    return {GRAD_OF[k]: t[k].grad.numpy() for k in GRAD_OF}


def pin_autograd(impl) -> float:
    """Every gradient against torch.autograd of an independent float64
    recurrence."""
    worst = 0.0
    for i in range(len(CASES)):
        inp, dy, dfinal, kw = case_inputs(i)
        g = call(impl, inp, dy, dfinal, kw)
        ref = torch_recurrence_grads(inp, dy, dfinal, kw)
        for k, r in ref.items():
            scale = max(float(np.abs(r).max()), 1e-12)
            worst = max(worst, float(np.abs(g[k] - r).max()) / scale)
    return worst


def pin_linearity(impl) -> float:
    """Gradients are linear in the cotangents (dy, dfinal)."""
    inp, dy, dfinal, kw = case_inputs(1)
    rng = np.random.default_rng(77)
    dy2, df2 = rng.standard_normal(dy.shape), rng.standard_normal(dfinal.shape)
    g1 = call(impl, inp, dy, dfinal, kw)
    g2 = call(impl, inp, dy2, df2, kw)
    g3 = call(impl, inp, dy + 2.0 * dy2, dfinal + 2.0 * df2, kw)
    worst = 0.0
    for k in GRAD_OF.values():
        r = g1[k] + 2.0 * g2[k]
        worst = max(worst, float(np.abs(g3[k] - r).max()) / max(float(np.abs(r).max()), 1e-12))
    return worst


def pin_clipped_steps_have_zero_dt_gradient(impl) -> float:
    """Where softplus(dt + bias) lies outside [dt_min, dt_max], Delta is a
    constant: its dt gradient is exactly zero."""
    inp, dy, dfinal, kw = case_inputs(3)
    g = call(impl, inp, dy, dfinal, kw)
    z = inp["dt"].astype(np.float64) + inp["dt_bias"][None, None, :].astype(np.float64)
    sp = np.logaddexp(0.0, z)
    clipped = (sp < float(np.float32(kw["dt_min"]))) | (sp > float(np.float32(kw["dt_max"])))
    assert clipped.any() and (~clipped).any()
    return float(np.abs(g["ddt"][clipped]).max())


BACKWARD_PINS = {
    "finite_differences": (pin_finite_differences, 1e-5),
    "autograd": (pin_autograd, 1e-10),
    "linearity": (pin_linearity, 1e-12),
    "clipped_zero": (pin_clipped_steps_have_zero_dt_gradient, 0.0),
}
