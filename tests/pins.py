"""Pins that tie an SSD scan implementation to facts other than itself.

Each pin takes an implementation `impl` with the signature of oracle.scan
(numpy/float32 inputs, returns float64 (y, final_state)) and returns the worst
error it saw.  The same pins are applied to the C oracle (test_oracle_pins.py)
and to deliberately broken copies of the recurrence (test_pin_mutants.py) to
show that a plausible slip fails at least one of them.

Sources: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching" -- Background (Eq. 2 recurrence, Eq. 3 dual form), SSD properties
(chunked recurrence), O(1) cache (prefill seeds the cache, decode continues).
"""
from __future__ import annotations

import math

import mpmath as mp
import numpy as np

import oracle
from oracle.brute import brute
from oracle.chunked import chunked
from oracle.dual_form import dual_form
from oracle.metrics import state_err, y_err
from ssd_inputs import make_inputs, make_tiny, as_f32_numpy

import golden_io


def np_inputs(w, with_h0=False, seed=None):
    t = make_inputs(w, seed=seed, with_initial_state=with_h0)
    out = {k: as_f32_numpy(v) for k, v in t.items()}
    if with_h0:
        out["h0"] = out["h0"].astype(np.float64)
    return out


def call(impl, inp, **kw):
    return impl(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                inp.get("dt_bias"), inp.get("h0"), **kw)


def _err(a, b):
    return max(y_err(a[0], b[0]), state_err(a[1], b[1]))


TINY_CASES = [
    # (Bt, T, H, P, N, G, h0)
    (1, 24, 2, 3, 4, 1, False),
    (2, 17, 4, 2, 3, 2, True),
    (1, 40, 3, 4, 2, 3, True),
]


def pin_dual_form(impl) -> float:
    """Eq. 3: the recurrence equals the dense lower-triangular materialisation."""
    worst = 0.0
    for i, (Bt, T, H, P, N, G, h0) in enumerate(TINY_CASES):
        inp = np_inputs(make_tiny(Bt, T, H, P, N, G, seed=100 + i), with_h0=h0)
        worst = max(worst, _err(call(impl, inp), call(dual_form, inp)))
    return worst


def pin_chunk_invariance(impl) -> float:
    """Chunked recurrence: the chunked algorithm at every chunk size (dividing
    T or not, from 1 to T) reproduces the recurrence."""
    inp = np_inputs(make_tiny(2, 36, 3, 3, 4, 1, seed=200), with_h0=True)
    ref = call(impl, inp)
    worst = 0.0
    for L in (1, 2, 5, 7, 12, 36, 50):
        worst = max(worst, _err(ref, call(chunked, inp, chunk=L)))
    return worst


def pin_continuation(impl) -> float:
    """O(1) cache: a prefill of T1 tokens followed by T2 single steps, or by a
    second scan seeded with the first one's final state, equals one scan of
    T1 + T2 tokens."""
    inp = np_inputs(make_tiny(2, 30, 2, 3, 4, 1, seed=300), with_h0=True)
    full = call(impl, inp)
    T1 = 19
    first = {k: (v[:, :T1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y1, s1 = call(impl, first)
    second = {k: (v[:, T1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    second["h0"] = s1
    y2, s2 = call(impl, second)
    worst = _err(full, (np.concatenate([y1, y2], axis=1), s2))
    # token by token
    s = s1
    ys = [y1]
    for t in range(T1, inp["x"].shape[1]):
        one = {k: (v[:, t:t + 1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        one["h0"] = s
        yt, s = call(impl, one)
        ys.append(yt)
    worst = max(worst, _err(full, (np.concatenate(ys, axis=1), s)))
    return worst


def pin_closed_forms(impl) -> float:
    """Special cases with closed forms (Eq. 2 unrolled by hand)."""
    worst = 0.0
    rng = np.random.default_rng(400)
    f32 = np.float32
    # (a) T = 1 from zero state: h = d x (x) B, y = d (C.B) x + D x
    Bt, H, P, N = 2, 3, 4, 5
    x = rng.standard_normal((Bt, 1, H, P)).astype(f32)
    dt = rng.uniform(0.01, 0.4, (Bt, 1, H)).astype(f32)
    A = -rng.uniform(1, 16, H).astype(f32)
    B = rng.standard_normal((Bt, 1, 1, N)).astype(f32)
    C = rng.standard_normal((Bt, 1, 1, N)).astype(f32)
    D = rng.standard_normal(H).astype(f32)
    y, fin = impl(x, dt, A, B, C, D, None, None, dt_softplus=False)
    d = dt.astype(np.float64)[:, 0]                                       # [Bt,H]
    h_ref = d[:, :, None, None] * x[:, 0, :, :, None] * B[:, 0, 0][:, None, None, :]
    cb = (C[:, 0, 0].astype(np.float64) * B[:, 0, 0]).sum(-1)            # [Bt]
    y_ref = (d * cb[:, None])[:, :, None] * x[:, 0] + D.astype(np.float64)[None, :, None] * x[:, 0]
    worst = max(worst, state_err(fin, h_ref), y_err(y, y_ref[:, None]))
    # (b) constant inputs, P = N = 1: geometric series
    T = 50
    dv, Av, xv, bv, cv, Dv = 0.25, -1.5, 0.75, 1.25, -0.5, 0.5
    x = np.full((1, T, 1, 1), xv, f32)
    dt = np.full((1, T, 1), dv, f32)
    B = np.full((1, T, 1, 1), bv, f32)
    C = np.full((1, T, 1, 1), cv, f32)
    y, fin = impl(x, dt, np.array([Av], f32), B, C, np.array([Dv], f32), None, None,
                  dt_softplus=False)
    al = math.exp(dv * Av)
    t = np.arange(T)
    h_ref = dv * bv * xv * (1 - al ** (t + 1)) / (1 - al)
    y_ref = cv * h_ref + Dv * xv
    worst = max(worst, float(np.abs(y[0, :, 0, 0] - y_ref).max() / np.abs(y_ref).max()),
                abs(fin[0, 0, 0, 0] - h_ref[-1]) / abs(h_ref[-1]))
    # (c) B = 0: y = D x exactly, state stays at zero
    inp = np_inputs(make_tiny(1, 20, 2, 3, 4, 1, seed=401))
    inp["B"] = np.zeros_like(inp["B"])
    y, fin = call(impl, inp)
    exact = inp["D"].astype(np.float64)[None, None, :, None] * inp["x"]
    worst = max(worst, float(np.abs(y - exact).max()) * 1e6, float(np.abs(fin).max()) * 1e6)
    # (d) A = 0: the state is a running sum of d x (x) B (numpy cumsum)
    inp = np_inputs(make_tiny(1, 20, 2, 3, 4, 1, seed=402))
    inp["A"] = np.zeros_like(inp["A"])
    y, fin = call(impl, inp)
    z = inp["dt"].astype(np.float64) + inp["dt_bias"][None, None, :]
    d = np.clip(np.logaddexp(0.0, z), float(f32(1e-4)), float(f32(0.5)))  # [1,T,H]
    Bb = inp["B"][:, :, 0, :].astype(np.float64)                        # [1,T,N]
    terms = d[..., None, None] * inp["x"][..., :, None] * Bb[:, :, None, None, :]
    hs = np.cumsum(terms, axis=1)                                       # [1,T,H,P,N]
    y_ref = np.einsum("bthpn,btn->bthp", hs, inp["C"][:, :, 0, :].astype(np.float64))
    y_ref += inp["D"].astype(np.float64)[None, None, :, None] * inp["x"]
    worst = max(worst, y_err(y, y_ref), state_err(fin, hs[:, -1]))
    # (e) clipping: a huge negative pre-activation pins Delta to dt_min, a huge
    # positive one to dt_max; with x = 0 the state only decays by exp(Delta A)
    x = np.zeros((1, 1, 2, 1), f32)
    dt = np.array([[[-60.0, 60.0]]], f32)
    A = np.array([-1.0, -3.0], f32)
    h0 = np.ones((1, 2, 1, 1))
    y, fin = impl(x, dt, A, np.ones((1, 1, 1, 1), f32), np.ones((1, 1, 1, 1), f32), None,
                  None, h0)
    ref = np.array([math.exp(float(f32(1e-4)) * -1.0), math.exp(float(f32(0.5)) * -3.0)])
    worst = max(worst, float(np.abs(fin[0, :, 0, 0] - ref).max() / ref.max()))
    # (f) softplus itself, at 40 digits, through the same decay read-out
    zs = np.array([-8.0, -1.0, -0.3, 0.0, 0.2, 0.45], f32)
    H = len(zs)
    y, fin = impl(np.zeros((1, 1, H, 1), f32), zs[None, None, :], -np.ones(H, f32),
                  np.ones((1, 1, 1, 1), f32), np.ones((1, 1, 1, 1), f32), None, None,
                  np.ones((1, H, 1, 1)), dt_min=1e-6, dt_max=10.0)
    with mp.workdps(40):
        sp = [float(mp.exp(-mp.log(1 + mp.exp(mp.mpf(float(z)))))) for z in zs]
    worst = max(worst, float(np.abs(fin[0, :, 0, 0] - np.array(sp)).max()))
    return worst


def pin_linearity(impl) -> float:
    """For fixed (Delta, A, B, C, D) the map (x, h0) -> (y, final) is linear:
    splitting x exactly into a high and a low part, the responses to
    (x_hi, 0), (x_lo, 0) and (0, h0) add up to the response to (x, h0)."""
    import torch
    inp = np_inputs(make_tiny(1, 28, 2, 3, 4, 1, seed=500), with_h0=True)
    x = inp["x"]
    x_hi = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    x_lo = (x - x_hi).astype(np.float32)          # exact: the bits bf16 dropped
    assert np.array_equal(x_hi + x_lo, x)
    full = call(impl, inp)
    parts = []
    for xx, hh in ((x_hi, None), (x_lo, None), (np.zeros_like(x), inp["h0"])):
        q = dict(inp)
        q["x"], q["h0"] = xx, hh
        parts.append(call(impl, q))
    y = parts[0][0] + parts[1][0] + parts[2][0]
    f = parts[0][1] + parts[1][1] + parts[2][1]
    return _err(full, (y, f))


def pin_brute_force(impl) -> float:
    """The recurrence at 50 digits bounds the double rounding (T <= 16)."""
    worst = 0.0
    for i, (Bt, T, H, P, N, G) in enumerate([(1, 16, 2, 2, 3, 1), (1, 9, 2, 3, 2, 2)]):
        inp = np_inputs(make_tiny(Bt, T, H, P, N, G, seed=600 + i), with_h0=True)
        worst = max(worst, _err(call(impl, inp), call(brute, inp)))
    return worst


def _golden_inputs(g):
    Bt, T, H, P, N, G = (int(v) for v in g["shape"])
    f32 = np.float32
    return dict(x=g["x"].reshape(Bt, T, H, P).astype(f32), dt=g["dt"].reshape(Bt, T, H).astype(f32),
                A=g["A"].astype(f32), B=g["B"].reshape(Bt, T, G, N).astype(f32),
                C=g["C"].reshape(Bt, T, G, N).astype(f32), D=g["D"].astype(f32)), (Bt, T, H, P, N, G)


def pin_golden(impl) -> float:
    """The hand-worked fixtures under tests/golden/."""
    g = golden_io.load("hand_accumulate.txt")
    inp, (Bt, T, H, P, N, G) = _golden_inputs(g)
    y, fin = impl(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], None, None,
                  dt_softplus=bool(g["softplus"][0]))
    worst = max(float(np.abs(y.reshape(-1) - g["y"]).max()),
                float(np.abs(fin.reshape(-1) - g["final"]).max()))
    g = golden_io.load("hand_decay.txt")
    inp, (Bt, T, H, P, N, G) = _golden_inputs(g)
    y, fin = impl(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], None, None,
                  dt_softplus=bool(g["softplus"][0]))
    al = math.exp(-0.5)
    powers = np.array([1.0, al, al * al])
    y_ref = g["ypoly"].reshape(T, 3) @ powers
    f_ref = g["finalpoly"].reshape(N, 3) @ powers
    worst = max(worst, float(np.abs(y.reshape(-1) - y_ref).max()),
                float(np.abs(fin.reshape(-1) - f_ref).max()))
    return worst


ALL_PINS = {
    "golden": (pin_golden, 1e-12),
    "dual_form": (pin_dual_form, 1e-12),
    "chunk_invariance": (pin_chunk_invariance, 1e-12),
    "continuation": (pin_continuation, 1e-12),
    "closed_forms": (pin_closed_forms, 1e-12),
    "linearity": (pin_linearity, 1e-12),
    "brute_force": (pin_brute_force, 1e-13),
}


def oracle_impl(*a, **kw):
    return oracle.scan(*a, **kw)
