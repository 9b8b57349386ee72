"""The oracle of the scan's gradients against its pins, and planted mistakes
against the pins.

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching", Background (Eq. 2, the recurrence) and Implementation (softplus and
clip on Delta).  The mistakes are planted in a plain numpy adjoint loop on
the CPU, in this test only.
"""
import numpy as np
import pytest

import oracle
from backward_pins import BACKWARD_PINS


@pytest.mark.parametrize("name", list(BACKWARD_PINS))
def test_backward_oracle_pin(name):
    pin, tol = BACKWARD_PINS[name]
    assert pin(oracle.scan_backward) <= tol


def test_backward_oracle_thread_count_bitwise():
    from backward_pins import call, case_inputs
    inp, dy, dfinal, kw = case_inputs(1)
    g1 = call(lambda *a, **k: oracle.scan_backward(*a, nthreads=1, **k), inp, dy, dfinal, kw)
    g8 = call(lambda *a, **k: oracle.scan_backward(*a, nthreads=8, **k), inp, dy, dfinal, kw)
    for k in g1:
        assert np.array_equal(g1[k], g8[k]), k


def test_backward_oracle_dA_is_the_delta_weighted_sum_of_dlda():
    from backward_pins import call, case_inputs
    for i in range(4):
        inp, dy, dfinal, kw = case_inputs(i)
        g = call(oracle.scan_backward, inp, dy, dfinal, kw)
        z = inp["dt"].astype(np.float64) + inp["dt_bias"][None, None, :]
        pre = np.logaddexp(0.0, z) if kw["dt_softplus"] else z
        d = np.clip(pre, float(np.float32(kw["dt_min"])), float(np.float32(kw["dt_max"])))
        assert np.allclose(g["dA"], (d * g["dlda"]).sum(axis=(0, 1)), rtol=1e-12, atol=1e-12)


MUTATIONS = ["decay_uses_h_t", "decay_before_add", "no_dfinal", "dB_no_delta", "dC_prev_state",
             "no_clip_gate", "softplus_grad_wrong", "dD_missing", "dA_missing_delta"]


def make_adjoint(mutation=None):
    def impl(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, dy, dfinal=None,
             dt_softplus=True, dt_min=1e-4, dt_max=0.5):
        x = np.asarray(x, np.float64)
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        hpg = H // G
        lo, hi = float(np.float32(dt_min)), float(np.float32(dt_max))
        out = {"dx": np.zeros((Bt, T, H, P)), "ddt": np.zeros((Bt, T, H)), "dA": np.zeros(H),
               "dB": np.zeros((Bt, T, G, N)), "dC": np.zeros((Bt, T, G, N)), "dD": np.zeros(H),
               "ddt_bias": np.zeros(H), "dh0": np.zeros((Bt, H, P, N))}
        for b in range(Bt):
            for h in range(H):
                g = h // hpg
                z = np.asarray(dt, np.float64)[b, :, h] + (0.0 if dt_bias is None else float(dt_bias[h]))
                pre = np.logaddexp(0.0, z) if dt_softplus else z
                d = np.clip(pre, lo, hi)
                Ah = float(A[h])
                Bg = np.asarray(B, np.float64)[b, :, g]
                Cg = np.asarray(C, np.float64)[b, :, g]
                X = x[b, :, h]
                hs = [np.zeros((P, N)) if h0 is None else np.array(h0[b, h], np.float64)]
                for t in range(T):
                    hs.append(np.exp(d[t] * Ah) * hs[-1] + d[t] * np.outer(X[t], Bg[t]))
                Gm = np.zeros((P, N)) if (dfinal is None or mutation == "no_dfinal") else \
                    np.array(dfinal[b, h], np.float64)
                for t in range(T - 1, -1, -1):
                    ab = np.exp(d[t] * Ah)
                    dyt = np.asarray(dy, np.float64)[b, t, h]
                    if mutation == "decay_before_add":
                        Gm = Gm * ab
                    Gm = Gm + np.outer(dyt, Cg[t])
                    hst = hs[t] if mutation == "dC_prev_state" else hs[t + 1]
                    out["dC"][b, t, g] += dyt @ hst
                    gb = Gm @ Bg[t]
                    out["dx"][b, t, h] = d[t] * gb + (float(D[h]) if D is not None else 0.0) * dyt
                    out["dB"][b, t, g] += (1.0 if mutation == "dB_no_delta" else d[t]) * (X[t] @ Gm)
                    hprev = hs[t + 1] if mutation == "decay_uses_h_t" else hs[t]
                    dec = float((Gm * hprev).sum())
                    dd = float(gb @ X[t]) + Ah * ab * dec
                    out["dA"][h] += (1.0 if mutation == "dA_missing_delta" else d[t]) * ab * dec
                    if mutation != "dD_missing":
                        out["dD"][h] += float(dyt @ X[t])
                    gate = 1.0 if (mutation == "no_clip_gate" or lo <= pre[t] <= hi) else 0.0
                    if dt_softplus:
                        gate *= pre[t] if mutation == "softplus_grad_wrong" else 1.0 / (1.0 + np.exp(-z[t]))
                    out["ddt"][b, t, h] = dd * gate
                    out["ddt_bias"][h] += dd * gate
                    if mutation != "decay_before_add":
                        Gm = Gm * ab
                out["dh0"][b, h] = Gm
        return out
    return impl


def test_unbroken_adjoint_passes_every_pin():
    impl = make_adjoint()
    for name, (pin, tol) in BACKWARD_PINS.items():
        assert pin(impl) <= tol, name


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_each_planted_mistake_fails_a_pin(mutation):
    impl = make_adjoint(mutation)
    failed = []
    for name, (pin, tol) in BACKWARD_PINS.items():
        try:
            ok = pin(impl) <= tol
        except AssertionError:
            ok = False
        if not ok:
            failed.append(name)
    assert failed, f"no pin caught {mutation}"
