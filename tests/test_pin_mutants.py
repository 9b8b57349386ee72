"""Planted mistakes: a plausible slip in the recurrence must fail some pin.

A plain numpy copy of the recurrence (Background, Eq. 2 of "Compiler-First
State Space Duality and Portable O(1) Autoregressive Caching") is broken in
one place at a time.  The unbroken copy passes every pin; each broken copy
must fail at least one, which shows the pins can see that kind of error.
The mistakes are planted on the CPU, in this test only.
"""
import numpy as np
import pytest

from pins import ALL_PINS


def make_recurrence(mutation=None):
    def impl(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, dt_softplus=True,
             dt_min=1e-4, dt_max=0.5):
        x = np.asarray(x, np.float64)
        Bt, T, H, P = x.shape
        G, N = B.shape[2], B.shape[3]
        y = np.zeros((Bt, T, H, P))
        fin = np.zeros((Bt, H, P, N))
        lo, hi = float(np.float32(dt_min)), float(np.float32(dt_max))
        for b in range(Bt):
            for h in range(H):
                g = (h % G) if mutation == "group_mod" else h // (H // G)
                S = np.zeros((P, N)) if (h0 is None or mutation == "h0_ignored") else \
                    np.array(h0[b, h], np.float64)
                prev_d = 0.0
                for t in range(T):
                    z = float(dt[b, t, h])
                    if dt_bias is not None and mutation != "bias_ignored":
                        z += float(dt_bias[h])
                    d = (max(z, 0.0) + np.log1p(np.exp(-abs(z)))) if (dt_softplus and mutation != "no_softplus") else z
                    if mutation != "no_clip":
                        d = min(max(d, lo), hi)
                    Ah = float(A[h]) * (-1.0 if mutation == "sign_A" else 1.0)
                    dd = prev_d if mutation == "decay_lag" else d
                    abar = np.exp(dd * Ah)
                    prev_d = d
                    Bv = np.asarray(C if mutation == "swap_BC" else B, np.float64)[b, t, g]
                    Cv = np.asarray(B if mutation == "swap_BC" else C, np.float64)[b, t, g]
                    if mutation == "zoh_input":
                        scale = (abar - 1.0) / Ah if Ah != 0 else d
                    elif mutation == "no_delta_input":
                        scale = 1.0
                    else:
                        scale = d
                    if mutation == "y_before_update":
                        yt = S @ Cv
                    S = abar * S + scale * np.outer(x[b, t, h], Bv)
                    if mutation != "y_before_update":
                        yt = S @ Cv
                    if D is not None and mutation != "drop_D":
                        yt = yt + float(D[h]) * x[b, t, h]
                    y[b, t, h] = yt
                fin[b, h] = S
        return y, fin
    return impl


MUTATIONS = ["drop_D", "y_before_update", "sign_A", "swap_BC", "group_mod", "no_softplus",
             "no_clip", "zoh_input", "no_delta_input", "decay_lag", "h0_ignored",
             "bias_ignored"]


def test_unbroken_copy_passes_every_pin():
    impl = make_recurrence(None)
    for name, (fn, tol) in ALL_PINS.items():
        if name == "brute_force":
            tol = 1e-12  # numpy's own summation order
        assert fn(impl) <= tol, name


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_mutant_fails_some_pin(mutation):
    impl = make_recurrence(mutation)
    failed = []
    for name, (fn, tol) in ALL_PINS.items():
        try:
            err = fn(impl)
        except Exception:  # a mutant that crashes a pin is caught too
            err = float("inf")
        if not err <= max(tol, 1e-12):
            failed.append(name)
    assert failed, f"mutation {mutation} slipped past every pin"
