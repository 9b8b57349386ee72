"""The conv1d oracle against its pins, and planted mistakes against the pins.

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching", O(1) cache section and Setup (depthwise convolution of width k = 4
over the cached k-1 previous inputs).  The mistakes are planted in a plain
numpy loop on the CPU, in this test only.
"""
import numpy as np
import pytest

import oracle
from conv_pins import CONV_PINS, CONV_PIN_TOL


@pytest.mark.parametrize("name", list(CONV_PINS))
def test_conv_oracle_pin(name):
    assert CONV_PINS[name](oracle.conv1d) <= CONV_PIN_TOL


def test_conv_oracle_thread_count_bitwise():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((3, 40, 17)).astype(np.float32)
    w = rng.uniform(-0.5, 0.5, (17, 4)).astype(np.float32)
    b = rng.uniform(-0.5, 0.5, 17).astype(np.float32)
    s = rng.standard_normal((3, 17, 3))
    y1, s1 = oracle.conv1d(x, w, b, s, silu=True, nthreads=1)
    y8, s8 = oracle.conv1d(x, w, b, s, silu=True, nthreads=8)
    assert np.array_equal(y1, y8) and np.array_equal(s1, s8)


def test_conv_oracle_step_is_one_token():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((2, 1, 5)).astype(np.float32)
    w = rng.uniform(-0.5, 0.5, (5, 4)).astype(np.float32)
    s = rng.standard_normal((2, 5, 3))
    y, st = oracle.conv1d_step(s, x[:, 0], w, None, silu=True)
    y2, st2 = oracle.conv1d(x, w, None, s, silu=True)
    assert np.array_equal(y, y2[:, 0]) and np.array_equal(st, st2)


MUTATIONS = ["flipped_kernel", "no_bias", "state_reversed", "state_ignored",
             "state_out_oldest", "sigmoid_only", "window_lag", "silu_always", "bias_per_token"]


def make_loop(mutation=None):
    def impl(x, w, bias=None, state=None, *, silu=False):
        x = np.asarray(x, np.float64)
        w = np.asarray(w, np.float64)
        Bt, T, D = x.shape
        K = w.shape[1]
        y = np.zeros((Bt, T, D))
        st = np.zeros((Bt, D, K - 1))
        for b in range(Bt):
            for c in range(D):
                if state is None or mutation == "state_ignored":
                    win = np.zeros(K - 1)
                else:
                    win = np.asarray(state[b, c], np.float64)
                    if mutation == "state_reversed":
                        win = win[::-1]
                xp = np.concatenate([win, x[b, :, c]])
                wc = w[c, ::-1] if mutation == "flipped_kernel" else w[c]
                for t in range(T):
                    if mutation == "window_lag":
                        seg = np.concatenate([[0.0], xp])[t:t + K]
                    else:
                        seg = xp[t:t + K]
                    z = float(wc @ seg)
                    if bias is not None and mutation != "no_bias":
                        z += float(bias[c]) * ((t + 1) if mutation == "bias_per_token" else 1)
                    if silu or mutation == "silu_always":
                        z = 1.0 / (1.0 + np.exp(-z)) if mutation == "sigmoid_only" else z / (1.0 + np.exp(-z))
                    y[b, t, c] = z
                st[b, c] = xp[:K - 1] if mutation == "state_out_oldest" else xp[T:]
        return y, st
    return impl


def test_unbroken_loop_passes_every_pin():
    impl = make_loop()
    for name, pin in CONV_PINS.items():
        assert pin(impl) <= CONV_PIN_TOL, name


@pytest.mark.parametrize("mutation", MUTATIONS)
def test_each_planted_mistake_fails_a_pin(mutation):
    impl = make_loop(mutation)
    failed = [name for name, pin in CONV_PINS.items() if not pin(impl) <= CONV_PIN_TOL]
    assert failed, f"no pin caught {mutation}"
