"""Pins of the CPU oracle (runs without a GPU).

The oracle is trusted only because it agrees with things other than itself:
hand-worked examples, the dense dual form (Eq. 3), the chunked algorithm at
every chunk size, prefix continuation (O(1) cache), closed forms, linearity
and a 50-digit evaluation.  Source: "Compiler-First State Space Duality and
Portable O(1) Autoregressive Caching" (Background; SSD properties; O(1) cache).
"""
import numpy as np
import pytest

import oracle
from pins import ALL_PINS, oracle_impl, np_inputs
from ssd_inputs import make_tiny, make_inputs, WORKLOADS


@pytest.mark.parametrize("name", list(ALL_PINS))
def test_oracle_pin(name):
    fn, tol = ALL_PINS[name]
    err = fn(oracle_impl)
    assert err <= tol, f"pin {name}: error {err:.3e} > {tol:.1e}"


def test_oracle_thread_count_bitwise():
    inp = np_inputs(make_tiny(3, 64, 5, 4, 6, 1, seed=9), with_h0=True)
    a = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["dt_bias"],
                    inp["h0"], nthreads=1)
    b = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], inp["dt_bias"],
                    inp["h0"], nthreads=7)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_oracle_step_is_one_token_scan():
    inp = np_inputs(make_tiny(2, 1, 3, 4, 5, 1, seed=11), with_h0=True)
    y, s = oracle.step(inp["h0"], inp["x"][:, 0], inp["dt"][:, 0], inp["A"], inp["B"][:, 0],
                       inp["C"][:, 0], inp["D"], inp["dt_bias"])
    y2, s2 = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                         inp["dt_bias"], inp["h0"])
    assert np.array_equal(y, y2[:, 0]) and np.array_equal(s, s2)


def test_oracle_empty_sequence_returns_initial_state():
    inp = np_inputs(make_tiny(1, 1, 2, 3, 4, 1, seed=12), with_h0=True)
    e = {k: (v[:, :0] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    y, s = oracle.scan(e["x"], e["dt"], e["A"], e["B"], e["C"], e["D"], e["dt_bias"], e["h0"])
    assert y.shape == (1, 0, 2, 3) and np.array_equal(s, inp["h0"])


def test_generator_is_seeded_and_has_the_stated_distributions():
    w = WORKLOADS["tiny_f32"]
    a, b = make_inputs(w), make_inputs(w)
    for k in a:
        assert a[k].equal(b[k]), k
    c = make_inputs(w, seed=w.seed + 1)
    assert not a["x"].equal(c["x"])
    import torch
    A = a["A"]
    assert bool((A <= -1.0).all() and (A >= -16.0 * (1 + 1e-6)).all())
    u = torch.nn.functional.softplus(a["dt_bias"].double())
    assert bool((u >= 1e-3 * (1 - 1e-5)).all() and (u <= 0.1 * (1 + 1e-5)).all())
    N = w.dstate
    assert abs(float(a["B"].double().std()) * np.sqrt(N) - 1.0) < 0.05
    assert abs(float(a["x"].double().std()) - 1.0) < 0.05
    assert abs(float(a["dt"].double().std()) - 0.5) < 0.03
    wb = WORKLOADS["m2p7_bf16"].with_(seqlen=64)
    t = make_inputs(wb)
    assert t["x"].dtype == torch.bfloat16 and t["B"].dtype == torch.bfloat16
    assert t["dt"].dtype == torch.float32
