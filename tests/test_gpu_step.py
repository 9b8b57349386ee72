"""GPU parity of ssd_step (one decode token, state updated in place) against
the CPU oracle, and of prefill-then-decode against a longer prefill.

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching", O(1) cache section (one recurrence step per token from the
fixed-size (B,H,P,N) state; prefill initialises the cache with its final
state).  Error metric and bars as in test_gpu_scan.py.
"""
import pytest
import torch

import oracle
from gpu_util import TOL, announce, need_gpu, oracle_scan, slice_bh, state_err, step_y_err, to_dev, y_err
from ssd_inputs import DECODE_PREFILL, DECODE_STEPS, WORKLOADS, make_inputs, make_tiny

pytestmark = pytest.mark.gpu


def gpu_step(ssd, d, state, t):
    return ssd.ssd_step(state, d["x"][:, t].contiguous(), d["dt"][:, t].contiguous(), d["A"],
                        d["B"][:, t].contiguous(), d["C"][:, t].contiguous(), d.get("D"),
                        dt_bias=d.get("dt_bias"))


STEP_CASES = [
    # (Bt, H, P, N, G, dtype)
    (1, 2, 16, 16, 1, "f32"),
    (3, 4, 32, 64, 2, "f32"),
    (2, 8, 64, 128, 1, "f32"),
    (2, 3, 128, 32, 3, "f32"),
    (4, 4, 64, 128, 1, "bf16"),
    (1, 6, 16, 16, 2, "bf16"),
    (2, 2, 128, 128, 1, "bf16"),
    (32, 64, 128, 64, 2, "f32"),      # 2048 slices: the row-split shape of large batches
]


@pytest.mark.parametrize("case", STEP_CASES, ids=lambda c: "x".join(map(str, c)))
def test_step_tiny_shapes(case):
    """A few consecutive steps from a random state, each against the oracle."""
    need_gpu()
    import state_space_model_amd as ssd
    Bt, H, P, N, G, dt = case
    w = make_tiny(Bt, 5, H, P, N, G, 32, dt, seed=2000 + STEP_CASES.index(case))
    inp = make_inputs(w, with_initial_state=True)
    announce(f"step tiny {case}")
    d = to_dev(inp)
    state = d["h0"].clone()
    ref_state = inp["h0"].double().numpy()
    ptr = state.data_ptr()
    for t in range(5):
        y = gpu_step(ssd, d, state, t)
        torch.cuda.synchronize()
        y_ref, ref_state = oracle.step(ref_state, inp["x"][:, t], inp["dt"][:, t], inp["A"],
                                       inp["B"][:, t], inp["C"][:, t], inp["D"], inp["dt_bias"])
        assert step_y_err(y, y_ref) <= TOL[dt], (t, step_y_err(y, y_ref))
        assert state_err(state, ref_state) <= TOL[dt], (t, state_err(state, ref_state))
    assert state.data_ptr() == ptr  # updated in place


@pytest.mark.parametrize("batch", [1, 16, 64])
def test_decode_after_prefill_matches_longer_prefill(batch):
    """2.7B-shaped cached decode: prefill 4096 tokens with ssd_chunk_scan, then
    1024 ssd_step calls.  Every (b, h) sequence is recomputed by the oracle
    over all 5120 tokens (one batch row at a time); the decoded outputs and
    the state after the last step are compared with it.  The decoded state
    must also equal a GPU prefill over all 5120 tokens within the bf16 bar."""
    need_gpu()
    import state_space_model_amd as ssd
    w = WORKLOADS["m2p7_decode"].with_(batch=batch)
    inp = make_inputs(w)
    announce(f"decode b={batch}: prefill {DECODE_PREFILL} + {DECODE_STEPS} steps")
    d = to_dev(inp)
    T0 = DECODE_PREFILL
    pre = {k: (v[:, :T0].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    _, state = ssd.ssd_chunk_scan(pre["x"], pre["dt"], pre["A"], pre["B"], pre["C"], pre["D"],
                                  chunk=w.chunk, dt_bias=pre["dt_bias"])
    ys = []
    for t in range(T0, T0 + DECODE_STEPS):
        ys.append(gpu_step(ssd, d, state, t))
    torch.cuda.synchronize()
    y_dec = torch.stack(ys, dim=1).cpu()                   # [b, 1024, H, P]
    y_full, f_full = ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                        chunk=w.chunk, dt_bias=d["dt_bias"])
    torch.cuda.synchronize()
    state = state.cpu()
    assert state_err(state, f_full.double().cpu()) <= TOL["bf16"]
    assert y_err(y_dec, y_full[:, T0:].double().cpu()) <= TOL["bf16"]
    worst_y = worst_s = 0.0
    for b in range(batch):
        row = {k: (v[b:b + 1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        y_ref, f_ref = oracle_scan(row, w)
        worst_s = max(worst_s, state_err(state[b:b + 1], f_ref))
        worst_y = max(worst_y, y_err(y_dec[b:b + 1], y_ref[:, T0:]))
    print(f"decode b={batch}: all {batch * w.nheads} sequences against the oracle: "
          f"y_t err {worst_y:.3e}  state err {worst_s:.3e}")
    assert worst_y <= TOL["bf16"] and worst_s <= TOL["bf16"]


def test_step_zero_batch_is_noop():
    need_gpu()
    import state_space_model_amd as ssd
    st = torch.zeros(0, 4, 16, 16, device="cuda")
    y = ssd.ssd_step(st, torch.zeros(0, 4, 16, device="cuda"), torch.zeros(0, 4, device="cuda"),
                     -torch.ones(4, device="cuda"), torch.zeros(0, 1, 16, device="cuda"),
                     torch.zeros(0, 1, 16, device="cuda"))
    assert y.shape == (0, 4, 16)
