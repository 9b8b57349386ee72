"""Kernel analogues of the two ablations of "Compiler-First State Space
Duality and Portable O(1) Autoregressive Caching", Implementation choices,
run through ssd_chunk_scan_ablation:

 * static masking: where the causal mask lives changes speed, not bits.  The
   variant that reads the mask of the diagonal tiles from a stored
   lower-triangular table must give bitwise the output of the in-register
   index comparison, on both bfloat16 schedules.
 * precision management: the decay held in bfloat16 instead of float32 costs
   accuracy.  The variant that rounds every decay factor of the output path
   to bfloat16 is compared with the oracle next to the float32 path; the
   chunk states, which the variant does not touch, stay bitwise equal.
"""
import pytest
import torch

from gpu_util import TOL, announce, need_gpu, oracle_scan, state_err, to_dev, workload_inputs, y_err
from oracle.metrics import token_rel_err
from ssd_inputs import WORKLOADS, make_inputs, make_tiny

pytestmark = pytest.mark.gpu


def run(ssd, d, w, variant):
    return ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=w.chunk,
                              dt_bias=d["dt_bias"], dt_limit=(w.dt_min, w.dt_max),
                              initial_state=d.get("h0"), variant=variant)


def timed(ssd, d, w, variant, reps=10):
    run(ssd, d, w, variant)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        run(ssd, d, w, variant)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


@pytest.mark.parametrize("name,bt,T,H", [
    ("phased", 1, 4096, 80),    # the 2.7B-shaped layer: phased schedule
    ("chain", 4, 2048, 64),     # 256 (batch, head) chains: chain schedule
])
def test_loaded_mask_is_bitwise_the_in_register_mask(name, bt, T, H):
    need_gpu()
    import state_space_model_amd as ssd
    w = make_tiny(bt, T, H, 64, 128, 1, 256, "bf16", seed=4500 + bt)
    inp = make_inputs(w, with_initial_state=True)
    d = to_dev(inp)
    sched = ssd.ssd_chunk_scan_schedule(d["x"], d["B"], 256)
    assert sched == (ssd.SSD_SCHEDULE_CHAIN if name == "chain" else ssd.SSD_SCHEDULE_PHASED)
    announce(f"ablation loaded mask {name} {bt}x{T} H{H}")
    y0, f0 = run(ssd, d, w, ssd.SSD_VARIANT_DEFAULT)
    y1, f1 = run(ssd, d, w, ssd.SSD_VARIANT_LOADED_MASK)
    torch.cuda.synchronize()
    assert torch.equal(y0, y1) and torch.equal(f0, f1)
    t0 = timed(ssd, d, w, ssd.SSD_VARIANT_DEFAULT)
    t1 = timed(ssd, d, w, ssd.SSD_VARIANT_LOADED_MASK)
    print(f"loaded mask {name}: bitwise equal; {t0 * 1e3:.1f} us in-register, "
          f"{t1 * 1e3:.1f} us loaded")


@pytest.mark.parametrize("name", ["m130_f32", "m2p7_bf16"])
def test_bf16_decay_costs_accuracy(name):
    """Both layer shapes in full against the oracle, float32 decay and
    bfloat16 decay side by side.  The bars of the float32 path still apply to
    it; the bfloat16-decay variant must be finite and change y (its error is
    the ablation's measurement), and with float32 io, where nothing else is
    rounded, its error must stand far above the float32 path's."""
    need_gpu()
    import state_space_model_amd as ssd
    w = WORKLOADS[name]
    inp = workload_inputs(name)
    d = to_dev(inp)
    announce(f"ablation bf16 decay {name}")
    y0, f0 = run(ssd, d, w, ssd.SSD_VARIANT_DEFAULT)
    y1, f1 = run(ssd, d, w, ssd.SSD_VARIANT_BF16_DECAY)
    torch.cuda.synchronize()
    y_ref, f_ref = oracle_scan(inp, w)
    e0, e1 = y_err(y0, y_ref), y_err(y1, y_ref)
    t0, t1 = token_rel_err(y0, y_ref), token_rel_err(y1, y_ref)
    print(f"{name}: y err float32 decay {e0:.3e} (per-token {t0:.3e}), "
          f"bf16 decay {e1:.3e} (per-token {t1:.3e}); final state err {state_err(f0, f_ref):.3e}")
    assert e0 <= TOL[w.io_dtype]
    assert torch.isfinite(y1.float()).all()
    assert not torch.equal(y0, y1)
    assert torch.equal(f0, f1)      # chunk states and recurrence are not part of the variant
    if w.io_dtype == "f32":
        assert e1 > 10 * e0
