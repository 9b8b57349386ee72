"""GPU parity of ssd_chunk_scan (the chunked prefill) against the CPU oracle.

Every case calls the HIP kernels through the C ABI (python binding) and
compares element by element with the fp64 token-by-token recurrence on the
same seeded inputs.  Error = max over (b, h) slices of
||gpu - oracle||_inf / ||oracle||_inf; bar: 1e-4 for float32 inputs, 2e-2 for
bfloat16 x/B/C (float32 decay, states and accumulation).

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching" (Background, Eq. 2-3; SSD properties: chunked recurrence; O(1)
cache: the prefill's final state seeds the decode cache).
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL, announce, need_gpu, oracle_scan, slice_bh, state_err, to_dev,
                      workload_inputs, y_err)
from oracle.metrics import token_rel_err
from ssd_inputs import WORKLOADS, make_inputs, make_tiny

pytestmark = pytest.mark.gpu


def run_gpu(inp, w, chunk=None, **kw):
    import state_space_model_amd as ssd
    d = to_dev(inp)
    y, fin = ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d.get("D"),
                                chunk=chunk or w.chunk, dt_bias=d.get("dt_bias"),
                                dt_limit=(w.dt_min, w.dt_max), initial_state=d.get("h0"), **kw)
    torch.cuda.synchronize()
    return y, fin


@pytest.mark.parametrize("name", ["tiny_f32", "m130_f32", "m2p7_bf16"])
def test_scan_workload_full(name):
    """Whole-problem parity on the tiny, 130M-shaped and 2.7B-shaped layers."""
    need_gpu()
    w = WORKLOADS[name]
    inp = workload_inputs(name)
    announce(f"scan {name} {w}")
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    ey, ef = y_err(y, y_ref), state_err(fin, f_ref)
    print(f"{name}: y err {ey:.3e}  final-state err {ef:.3e}")
    assert ey <= TOL[w.io_dtype] and ef <= TOL[w.io_dtype]


# The phased bf16 chunk states run several heads per workgroup (the count
# chosen from the number of chunks and heads); at 4097 tokens the last chunk
# holds one token and the heads of a group split into runs of 6 with a
# shorter last run, with one and with two groups (a run starting inside the
# second group's heads).
@pytest.mark.parametrize("G", [1, 2])
def test_scan_phased_head_runs(G):
    """2.7B-shaped bf16 prefill at 4097 tokens (phased: 80 chains), every
    (b, h) sequence against the oracle."""
    need_gpu()
    import state_space_model_amd as ssd
    w = make_tiny(1, 4097, 80, 64, 128, G, 256, "bf16", seed=5100 + G)
    inp = make_inputs(w)
    d = to_dev(inp)
    assert ssd.ssd_chunk_scan_schedule(d["x"], d["B"], 256) == ssd.SSD_SCHEDULE_PHASED
    announce(f"scan head runs 1x4097 H80 G{G} bf16")
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    ey, ef = y_err(y, y_ref), state_err(fin, f_ref)
    print(f"head runs G={G}: y err {ey:.3e}  final-state err {ef:.3e}")
    assert ey <= TOL["bf16"] and ef <= TOL["bf16"]


def test_scan_long_batched_full():
    """1.3B-shaped batched long prefill (8 x 16384, H=64, bf16) at chunk
    128, 256 and 512, each run whole on the GPU in the benchmark's launch
    configuration, and every one of the 512 (b, h) sequences compared with
    the oracle (one batch row at a time, to bound host memory; the oracle
    does not depend on the chunk, so each row's reference serves all three)."""
    need_gpu()
    import state_space_model_amd as ssd
    w = WORKLOADS["m1p3_long_bf16"]
    inp = workload_inputs("m1p3_long_bf16")
    d = to_dev(inp)
    outs = {}
    for chunk in (128, 256, 512):
        announce(f"scan m1p3_long_bf16 chunk={chunk} schedule "
                 f"{ssd.ssd_chunk_scan_schedule(d['x'], d['B'], chunk)}")
        outs[chunk] = ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                         chunk=chunk, dt_bias=d["dt_bias"],
                                         dt_limit=(w.dt_min, w.dt_max))
    torch.cuda.synchronize()
    del d
    worst = {L: [0.0, 0.0, 0.0] for L in outs}
    for b in range(w.batch):
        row = {k: (v[b:b + 1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        y_ref, f_ref = oracle_scan(row, w)
        for L, (y, fin) in outs.items():
            yb = y[b:b + 1].cpu()
            e = (y_err(yb, y_ref), state_err(fin[b:b + 1].cpu(), f_ref),
                 token_rel_err(yb, y_ref))
            worst[L] = [max(a_, b_) for a_, b_ in zip(worst[L], e)]
        print(f"row {b}: " + "  ".join(f"L{L} y {v[0]:.2e} fin {v[1]:.2e}"
                                       for L, v in worst.items()), flush=True)
    for L, (ey, ef, et) in worst.items():
        print(f"chunk {L}: y err {ey:.3e}  final-state err {ef:.3e}  "
              f"(per-token normalised {et:.3e}, information)")
        assert ey <= TOL["bf16"] and ef <= TOL["bf16"], (L, ey, ef)


def test_scan_chunk_size_invariance_on_gpu():
    """The same inputs at chunk 64/128/256 give the same result up to rounding
    (chunked recurrence: the chunk size trades work, not the answer)."""
    need_gpu()
    w = make_tiny(2, 1000, 8, 64, 128, 2, 64, "bf16", seed=31)
    inp = make_inputs(w)
    announce("scan chunk invariance 2x1000 H8 P64 N128 G2 bf16")
    outs = [run_gpu(inp, w, chunk=L) for L in (64, 128, 256)]
    y_ref, f_ref = oracle_scan(inp, w)
    for y, f in outs:
        assert y_err(y, y_ref) <= TOL["bf16"] and state_err(f, f_ref) <= TOL["bf16"]
    for y, f in outs[1:]:
        assert y_err(y, outs[0][0].double().cpu()) <= TOL["bf16"]


TINY = [
    # (Bt, T, H, P, N, G, L, dtype)
    (1, 96, 2, 16, 16, 1, 32, "f32"),        # three chunks
    (2, 200, 4, 32, 32, 2, 64, "f32"),       # ragged last chunk, groups
    (1, 77, 3, 16, 64, 1, 96, "f32"),        # one partial chunk, L not a power of two
    (1, 1, 2, 16, 16, 1, 64, "f32"),         # a single token
    (2, 333, 4, 64, 128, 1, 128, "f32"),     # ragged, 130M head shape
    (1, 300, 2, 128, 128, 1, 256, "f32"),    # P = 128
    (1, 512, 2, 64, 64, 2, 512, "f32"),      # L = 512
    (1, 100, 4, 16, 32, 4, 32, "bf16"),      # one group per head
    (2, 257, 4, 64, 128, 1, 256, "bf16"),    # 2.7B head shape, one token past a chunk
    (1, 700, 2, 32, 64, 1, 512, "bf16"),     # L = 512, ragged
    (1, 130, 2, 128, 32, 1, 64, "bf16"),     # P = 128
    (3, 64, 6, 16, 128, 3, 32, "bf16"),      # many chunks of 32
]


@pytest.mark.parametrize("case", TINY, ids=lambda c: "x".join(map(str, c)))
def test_scan_tiny_shapes(case):
    need_gpu()
    Bt, T, H, P, N, G, L, dt = case
    w = make_tiny(Bt, T, H, P, N, G, L, dt, seed=1000 + TINY.index(case))
    inp = make_inputs(w, with_initial_state=True)
    announce(f"scan tiny {case}")
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    assert y_err(y, y_ref) <= TOL[dt], y_err(y, y_ref)
    assert state_err(fin, f_ref) <= TOL[dt], state_err(fin, f_ref)


CHAIN = [
    # (Bt, T, H, P, N, G, L): batch x heads >= 256 with bf16 io selects the chain schedule
    (4, 700, 64, 64, 128, 1, 256),     # 2.7B head shape, ragged last chunk
    (2, 600, 128, 64, 64, 2, 128),     # N = 64, two groups
    (16, 333, 16, 32, 128, 4, 128),    # P = 32, four groups, ragged
    (8, 64, 32, 32, 64, 1, 64),        # a single full chunk
    (16, 1, 16, 64, 128, 1, 256),      # a single token
    (1, 1100, 256, 64, 128, 8, 256),   # one batch row, many heads
]


@pytest.mark.parametrize("case", CHAIN, ids=lambda c: "x".join(map(str, c)))
def test_scan_chain_schedule(case):
    """Shapes that run the chain schedule (one workgroup per (batch, head)
    walking the chunks with the state on chip) against the oracle."""
    need_gpu()
    import state_space_model_amd as ssd
    Bt, T, H, P, N, G, L = case
    w = make_tiny(Bt, T, H, P, N, G, L, "bf16", seed=2000 + CHAIN.index(case))
    inp = make_inputs(w, with_initial_state=True)
    announce(f"scan chain {case}")
    d = to_dev(inp)
    assert ssd.ssd_chunk_scan_schedule(d["x"], d["B"], L) == ssd.SSD_SCHEDULE_CHAIN
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    assert y_err(y, y_ref) <= TOL["bf16"], y_err(y, y_ref)
    assert state_err(fin, f_ref) <= TOL["bf16"], state_err(fin, f_ref)


def test_chain_and_phased_schedules_agree_bitwise():
    """A batch of 32 x 8 heads runs the chain schedule; each row alone (8
    heads) runs the phased one.  The two must agree bit for bit, so the
    batch-size invariance holds across the schedule switch."""
    need_gpu()
    import state_space_model_amd as ssd
    w = make_tiny(32, 600, 8, 64, 128, 1, 256, "bf16", seed=78)
    inp = make_inputs(w, with_initial_state=True)
    announce("scan chain vs phased bitwise 32x600 H8 P64 N128 L256")
    d = to_dev(inp)
    assert ssd.ssd_chunk_scan_schedule(d["x"], d["B"], 256) == ssd.SSD_SCHEDULE_CHAIN
    y1, f1 = run_gpu(inp, w)
    for b in (0, 13, 31):
        one = {k: (v[b:b + 1] if k in ("x", "dt", "B", "C", "h0") else v) for k, v in inp.items()}
        d1 = to_dev(one)
        assert ssd.ssd_chunk_scan_schedule(d1["x"], d1["B"], 256) == ssd.SSD_SCHEDULE_PHASED
        ya, fa = run_gpu(one, w.with_(batch=1))
        assert torch.equal(ya, y1[b:b + 1]) and torch.equal(fa, f1[b:b + 1]), b


@pytest.mark.parametrize("case", [
    # (Bt, T, H, G, io): groups of 8 heads sharing B/C, at layer scale
    (1, 4096, 64, 8, "f32"),
    (1, 4096, 64, 8, "bf16"),
    (4, 1024, 64, 8, "bf16"),     # batch x heads = 256: the chain schedule
], ids=lambda c: "_".join(map(str, c)))
def test_scan_groups_at_scale(case):
    """G > 1 at layer scale (8 B/C groups of 8 heads, P = 64, N = 128,
    L = 256) against the oracle in full."""
    need_gpu()
    Bt, T, H, G, io = case
    w = make_tiny(Bt, T, H, 64, 128, G, 256, io, seed=4100 + T + Bt)
    inp = make_inputs(w, with_initial_state=True)
    import state_space_model_amd as ssd
    sched = ssd.ssd_chunk_scan_schedule(inp["x"], inp["B"], 256)
    assert sched == (ssd.SSD_SCHEDULE_CHAIN if Bt * H >= 256 and io == "bf16"
                     else ssd.SSD_SCHEDULE_PHASED)
    announce(f"scan groups at scale {case} schedule {sched}")
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    ey, ef = y_err(y, y_ref), state_err(fin, f_ref)
    print(f"groups {case}: y err {ey:.3e}  final-state err {ef:.3e}")
    assert ey <= TOL[io] and ef <= TOL[io]


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_chunked_prefill_chain(io):
    """Chunked prefill ([SSD] O(1) cache: the prefill's final state seeds what
    follows): the 4096-token sequence run as pieces of 1000, 1, 1000, 2047 and
    48 tokens (chunk boundaries not aligned with the pieces), each seeded with
    the previous piece's final state, against the oracle over the whole
    sequence, and against the one-shot GPU scan."""
    need_gpu()
    import state_space_model_amd as ssd
    w = make_tiny(2, 4096, 24, 64, 128, 1, 256, io, seed=4200)
    inp = make_inputs(w, with_initial_state=True)
    d = to_dev(inp)
    announce(f"scan chunked prefill chain {io}")
    y_one, f_one = run_gpu(inp, w)
    state = d["h0"]
    ys = []
    lo = 0
    for n in (1000, 1, 1000, 2047, 48):
        sl = {k: (v[:, lo:lo + n].contiguous() if k in ("x", "dt", "B", "C") else v)
              for k, v in d.items()}
        y, state = ssd.ssd_chunk_scan(sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"],
                                      chunk=w.chunk, dt_bias=sl["dt_bias"], initial_state=state)
        ys.append(y)
        lo += n
    assert lo == 4096
    torch.cuda.synchronize()
    y_chain = torch.cat(ys, 1)
    y_ref, f_ref = oracle_scan(inp, w)
    ey, ef = y_err(y_chain, y_ref), state_err(state, f_ref)
    print(f"chain {io}: y err {ey:.3e}  final-state err {ef:.3e}")
    assert ey <= TOL[io] and ef <= TOL[io]
    assert y_err(y_chain, y_one.double().cpu().numpy()) <= TOL[io]
    assert state_err(state, f_one.double().cpu().numpy()) <= TOL[io]


# Delta at its clip limits ([SSD] Implementation: softplus then clip).  At
# dt_max with A = -16 every token decays by e^-8, so the decay across a chunk
# underflows float32 (the masked and factored exponentials must flush to 0,
# never overflow); at dt_min with A = -1 the memory is near-identity over
# 16384 tokens (large states, tiny per-token decay).
CLIP_CASES = [
    # (Bt, T, H, io, bound): bf16 with 256 chains runs the chain schedule
    (2, 4096, 8, "f32", "max"),
    (2, 4096, 8, "bf16", "max"),
    (4, 2048, 64, "bf16", "max"),
    (1, 16384, 8, "f32", "min"),
    (1, 16384, 8, "bf16", "min"),
    (4, 16384, 64, "bf16", "min"),
]


@pytest.mark.parametrize("case", CLIP_CASES, ids=lambda c: "_".join(map(str, c)))
def test_scan_delta_at_clip_bounds(case):
    need_gpu()
    import state_space_model_amd as ssd
    Bt, T, H, io, bound = case
    w = make_tiny(Bt, T, H, 64, 128, 1, 256, io, seed=4300 + CLIP_CASES.index(case))
    inp = make_inputs(w, with_initial_state=(bound == "max"))
    if bound == "max":
        inp["dt_bias"] = torch.full((H,), 5.0)    # softplus ~ 5 -> clipped to 0.5
        inp["A"] = torch.full((H,), -16.0)
    else:
        inp["dt_bias"] = torch.full((H,), -20.0)  # softplus ~ 2e-9 -> clipped to 1e-4
        inp["A"] = torch.full((H,), -1.0)
    d = to_dev(inp)
    announce(f"scan delta at dt_{bound} {case} schedule "
             f"{ssd.ssd_chunk_scan_schedule(d['x'], d['B'], 256)}")
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    ey, ef = y_err(y, y_ref), state_err(fin, f_ref)
    print(f"dt_{bound} {case}: y err {ey:.3e}  final-state err {ef:.3e}  "
          f"per-token {token_rel_err(y, y_ref):.3e}")
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    assert ey <= TOL[io] and ef <= TOL[io]


# Chunk sizes that are multiples of 32 but not of 64 (the kernels work in
# 64-token key blocks, so the last block of each chunk is partial), on both
# bf16 schedules and in float32, with several full chunks and a ragged one.
ODD_CHUNK = [
    # (Bt, T, H, P, N, G, L, io)
    (1, 500, 4, 64, 128, 1, 96, "bf16"),
    (2, 700, 4, 32, 64, 2, 160, "bf16"),
    (1, 1500, 2, 64, 128, 1, 480, "bf16"),
    (1, 333, 4, 128, 32, 1, 224, "bf16"),
    (4, 700, 64, 64, 128, 1, 96, "bf16"),     # chain
    (2, 1000, 128, 32, 64, 2, 160, "bf16"),   # chain
    (1, 900, 256, 64, 128, 4, 224, "bf16"),   # chain
    (2, 500, 4, 64, 128, 1, 96, "f32"),
    (1, 700, 4, 64, 128, 2, 160, "f32"),
    (1, 1500, 2, 64, 64, 1, 480, "f32"),
]


@pytest.mark.parametrize("case", ODD_CHUNK, ids=lambda c: "x".join(map(str, c)))
def test_scan_chunk_not_multiple_of_64(case):
    need_gpu()
    import state_space_model_amd as ssd
    Bt, T, H, P, N, G, L, io = case
    w = make_tiny(Bt, T, H, P, N, G, L, io, seed=4400 + ODD_CHUNK.index(case))
    inp = make_inputs(w, with_initial_state=True)
    d = to_dev(inp)
    sched = ssd.ssd_chunk_scan_schedule(d["x"], d["B"], L)
    assert sched == (ssd.SSD_SCHEDULE_CHAIN if io == "bf16" and Bt * H >= 256 and L <= 256
                     else ssd.SSD_SCHEDULE_PHASED)
    announce(f"scan chunk {L} {case} schedule {sched}")
    y, fin = run_gpu(inp, w)
    y_ref, f_ref = oracle_scan(inp, w)
    ey, ef = y_err(y, y_ref), state_err(fin, f_ref)
    print(f"{case}: y err {ey:.3e}  final-state err {ef:.3e}")
    assert ey <= TOL[io] and ef <= TOL[io]


def test_scan_options_off():
    """No D, no dt_bias, softplus off, no initial state, no final state requested."""
    need_gpu()
    import state_space_model_amd as ssd
    w = make_tiny(2, 150, 4, 32, 64, 2, 64, "f32", seed=5)
    inp = make_inputs(w)
    inp["dt"] = inp["dt"].abs() * 0.2 + 0.01  # already a step size
    announce("scan options off")
    d = to_dev(inp)
    y, fin = ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], None, chunk=64,
                                dt_softplus=False, return_final_state=False)
    torch.cuda.synchronize()
    assert fin is None
    y_ref, _ = oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], None, None, None,
                           dt_softplus=False)
    assert y_err(y, y_ref) <= TOL["f32"]


def test_scan_is_deterministic_and_batch_invariant():
    """Bitwise repeatable, and a batch row computed inside a batch of 8 equals
    the same row computed alone (the pages' batch-size invariance)."""
    need_gpu()
    w = make_tiny(8, 600, 8, 64, 128, 1, 256, "bf16", seed=77)
    inp = make_inputs(w, with_initial_state=True)
    announce("scan determinism / batch invariance")
    y1, f1 = run_gpu(inp, w)
    y2, f2 = run_gpu(inp, w)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)
    b = 5
    one = {k: (v[b:b + 1] if k in ("x", "dt", "B", "C", "h0") else v) for k, v in inp.items()}
    ya, fa = run_gpu(one, w.with_(batch=1))
    assert torch.equal(ya, y1[b:b + 1]) and torch.equal(fa, f1[b:b + 1])


def test_scan_empty_inputs():
    need_gpu()
    import state_space_model_amd as ssd
    announce("scan empty inputs")
    dev = "cuda"
    H, P, N = 4, 16, 16
    A = -torch.ones(H, device=dev)
    # batch 0
    y, fin = ssd.ssd_chunk_scan(torch.zeros(0, 10, H, P, device=dev), torch.zeros(0, 10, H, device=dev),
                                A, torch.zeros(0, 10, 1, N, device=dev),
                                torch.zeros(0, 10, 1, N, device=dev), chunk=64)
    assert y.shape == (0, 10, H, P) and fin.shape == (0, H, P, N)
    # seqlen 0: the final state is the initial state, or zeros
    h0 = torch.randn(2, H, P, N, device=dev)
    e = dict(x=torch.zeros(2, 0, H, P, device=dev), dt=torch.zeros(2, 0, H, device=dev),
             B=torch.zeros(2, 0, 1, N, device=dev))
    y, fin = ssd.ssd_chunk_scan(e["x"], e["dt"], A, e["B"], e["B"].clone(), chunk=64,
                                initial_state=h0)
    torch.cuda.synchronize()
    assert y.shape == (2, 0, H, P) and torch.equal(fin, h0)
    y, fin = ssd.ssd_chunk_scan(e["x"], e["dt"], A, e["B"], e["B"].clone(), chunk=64)
    torch.cuda.synchronize()
    assert torch.count_nonzero(fin) == 0


def test_scan_rejects_unsupported_shapes_before_launch():
    need_gpu()
    import state_space_model_amd as ssd
    dev = "cuda"
    x = torch.zeros(1, 64, 2, 24, device=dev)
    B = torch.zeros(1, 64, 1, 16, device=dev)
    with pytest.raises(ssd.SSDError, match="UNSUPPORTED"):
        ssd.ssd_chunk_scan(x, torch.zeros(1, 64, 2, device=dev), -torch.ones(2, device=dev), B, B,
                           chunk=64)
    x = torch.zeros(1, 64, 2, 16, device=dev, dtype=torch.bfloat16)
    B = torch.zeros(1, 64, 1, 16, device=dev, dtype=torch.bfloat16)
    with pytest.raises(ssd.SSDError, match="UNSUPPORTED"):
        ssd.ssd_chunk_scan(x, torch.zeros(1, 64, 2, device=dev), -torch.ones(2, device=dev), B, B,
                           chunk=64)
