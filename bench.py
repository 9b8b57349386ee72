"""Benchmark of the MI355X SSD library: chunked-scan prefill and cached decode.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                [--decode-batch B] [--no-cpu-baseline]

One step is one ssd_chunk_scan over the workload's whole batch (the prefill
path: Delta preparation, per-chunk prefix sum, decay matrix, C B^T, the
intra-chunk product, chunk states, the inter-chunk recurrence and the
state-to-output term).  The headline workload is the largest one-GPU prefill,
the 1.3B-shaped batched long prefill (8 x 16384 tokens, 64 heads, bf16 x/B/C,
chunk 256).  The 130M- and 2.7B-shaped layer prefills are timed in the same
run ("prefill_configs"), and so is the cached-decode path (ssd_step) at
batch 1, 16 and 64 ("decode").  Inputs are seeded synthetic
activations resident in device memory before timing starts; K steps are
timed between two device synchronisations.  Input/output sets are rotated so
that their total exceeds the 256 MB Infinity Cache.

Prints ONE JSON line.  Algorithmic work counts (what the method must do: the
causal half of each L x L block, C B^T once per group):
  FLOP/token = H[(L+1)P + 4NP + 2PN/L] + G(L+1)N
  decode bytes/token = 8HPN (state read + write) + HP(s_x + s_y) + 4H + 2GN s_BC
Peaks are MI355X's published dense figures (fp32 MFMA 157.3 TFLOP/s, bf16
2.5 PFLOP/s, HBM3E 8 TB/s).

roofline.traffic is the HBM bytes one launch of the reported kernel moved,
from rocprofv3 FETCH_SIZE and WRITE_SIZE counter runs (one counter per run)
scaled by what the same counters read for a plain copy of known size
(python bench.py --copy-calibration: the library's own float4 copy kernel on
a 1 GiB state).  The values are kept in TRAFFIC below with a digest of the
kernel's sources; once a source changes the digest no longer matches and
traffic is reported as null until the counters are taken again.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import platform
import sys
import statistics
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("SSD prefill tokens/s (% MFMA peak); cached decode tokens/s (% HBM GB/s peak)")
PEAK_TFLOPS = {"f32": 157.3, "bf16": 2500.0}
PEAK_HBM_GBS = 8000.0
MALL_BYTES = 256 << 20
DEFAULT_WORKLOAD = "m1p3_long_bf16"
SUB_WORKLOADS = ("m130_f32", "m2p7_bf16")
DECODE_BATCHES = (1, 16, 64)
CSRC = os.path.join(ROOT, "state_space_model_amd", "csrc")
# sources a kernel's code comes from (the digest that keys TRAFFIC)
KERNEL_SOURCES = {
    "chunk_out/f32": ["ssd_prefill_f32.hip", "ssd_prefill_common.h", "ssd_device.h"],
    "chunk_out/bf16": ["ssd_prefill_bf16.hip", "ssd_prefill_common.h", "ssd_device.h"],
    "chain/bf16": ["ssd_prefill_bf16.hip", "ssd_prefill_common.h", "ssd_device.h"],
    "decode": ["ssd_step.hip", "ssd_device.h"],
    "conv1d": ["ssd_conv.hip", "ssd_device.h"],
}
# HBM bytes per launch from the counter runs: (kernel key, workload) -> (bytes, digest)
TRAFFIC = {
    # counter runs and calibration: profiles/hbm_bytes_prefill_decode_kernels.txt
    ("chain/bf16", "m1p3_long_bf16"): (1566.49e6 + 1096.93e6, "a4525c742d855750"),
    ("chunk_out/bf16", "m2p7_bf16"): (67.05e6 + 41.94e6, "a4525c742d855750"),
    ("chunk_out/f32", "m130_f32"): (43.13e6 + 30.60e6, "a69d264b603eff81"),
    ("decode", "m2p7_decode_b1"): (2.76e6 + 2.63e6, "f187b92f35e363d9"),
    ("decode", "m2p7_decode_b16"): (42.37e6 + 42.11e6, "f187b92f35e363d9"),
    ("decode", "m2p7_decode_b64"): (171.07e6 + 168.43e6, "f187b92f35e363d9"),
    ("conv1d", "conv_m2p7_bf16"): (49.20e6 + 44.07e6, "8b295ccdaccd2f32"),
    ("conv1d", "conv_m2p7_decode_b64"): (3.64e6 + 2.75e6, "8b295ccdaccd2f32"),
}
COPY_CALIBRATION_BYTES = 1 << 30


def prefill_flops_per_token(w):
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    return H * ((L + 1) * P + 4 * N * P + 2 * P * N / L) + G * (L + 1) * N


def uses_prepass(w, chain):
    """The bfloat16 scan at the chain kernel's head shapes (P in {32, 64}, N in
    {64, 128}, L <= 256) starts with the C B^T / B^T pre-pass on both schedules."""
    return chain or (w.io_dtype == "bf16" and w.headdim in (32, 64) and w.dstate in (64, 128)
                     and w.chunk <= 256)


def phase_flops_per_token(w, chain):
    """Algorithmic FLOP/token of each kernel of the scan, by schedule.
    chain: a C B^T / B^T pre-pass, then one kernel doing the chunk states,
    the inter-chunk recurrence and the outputs (a5-a8).  phased: chunk
    states (with C B^T in the same launch, or after the pre-pass), the state
    pass, the outputs."""
    H, P, N, G, L = w.nheads, w.headdim, w.dstate, w.ngroups, w.chunk
    cb = G * (L + 1) * N
    if chain:
        return {"cb_bt_prepass": cb, "chain": H * ((L + 1) * P + 4 * N * P + 2 * P * N / L)}
    per = {"chunk_state": H * 2 * N * P,
           "state_pass": H * 2 * P * N / L,                                # inter-chunk recurrence
           "chunk_out": H * ((L + 1) * P + 2 * N * P)}                     # decay, products
    if uses_prepass(w, chain):
        per["cb_bt_prepass"] = cb
    else:
        per["chunk_state"] += cb
    return per


# kernel (phase) names of each schedule, and the event interval that times
# each: the timed call records an event before each of its 4 phases and one
# after the last; an empty phase's two events add only event overhead, so
# empty phases are not reported.
def phase_plan(w, chain):
    if chain:
        return {"cb_bt_prepass": (0, 1), "chain": (3, 4)}
    plan = {"chunk_state": (1, 2), "state_pass": (2, 3), "chunk_out": (3, 4)}
    if uses_prepass(w, chain):
        plan = {"cb_bt_prepass": (0, 1), **plan}
    return plan


def kernel_names(w, chain):
    return {"chunk_state": "k_chunk_state_bf16" if uses_prepass(w, chain) else "k_cb_and_chunk_state",
            "state_pass": "k_state_pass", "chunk_out": "k_chunk_out",
            "cb_bt_prepass": "k_cb_and_bt_bf16", "chain": "k_chain_bf16"}


def prefill_bytes_per_token(w, T):
    s = 2 if w.io_dtype == "bf16" else 4
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    return H * P * (s + s) + 4 * H + 2 * G * N * s + 4 * H * P * N / T


def decode_bytes_per_token(H, P, N, G, s):
    return 8 * H * P * N + H * P * 2 * s + 4 * H + 2 * G * N * s


def source_digest(key):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[key]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def traffic_for(key, workload):
    """Counter-derived HBM bytes per launch, or None if not measured for the current sources."""
    entry = TRAFFIC.get((key, workload))
    if entry is None or entry[1] != source_digest(key):
        return None
    return entry[0]


def copy_calibration(ssd, torch, reps=5):
    """A plain copy of known size for the counter calibration: an empty-sequence
    scan copies the initial state (1 GiB) to the final state with the library's
    float4 copy kernel (k_copy_or_zero)."""
    Bt, H, P, N = 512, 64, 64, 128          # 2^28 float32 = 1 GiB
    h0 = torch.randn(Bt, H, P, N, device="cuda")
    fin = torch.empty_like(h0)
    x = torch.empty(Bt, 0, H, P, device="cuda")
    dt = torch.empty(Bt, 0, H, device="cuda")
    B = torch.empty(Bt, 0, 1, N, device="cuda")
    A = -torch.ones(H, device="cuda")
    for _ in range(reps):
        ssd.ssd_chunk_scan(x, dt, A, B, B, None, chunk=64, initial_state=h0, final_state=fin)
    torch.cuda.synchronize()
    assert torch.equal(fin, h0)
    return {"copy_bytes_read": h0.numel() * 4, "copy_bytes_written": fin.numel() * 4,
            "dispatches": reps, "kernel": "k_copy_or_zero"}


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def bench_prefill(ssd, torch, w, steps, warmup):
    from ssd_inputs import make_inputs
    inp = make_inputs(w)
    dev = torch.device("cuda")
    shared = {k: inp[k].to(dev) for k in ("A", "D", "dt_bias")}
    Bt, T, H, P = inp["x"].shape
    N = inp["B"].shape[3]
    x0 = inp["x"].to(dev)
    B0 = inp["B"].to(dev)
    ws_bytes = ssd.ssd_chunk_scan_workspace_bytes(x0, B0, w.chunk)
    es = x0.element_size()
    set_bytes = (2 * x0.numel() * es + inp["dt"].numel() * 4 + 2 * B0.numel() * es
                 + Bt * H * P * N * 4 + ws_bytes)
    nsets = max(1, min(16, math.ceil(2 * MALL_BYTES / set_bytes)))
    sets = []
    for _ in range(nsets):
        s = {"x": x0.clone(), "dt": inp["dt"].to(dev), "B": B0.clone(), "C": inp["C"].to(dev),
             "y": torch.empty_like(x0),
             "fin": torch.empty(Bt, H, P, N, device=dev, dtype=torch.float32),
             "ws": torch.empty(ws_bytes, device=dev, dtype=torch.uint8)}
        sets.append(s)

    def run(i, events=None):
        s = sets[i % nsets]
        ssd.ssd_chunk_scan(s["x"], s["dt"], shared["A"], s["B"], s["C"], shared["D"],
                           chunk=w.chunk, dt_bias=shared["dt_bias"], dt_limit=(w.dt_min, w.dt_max),
                           y=s["y"], final_state=s["fin"], workspace=s["ws"], phase_events=events)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        run(i)
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # five more timed runs of the same K steps: spread of the step time
    rep_ms = []
    for _ in range(5):
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        r0.record()
        for i in range(steps):
            run(i)
        r1.record()
        torch.cuda.synchronize()
        rep_ms.append(r0.elapsed_time(r1) / steps)
    # per-kernel durations, HIP events on the stream the kernels run on
    nph = ssd.SSD_SCAN_PHASES
    chain = ssd.ssd_chunk_scan_schedule(x0, B0, w.chunk) == ssd.SSD_SCHEDULE_CHAIN
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nph + 1)] for _ in range(steps)]
    for i in range(steps):
        run(i, evs[i])
    torch.cuda.synchronize()
    phase_ms = {n: sum(evs[i][a].elapsed_time(evs[i][b]) for i in range(steps)) / steps
                for n, (a, b) in phase_plan(w, chain).items()}
    return {"ms": ms, "wall_ms": wall * 1e3 / steps, "phase_ms": phase_ms, "nsets": nsets,
            "set_bytes": set_bytes, "tokens": Bt * T, "rep_ms": rep_ms, "chain": chain}


def prefill_report(w, pf, headline=False):
    """The prefill numbers of one workload: whole call against the MFMA peak
    of its dtype, and the dominant kernel's roofline (its own algorithmic
    FLOPs over its event-timed launch duration)."""
    tokens_s = pf["tokens"] / (pf["ms"] * 1e-3)
    fpt = prefill_flops_per_token(w)
    per = phase_flops_per_token(w, pf["chain"])
    peak = PEAK_TFLOPS[w.io_dtype]
    dom = max(pf["phase_ms"], key=pf["phase_ms"].get)
    dom_flops = per[dom] * pf["tokens"]
    dom_ms = pf["phase_ms"][dom]
    achieved = dom_flops / (dom_ms * 1e-3) / 1e12
    key = f"{dom}/{w.io_dtype}"
    whole_tflops = fpt * pf["tokens"] / (pf["ms"] * 1e-3) / 1e12
    bpt = prefill_bytes_per_token(w, w.seqlen)
    roof = {"bound": "mfma", "kernel": kernel_names(w, pf["chain"])[dom], "achieved": achieved, "peak": peak,
            "unit": "TFLOP/s", "frac": achieved / peak,
            "traffic": traffic_for(key, w.name) if key in KERNEL_SOURCES else None,
            "flops_per_launch": dom_flops, "avg_launch_ms": dom_ms}
    rep = {"workload": w.name, "schedule": "chain" if pf["chain"] else "phased",
           "ms_per_step": pf["ms"], "tokens_per_s": tokens_s,
           "algorithmic_tflops": whole_tflops, "mfma_peak_frac": whole_tflops / peak,
           "flops_per_token": fpt, "bytes_per_token": bpt,
           "hbm_gbs_algorithmic": bpt * tokens_s / 1e9,
           "hbm_peak_frac_algorithmic": bpt * tokens_s / 1e9 / PEAK_HBM_GBS,
           "phase_ms": pf["phase_ms"],
           "phase_tflops": {n: per[n] * pf["tokens"] / (ms * 1e-3) / 1e12
                            for n, ms in pf["phase_ms"].items()},
           "wall_ms_per_step": pf["wall_ms"],
           "repeat_ms_per_step": {"runs": 5, "mean": statistics.mean(pf["rep_ms"]),
                                  "std": statistics.stdev(pf["rep_ms"]),
                                  "min": min(pf["rep_ms"]), "max": max(pf["rep_ms"])},
           "rotated_sets": pf["nsets"]}
    if not headline:
        rep["roofline"] = roof
    return rep, roof


def bench_decode(ssd, torch, batch, steps_n, warmup):
    """2.7B-shaped decode (H=80, P=64, N=128, bf16 x/B/C, fp32 state): steps
    captured in one HIP graph; states rotated over >= 512 MB (one state per
    layer-like buffer) so that the state streams from HBM, not the cache."""
    from ssd_inputs import WORKLOADS, make_inputs
    w = WORKLOADS["m2p7_decode"].with_(batch=batch, seqlen=steps_n)
    inp = make_inputs(w)
    dev = torch.device("cuda")
    H, P, N, G = w.nheads, w.headdim, w.dstate, w.ngroups
    xs = inp["x"].transpose(0, 1).contiguous().to(dev)     # [steps, b, H, P]
    dts = inp["dt"].transpose(0, 1).contiguous().to(dev)   # [steps, b, H]
    Bs = inp["B"].transpose(0, 1).contiguous().to(dev)     # [steps, b, G, N]
    Cs = inp["C"].transpose(0, 1).contiguous().to(dev)
    A, D, bias = inp["A"].to(dev), inp["D"].to(dev), inp["dt_bias"].to(dev)
    state_bytes = batch * H * P * N * 4
    nstates = max(1, math.ceil(2 * MALL_BYTES / state_bytes))
    states = [torch.randn(batch, H, P, N, device=dev) * 0.1 for _ in range(nstates)]
    ys = torch.empty(steps_n, batch, H, P, device=dev, dtype=xs.dtype)

    def body():
        for t in range(steps_n):
            ssd.ssd_step(states[t % nstates], xs[t], dts[t], A, Bs[t], Cs[t], D, dt_bias=bias,
                         y_t=ys[t])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(max(1, min(warmup, 3))):   # eager passes before the capture
            body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    reps = 3
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (reps * steps_n)
    s_io = xs.element_size()
    bpt = decode_bytes_per_token(H, P, N, G, s_io)
    achieved = bpt * batch / (ms_step * 1e-3) / 1e9
    copy_us = device_copy_us(torch, states, steps_n)
    return {"batch": batch, "steps": steps_n, "graph_replays": reps, "ms_per_step": ms_step,
            "device_copy_us": copy_us,
            "tokens_per_s": batch / (ms_step * 1e-3), "state_buffers": nstates,
            "state_bytes_each": state_bytes,
            "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS,
                         "traffic": traffic_for("decode", f"m2p7_decode_b{batch}")},
            "bytes_per_token": bpt}


def device_copy_us(torch, states, steps_n, reps=3):
    """Time per step of torch's device copy of one state into another buffer
    (the decode step's state bytes, read once and written once), replayed
    from a HIP graph over the same rotation of buffers: a plain copy of the
    step's bytes, for scale beside the step's own time."""
    dst = [torch.empty_like(t) for t in states]
    n = len(states)

    def body():
        for t in range(steps_n):
            dst[t % n].copy_(states[t % n])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * steps_n)
    del g, dst
    return us


def launch_floor_us(ssd, torch, n=1024):
    """Time per node of a HIP graph of n launches of the library's smallest
    kernel (the float4 copy an empty-sequence scan makes of a 1 KiB state):
    the launch/latency floor a one-row decode step sits on."""
    H, P, N = 1, 16, 16
    h0 = torch.randn(1, H, P, N, device="cuda")
    fin = torch.empty_like(h0)
    x = torch.empty(1, 0, H, P, device="cuda")
    dt = torch.empty(1, 0, H, device="cuda")
    B = torch.empty(1, 0, 1, N, device="cuda")
    A = -torch.ones(H, device="cuda")

    def body():
        for _ in range(n):
            ssd.ssd_chunk_scan(x, dt, A, B, B, None, chunk=64, initial_state=h0, final_state=fin)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (3 * n)


def bench_cached_vs_recompute(ssd, torch, context=4096, reps=20):
    """Cached decode against recomputing the prefix: the time to produce the
    output of token `context` from the cached state with one ssd_step, and by
    re-running ssd_chunk_scan over all context+1 tokens (2.7B shape, batch 1,
    bf16 x/B/C).  The layer-level analogue of the pages' cached-versus-
    recompute comparison at a 4096-token context."""
    from ssd_inputs import WORKLOADS, make_inputs
    w = WORKLOADS["m2p7_decode"].with_(batch=1, seqlen=context + 1)
    inp = make_inputs(w)
    d = {k: v.cuda() for k, v in inp.items()}
    Bt, T, H, P = d["x"].shape
    N = d["B"].shape[3]
    y = torch.empty_like(d["x"])
    fin = torch.empty(Bt, H, P, N, device="cuda")
    ws = torch.empty(ssd.ssd_chunk_scan_workspace_bytes(d["x"], d["B"], w.chunk),
                     dtype=torch.uint8, device="cuda")
    state = torch.empty(Bt, H, P, N, device="cuda")
    x_t, dt_t = d["x"][:, T - 1].contiguous(), d["dt"][:, T - 1].contiguous()
    B_t, C_t = d["B"][:, T - 1].contiguous(), d["C"][:, T - 1].contiguous()
    y_t = torch.empty_like(x_t)

    def recompute():
        ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=w.chunk,
                           dt_bias=d["dt_bias"], y=y, final_state=fin, workspace=ws)

    def step():
        ssd.ssd_step(state, x_t, dt_t, d["A"], B_t, C_t, d["D"], dt_bias=d["dt_bias"], y_t=y_t)

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3

    def graphed(fn):
        """The same calls captured in one HIP graph (no host launch cost):
        `reps` calls per replay, three replays timed."""
        fn()
        torch.cuda.synchronize()
        s_ = torch.cuda.Stream()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s_):
            with torch.cuda.graph(g, stream=s_):
                for _ in range(reps):
                    fn()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (3 * reps) * 1e3

    t_re = timed(recompute)
    state.copy_(fin)
    t_st = timed(step)
    g_re = graphed(recompute)
    state.copy_(fin)
    g_st = graphed(step)
    return {"context": context, "shape": "H=80 P=64 N=128 bf16 x/B/C, batch 1",
            "recompute_us": t_re, "cached_step_us": t_st, "speedup": t_re / t_st,
            "graph": {"recompute_us": g_re, "cached_step_us": g_st, "speedup": g_re / g_st},
            "note": "eager: one host launch per call (the step is host-bound); graph: the "
                    "calls replayed from one HIP graph"}


def backward_flops(w):
    """Algorithmic FLOP of one ssd_chunk_scan_backward call: the products a
    chunked backward of the scan must form, causal halves of each L x L block
    counted as L(L+1)/2, C B^T once per (chunk, group):
      per (chunk, head): 2LPN each for the recomputed chunk state, the adjoint
        chunk state, and the state terms of dx, dC and dB (5 x 2LPN); L(L+1)/2 * 2P
        each for dy x^T and the intra-chunk term of dx;
      per (chunk, group): L(L+1)/2 * 2N each for C B^T and the intra-chunk
        terms of dC (M B) and dB (M^T C)."""
    L, P, N = w.chunk, w.headdim, w.dstate
    Nc = -(-w.seqlen // L)
    tri = L * (L + 1) // 2
    per_head = 5 * 2 * L * P * N + 2 * tri * 2 * P
    per_group = 3 * tri * 2 * N
    return w.batch * Nc * (w.nheads * per_head + w.ngroups * per_group)


def bench_backward(ssd, torch, w, reps=10):
    """The scan's gradients (ssd_chunk_scan_backward) on the headline layer:
    time per call and per token, against the forward scan of the same
    inputs timed the same way (eager launches, inputs resident)."""
    from ssd_inputs import make_inputs
    inp = make_inputs(w, with_initial_state=True)
    d = {k: v.cuda() for k, v in inp.items()}
    g = torch.Generator(device="cpu").manual_seed(6500)
    dy = torch.randn(d["x"].shape, generator=g).to(d["x"].dtype).cuda()
    dfinal = torch.randn(d["h0"].shape, generator=g).cuda()
    ws = torch.empty(ssd.ssd_chunk_scan_backward_workspace_bytes(d["x"], d["B"], w.chunk),
                     dtype=torch.uint8, device="cuda")
    fws = torch.empty(ssd.ssd_chunk_scan_workspace_bytes(d["x"], d["B"], w.chunk),
                      dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    fin = torch.empty_like(d["h0"])
    grads = ssd.ssd_chunk_scan_backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], dy=dy,
                                        dfinal_state=dfinal, chunk=w.chunk, dt_bias=d["dt_bias"],
                                        initial_state=d["h0"], workspace=ws)

    def bwd():
        ssd.ssd_chunk_scan_backward(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], dy=dy,
                                    dfinal_state=dfinal, chunk=w.chunk, dt_bias=d["dt_bias"],
                                    initial_state=d["h0"], workspace=ws, grads=grads)

    def fwd():
        ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], chunk=w.chunk,
                           dt_bias=d["dt_bias"], initial_state=d["h0"], y=y, final_state=fin,
                           workspace=fws)

    def timed(fn):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_b = timed(bwd)
    ms_f = timed(fwd)
    tokens = w.batch * w.seqlen
    flops = backward_flops(w)
    tflops = flops / (ms_b * 1e-3) / 1e12
    return {"workload": w.name, "ms": ms_b, "tokens_per_s": tokens / (ms_b * 1e-3),
            "forward_ms_same_inputs": ms_f, "backward_over_forward": ms_b / ms_f,
            "flops_per_call": flops, "algorithmic_tflops": tflops,
            "mfma_fp32_frac": tflops / PEAK_TFLOPS["f32"],
            "workspace_bytes": ws.numel(),
            "note": "gradients of every input; recomputes the forward chunk states; the "
                    "two scans run the io type's kernels, the gradient kernels float32 "
                    "matrix-core products (mfma_fp32_frac prices all of it at the fp32 peak)"}


def conv_bytes(Bt, T, D, K, es):
    """Algorithmic bytes of one conv1d call: x read and y written once, the
    window read and written once, weights and bias read once."""
    return 2 * Bt * T * D * es + 2 * Bt * D * (K - 1) * es + D * (K + 1) * 4


def bench_conv(ssd, torch, warmup, reps=20, steps_n=256):
    """The depthwise causal conv1d before the scan: a 4096-token prefill of
    the 2.7B shape (D_conv 5376, bf16) and the one-token step at batch 64,
    the latter captured in a HIP graph.  Inputs rotate over enough buffers
    to exceed twice the 256 MB last-level cache."""
    from ssd_inputs import CONV_WORKLOADS, make_conv_inputs
    out = {}
    w = CONV_WORKLOADS["conv_m2p7_bf16"]
    inp = make_conv_inputs(w, with_state=True)
    d = {k: v.cuda() for k, v in inp.items()}
    Bt, T, Dc = d["x"].shape
    K = d["weight"].shape[1]
    es = d["x"].element_size()
    nbytes = conv_bytes(Bt, T, Dc, K, es)
    nsets = max(1, math.ceil(2 * MALL_BYTES / nbytes))
    xs = [d["x"]] + [torch.randn_like(d["x"], dtype=torch.float32).to(d["x"].dtype)
                     for _ in range(nsets - 1)]
    ys = [torch.empty_like(d["x"]) for _ in range(nsets)]
    sts = [torch.empty_like(d["state"]) for _ in range(nsets)]
    for i in range(max(1, warmup)):
        ssd.ssd_conv1d(xs[i % nsets], d["weight"], d["bias"], state=d["state"], y=ys[i % nsets],
                       state_out=sts[i % nsets])
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        ssd.ssd_conv1d(xs[i % nsets], d["weight"], d["bias"], state=d["state"], y=ys[i % nsets],
                       state_out=sts[i % nsets])
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    gbs = nbytes / (ms * 1e-3) / 1e9
    out["prefill"] = {"workload": w.name, "batch": Bt, "seqlen": T, "channels": Dc, "width": K,
                      "io_dtype": w.io_dtype, "silu": w.silu, "ms": ms,
                      "tokens_per_s": Bt * T / (ms * 1e-3), "bytes_per_launch": nbytes,
                      "rotated_sets": nsets,
                      "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                   "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                   "traffic": traffic_for("conv1d", w.name)}}
    wd = CONV_WORKLOADS["conv_m2p7_decode"]
    inp = make_conv_inputs(wd.with_(seqlen=steps_n), with_state=True)
    dd = {k: v.cuda() for k, v in inp.items()}
    Bt = wd.batch
    xs = dd["x"].transpose(0, 1).contiguous()        # [steps, Bt, D]
    ys = torch.empty_like(xs)
    win_bytes = Bt * Dc * (K - 1) * es
    nwin = max(1, math.ceil(2 * MALL_BYTES / (win_bytes + 2 * Bt * Dc * es)))
    nwin = min(nwin, steps_n)
    wins = [dd["state"].clone() for _ in range(nwin)]

    def body():
        for t in range(steps_n):
            ssd.ssd_conv1d_step(wins[t % nwin], xs[t], dd["weight"], dd["bias"], y_t=ys[t])

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        body()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (3 * steps_n)
    sbytes = conv_bytes(Bt, 1, Dc, K, es)
    gbs = sbytes / (ms_step * 1e-3) / 1e9
    out["step"] = {"workload": wd.name, "batch": Bt, "channels": Dc, "width": K,
                   "io_dtype": wd.io_dtype, "steps": steps_n, "graph_replays": 3,
                   "us_per_step": ms_step * 1e3, "tokens_per_s": Bt / (ms_step * 1e-3),
                   "bytes_per_step": sbytes, "windows": nwin,
                   "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS,
                                "unit": "GB/s", "frac": gbs / PEAK_HBM_GBS,
                                "traffic": traffic_for("conv1d", f"{wd.name}_b{Bt}")}}
    return out


def cpu_baseline(w, target_s=10.0):
    """The fp64 oracle on the host cores, on a bounded sample of the workload."""
    import oracle
    from ssd_inputs import make_inputs
    threads = oracle.max_threads()
    inp = make_inputs(w)
    Bt, H = w.batch, w.nheads
    pairs_full = Bt * H
    # sample: batch row 0, the first k heads (k = all heads if they fit ~2 rounds of threads)
    k = H if (Bt == 1 and H <= 4 * threads) else min(H, 2 * threads)
    sl = {kk: v for kk, v in inp.items()}
    if k < H or Bt > 1:
        sl = {"x": inp["x"][:1, :, :k], "dt": inp["dt"][:1, :, :k], "A": inp["A"][:k],
              "B": inp["B"][:1], "C": inp["C"][:1], "D": inp["D"][:k], "dt_bias": inp["dt_bias"][:k]}
    t0 = time.perf_counter()
    reps = 0
    while True:
        oracle.scan(sl["x"], sl["dt"], sl["A"], sl["B"], sl["C"], sl["D"], sl["dt_bias"], None,
                    dt_min=w.dt_min, dt_max=w.dt_max)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el * (reps + 1) / reps > 3 * target_s:
            break
    per_rep = el / reps
    scale = pairs_full / k          # the full workload has this many times the (b, h) pairs
    full_s = per_rep * scale
    # one thread, one (b, h) sequence: the oracle's serial rate, scaled the same way
    one = {kk: (v[:1, :, :1] if kk in ("x", "dt") else v[:1] if kk in ("B", "C") else v[:1])
           for kk, v in sl.items()}
    t1 = time.perf_counter()
    oracle.scan(one["x"], one["dt"], one["A"], one["B"], one["C"], one["D"], one["dt_bias"], None,
                dt_min=w.dt_min, dt_max=w.dt_max, nthreads=1)
    one_s = (time.perf_counter() - t1) * pairs_full
    return {"value": Bt * w.seqlen / full_s, "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "value_1_thread": Bt * w.seqlen / one_s,
            "sample": (f"fp64 recurrence on {k} of {pairs_full} (batch, head) sequences of "
                       f"{w.seqlen} tokens, {reps} repetition(s) in {el:.1f} s, scaled by "
                       f"{scale:g} to the whole workload; host CPU: {cpu_model()}")}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="one decode batch size (default: 1, 16 and 64)")
    ap.add_argument("--no-sub-configs", action="store_true",
                    help="skip the 130M- and 2.7B-shaped prefill lines")
    ap.add_argument("--decode-steps", type=int, default=1024)
    ap.add_argument("--chunk", type=int, default=0, help="override the workload's chunk size")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the gradients (their reversed scan reuses the forward kernels)")
    ap.add_argument("--backward-only", action="store_true",
                    help="only time the scan's gradients (ssd_chunk_scan_backward) on the workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the known-size copy used to calibrate the HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the library has no multi-GPU path "
              "(batch rows and heads are independent, so a split over GPUs would need "
              "no communication in the forward scan).",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import state_space_model_amd as ssd
    from ssd_inputs import WORKLOADS
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        print(json.dumps(copy_calibration(ssd, torch)))
        return
    w = WORKLOADS[args.workload]
    if args.chunk:
        w = w.with_(chunk=args.chunk)
    if args.backward_only:
        print(f"[bench] backward {w.name} L={w.chunk}", file=sys.stderr, flush=True)
        print(json.dumps(bench_backward(ssd, torch, w)))
        return
    print(f"[bench] prefill {w.name} L={w.chunk} steps={args.steps} warmup={args.warmup}",
          file=sys.stderr, flush=True)
    pf = bench_prefill(ssd, torch, w, args.steps, args.warmup)
    head, roof = prefill_report(w, pf, headline=True)
    out = {
        "metric": METRIC, "value": head["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pf["ms"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.io_dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seqlen": w.seqlen, "nheads": w.nheads,
                   "headdim": w.headdim, "dstate": w.dstate, "ngroups": w.ngroups,
                   "chunk": w.chunk, "io_dtype": w.io_dtype, "parallelism": "single GPU"},
        "roofline": roof,
        "prefill": head,
    }
    if not args.no_sub_configs and args.workload == DEFAULT_WORKLOAD and not args.chunk:
        out["prefill_configs"] = {}
        for name in SUB_WORKLOADS:
            ws = WORKLOADS[name]
            print(f"[bench] prefill {name} L={ws.chunk}", file=sys.stderr, flush=True)
            out["prefill_configs"][name] = prefill_report(
                ws, bench_prefill(ssd, torch, ws, args.steps, args.warmup))[0]
    if not args.no_decode:
        out["decode"] = {}
        batches = DECODE_BATCHES if args.decode_batch == 0 else (args.decode_batch,)
        for b in batches:
            print(f"[bench] decode b={b} steps={args.decode_steps}", file=sys.stderr, flush=True)
            out["decode"][f"b{b}"] = bench_decode(ssd, torch, b, args.decode_steps, args.warmup)
        if 1 in batches:
            out["decode"]["b1"]["launch_floor_us"] = launch_floor_us(ssd, torch)
        print("[bench] cached decode vs recompute at 4096", file=sys.stderr, flush=True)
        out["cached_vs_recompute"] = bench_cached_vs_recompute(ssd, torch)
        print("[bench] conv1d prefill and step", file=sys.stderr, flush=True)
        out["conv1d"] = bench_conv(ssd, torch, args.warmup)
        if not args.no_backward:
            out["backward"] = {}
            for name in SUB_WORKLOADS:
                print(f"[bench] backward {name}", file=sys.stderr, flush=True)
                out["backward"][name] = bench_backward(ssd, torch, WORKLOADS[name])
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
