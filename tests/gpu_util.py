"""Shared helpers of the GPU parity tests (device transfer, oracle slices)."""
from __future__ import annotations

import functools
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle.metrics import state_err, step_y_err, y_err
from ssd_inputs import WORKLOADS, make_inputs

# Tolerances (max over (b, h) slices of ||got - ref||_inf / ||ref||_inf):
# float32 inputs 1e-4; bfloat16 x/B/C with float32 decay, state and
# accumulation 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def gpu_available() -> bool:
    try:
        return torch.cuda.is_available() and torch.cuda.device_count() > 0
    except Exception:
        return False


def need_gpu():
    if not gpu_available():
        pytest.skip("no GPU")


def announce(msg: str):
    """Name the case before a GPU step, so a crash can be attributed."""
    print(f"\n[gpu-case] {msg}", file=sys.stderr, flush=True)


def to_dev(inp: dict) -> dict:
    return {k: v.to("cuda") for k, v in inp.items()}


@functools.lru_cache(maxsize=2)
def workload_inputs(name: str, with_h0: bool = False):
    return make_inputs(WORKLOADS[name], with_initial_state=with_h0)


def oracle_scan(inp: dict, w, h0=None):
    return oracle.scan(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp.get("D"),
                       inp.get("dt_bias"), h0 if h0 is not None else inp.get("h0"),
                       dt_softplus=True, dt_min=w.dt_min, dt_max=w.dt_max)


def slice_bh(inp: dict, b: int, h: int, G: int, H: int) -> dict:
    """The independent sub-problem of batch row b and head h (H = 1)."""
    g = h // (H // G)
    out = {}
    for k, v in inp.items():
        if k == "x":
            out[k] = v[b:b + 1, :, h:h + 1]
        elif k == "dt":
            out[k] = v[b:b + 1, :, h:h + 1]
        elif k in ("B", "C"):
            out[k] = v[b:b + 1, :, g:g + 1]
        elif k in ("A", "D", "dt_bias"):
            out[k] = v[h:h + 1]
        elif k == "h0":
            out[k] = v[b:b + 1, h:h + 1]
        else:
            out[k] = v
    return out


__all__ = ["TOL", "need_gpu", "announce", "to_dev", "workload_inputs", "oracle_scan", "slice_bh",
           "y_err", "state_err", "step_y_err", "np"]
