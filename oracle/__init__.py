"""CPU oracle for the Mamba-2 SSD scan and single-token step.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's CPU
baseline leg may import this package.  The GPU library neither imports nor
links anything here, and nothing here imports the GPU library.

Contents
  scan(...)         token-by-token fp64 recurrence (C, OpenMP over (b, h))
  step(...)         the same recurrence run for one token from a given state
  conv1d(...)       depthwise causal convolution over time with its k-1 input
                    window carried in and out (C, fp64)
  conv1d_step(...)  the same convolution for one token from a cached window
  scan_backward(...) gradients of the scan: the adjoint recurrence run
                    backwards in time from checkpointed states (C, fp64)
  dual_form.py      dense quadratic "dual form" materialisation (numpy, fp64)
  chunked.py        chunked SSD algorithm written step by step (numpy, fp64)
  brute.py          the recurrence at 50 significant digits (mpmath)

The source is "Compiler-First State Space Duality and Portable O(1)
Autoregressive Caching" (Background, Eq. 1-3; SSD properties; O(1) cache;
Setup for the convolution width).
The recurrence is what the chunked method computes faster; the other three are
independent formulations used to pin it.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from . import build as _build

_lib = None


def _load():
    global _lib
    if _lib is None:
        path = _build.build(force=False)
        lib = ctypes.CDLL(path)
        lib.ssd_oracle_scan.restype = ctypes.c_int
        i64, vp = ctypes.c_int64, ctypes.c_void_p
        lib.ssd_oracle_scan.argtypes = [i64] * 6 + [vp] * 8 + [ctypes.c_int, ctypes.c_double,
                                                           ctypes.c_double, vp, vp, ctypes.c_int]
        lib.ssd_oracle_conv1d.restype = ctypes.c_int
        lib.ssd_oracle_conv1d.argtypes = [i64] * 4 + [vp] * 4 + [ctypes.c_int, vp, vp, ctypes.c_int]
        lib.ssd_oracle_scan_backward.restype = ctypes.c_int
        lib.ssd_oracle_scan_backward.argtypes = ([i64] * 6 + [vp] * 8 + [ctypes.c_int, ctypes.c_double,
                                                 ctypes.c_double] + [vp] * 11 + [ctypes.c_int])
        lib.ssd_oracle_max_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def max_threads() -> int:
    return int(_load().ssd_oracle_max_threads())


def _f32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: exact upcast (bf16 -> f32 is exact)
        import torch
        a = a.detach().to("cpu", torch.float32).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float64).contiguous().numpy()
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def scan(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, dt_softplus: bool = True,
         dt_min: float = 1e-4, dt_max: float = 0.5, nthreads: int = 0
         ) -> Tuple[np.ndarray, np.ndarray]:
    """Run the fp64 token-by-token recurrence.

    Shapes: x [Bt,T,H,P], dt [Bt,T,H], A/D/dt_bias [H], B/C [Bt,T,G,N],
    h0 [Bt,H,P,N] (None means zeros).  Float inputs are taken as float32
    values (bf16 tensors upcast exactly); h0 is taken in float64.
    dt_min/dt_max are compared in double against d, after rounding them to
    float32 as the C-ABI receives them.
    Returns (y [Bt,T,H,P], final_state [Bt,H,P,N]), both float64.
    """
    x, dt, A, B, C = _f32(x), _f32(dt), _f32(A), _f32(B), _f32(C)
    D, dt_bias, h0 = _f32(D), _f32(dt_bias), _f64(h0)
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (Bt, T, H) and A.shape == (H,)
    assert B.shape == (Bt, T, G, N) and C.shape == (Bt, T, G, N)
    assert D is None or D.shape == (H,)
    assert dt_bias is None or dt_bias.shape == (H,)
    assert h0 is None or h0.shape == (Bt, H, P, N)
    y = np.empty((Bt, T, H, P), dtype=np.float64)
    fin = np.empty((Bt, H, P, N), dtype=np.float64)
    lo = float(np.float32(dt_min))
    hi = float(np.float32(dt_max))
    rc = _load().ssd_oracle_scan(Bt, T, H, P, N, G, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
                                 _ptr(B), _ptr(C), _ptr(D), _ptr(h0), int(bool(dt_softplus)),
                                 lo, hi, _ptr(y), _ptr(fin), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_scan failed with code {rc}")
    return y, fin


def step(state, x_t, dt_t, A, B_t, C_t, D=None, dt_bias=None, *, dt_softplus: bool = True,
         dt_min: float = 1e-4, dt_max: float = 0.5) -> Tuple[np.ndarray, np.ndarray]:
    """One recurrence step: state [Bt,H,P,N], x_t [Bt,H,P], dt_t [Bt,H],
    B_t/C_t [Bt,G,N].  Returns (y_t [Bt,H,P], new_state), both float64."""
    x_t, dt_t, B_t, C_t = _f32(x_t), _f32(dt_t), _f32(B_t), _f32(C_t)
    y, fin = scan(x_t[:, None], dt_t[:, None], A, B_t[:, None], C_t[:, None], D, dt_bias,
                  state, dt_softplus=dt_softplus, dt_min=dt_min, dt_max=dt_max)
    return y[:, 0], fin


def conv1d(x, w, bias=None, state=None, *, silu: bool = False, nthreads: int = 0
           ) -> Tuple[np.ndarray, np.ndarray]:
    """Depthwise causal convolution over time (O(1) cache section: a sliding
    window of the k-1 previous inputs per channel; Setup: k = 4).

    Shapes: x [Bt,T,D], w [D,k] (w[c][0] multiplies the oldest input of the
    window, w[c][k-1] the current one), bias [D] or None, state [Bt,D,k-1]
    (the k-1 inputs before x[:,0], oldest first) or None for zeros.
    Float inputs are taken as float32 values; state in float64.
    Returns (y [Bt,T,D], state_out [Bt,D,k-1] = the last k-1 inputs), float64.
    """
    x, w, bias, state = _f32(x), _f32(w), _f32(bias), _f64(state)
    Bt, T, D = x.shape
    K = w.shape[1]
    assert w.shape == (D, K) and K >= 1
    assert bias is None or bias.shape == (D,)
    assert state is None or state.shape == (Bt, D, K - 1)
    y = np.empty((Bt, T, D), dtype=np.float64)
    st = np.empty((Bt, D, K - 1), dtype=np.float64)
    rc = _load().ssd_oracle_conv1d(Bt, T, D, K, _ptr(x), _ptr(w), _ptr(bias), _ptr(state),
                                   int(bool(silu)), _ptr(y), _ptr(st), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_conv1d failed with code {rc}")
    return y, st


def conv1d_step(state, x_t, w, bias=None, *, silu: bool = False
                ) -> Tuple[np.ndarray, np.ndarray]:
    """One token of conv1d from a cached window: state [Bt,D,k-1], x_t [Bt,D].
    Returns (y_t [Bt,D], new_state [Bt,D,k-1]), both float64."""
    x_t = _f32(x_t)
    y, st = conv1d(x_t[:, None], w, bias, state, silu=silu)
    return y[:, 0], st


def scan_backward(x, dt, A, B, C, D=None, dt_bias=None, h0=None, *, dy, dfinal=None,
                  dt_softplus: bool = True, dt_min: float = 1e-4, dt_max: float = 0.5,
                  nthreads: int = 0) -> dict:
    """Gradients of L = sum(dy * y) + sum(dfinal * final_state) of scan(...)
    with respect to every input, by the adjoint recurrence in fp64.

    dy [Bt,T,H,P] and dfinal [Bt,H,P,N] (None: zeros) are taken in float64.
    Returns a dict of float64 arrays: dx, ddt (w.r.t. the pre-activation dt),
    dA, dB, dC, dD, ddt_bias, dh0 (shapes of the inputs; dD, ddt_bias and dA
    are [H], computed also when D or dt_bias is None), and dlda [Bt,T,H] =
    dL/d(Delta_t A), whose Delta-weighted sum over (b, t) is dA."""
    x, dt, A, B, C = _f32(x), _f32(dt), _f32(A), _f32(B), _f32(C)
    D, dt_bias, h0 = _f32(D), _f32(dt_bias), _f64(h0)
    dy, dfinal = _f64(dy), _f64(dfinal)
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dy.shape == (Bt, T, H, P)
    assert dfinal is None or dfinal.shape == (Bt, H, P, N)
    out = {"dx": np.empty((Bt, T, H, P)), "ddt": np.empty((Bt, T, H)), "dA": np.empty(H),
           "dB": np.empty((Bt, T, G, N)), "dC": np.empty((Bt, T, G, N)), "dD": np.empty(H),
           "ddt_bias": np.empty(H), "dh0": np.empty((Bt, H, P, N)), "dlda": np.empty((Bt, T, H))}
    lo = float(np.float32(dt_min))
    hi = float(np.float32(dt_max))
    rc = _load().ssd_oracle_scan_backward(
        Bt, T, H, P, N, G, _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(h0), int(bool(dt_softplus)), lo, hi, _ptr(dy), _ptr(dfinal), _ptr(out["dx"]),
        _ptr(out["ddt"]), _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]),
        _ptr(out["ddt_bias"]), _ptr(out["dh0"]), _ptr(out["dlda"]), int(nthreads))
    if rc != 0:
        raise RuntimeError(f"ssd_oracle_scan_backward failed with code {rc}")
    return out
