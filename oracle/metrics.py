"""Error metrics for comparing a result with the oracle (test infrastructure).

The error of a result R against a reference Ref is taken per (b, h) slice as
||R - Ref||_inf / ||Ref||_inf and the maximum over slices is reported.  The
pages give tolerances only at model level; this slice-normalised max-norm is
the reading used for the per-layer tolerances (1e-4 for float32 inputs, 2e-2
for bfloat16 inputs with float32 accumulation and state).
"""
from __future__ import annotations

import numpy as np


def _as64(a):
    if hasattr(a, "detach"):
        import torch
        a = a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, np.float64)


def slice_rel_err(got, ref, head_axis: int, other_axes) -> float:
    """max over (batch, head) slices of ||got-ref||_inf / ||ref||_inf.

    head_axis: axis of the head index; other_axes: axes reduced inside a slice
    (all axes except batch (axis 0) and head)."""
    g, r = _as64(got), _as64(ref)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if g.size == 0:
        return 0.0
    if not np.all(np.isfinite(g)):
        return float("inf")
    num = np.abs(g - r).max(axis=tuple(other_axes))
    den = np.abs(r).max(axis=tuple(other_axes))
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def y_err(got, ref) -> float:
    """y / x layout [Bt, T, H, P]."""
    return slice_rel_err(got, ref, 2, (1, 3))


def state_err(got, ref) -> float:
    """state layout [Bt, H, P, N]."""
    return slice_rel_err(got, ref, 1, (2, 3))


def step_y_err(got, ref) -> float:
    """y_t layout [Bt, H, P]."""
    return slice_rel_err(got, ref, 1, (2,))


def token_rel_err(got, ref, floor: float = 1e-3) -> float:
    """max over (b, t, h) of ||got-ref||_inf / ||ref||_inf taken over one
    token's P outputs, the denominator floored at `floor` times its (b, h)
    slice's ||ref||_inf (tokens whose output is near zero would otherwise
    divide by almost nothing).  Layout [Bt, T, H, P].  Reported beside the
    slice metric: it shows a local error that a slice's largest value could
    hide."""
    g, r = _as64(got), _as64(ref)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch {g.shape} vs {r.shape}")
    if g.size == 0:
        return 0.0
    num = np.abs(g - r).max(axis=3)
    den = np.abs(r).max(axis=3)
    slice_den = np.abs(r).max(axis=(1, 3), keepdims=True)[..., 0]
    den = np.maximum(den, floor * np.where(slice_den > 0, slice_den, 1.0))
    return float((num / den).max())
