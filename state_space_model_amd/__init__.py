"""Python binding of libssd, the gfx950 Mamba-2 SSD library.

Argument marshalling only: every step of the scan and of the decode step runs
in the HIP kernels behind the C ABI declared in include/ssd.h.  PyTorch is
used for device memory and for the current HIP stream; there is no CPU or
PyTorch fallback -- if libssd.so is missing, importing this package raises.

  ssd_chunk_scan(x, dt, A, B, C, D=None, *, chunk=256, ...) -> (y, final_state)
  ssd_step(state, x_t, dt_t, A, B_t, C_t, D=None, ...)      -> y_t  (state updated in place)
  ssd_chunk_scan_workspace_bytes(...)                        -> int

Source: "Compiler-First State Space Duality and Portable O(1) Autoregressive
Caching" (Background, Eq. 2-3; O(1) cache).
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libssd.so")

SSD_OK = 0
SSD_F32 = 0
SSD_BF16 = 1
SSD_SCAN_PHASES = 4
SSD_SCHEDULE_PHASED = 0
SSD_SCHEDULE_CHAIN = 1
STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_INVALID_ARG", 2: "SSD_ERR_SHAPE", 3: "SSD_ERR_DTYPE",
                4: "SSD_ERR_ALIGNMENT", 5: "SSD_ERR_UNSUPPORTED", 6: "SSD_ERR_WORKSPACE",
                7: "SSD_ERR_HIP"}
SSD_VARIANT_DEFAULT = 0
SSD_VARIANT_BF16_DECAY = 1
SSD_VARIANT_LOADED_MASK = 2
SSD_NOALLOC_MAX_WORKSPACE = 96 << 20
EXPORTED = ("ssd_chunk_scan", "ssd_chunk_scan_timed", "ssd_chunk_scan_workspace_bytes",
            "ssd_chunk_scan_schedule", "ssd_chunk_scan_ablation", "ssd_chunk_scan_noalloc",
            "ssd_step", "ssd_conv1d", "ssd_conv1d_step",
            "ssd_chunk_scan_backward", "ssd_chunk_scan_backward_workspace_bytes",
            "ssd_status_string", "ssd_abi_version")


class ScanDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("dt_softplus", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


class StepDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("nheads", ctypes.c_int64),
                ("headdim", ctypes.c_int64), ("dstate", ctypes.c_int64),
                ("ngroups", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("dt_softplus", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


class ConvDesc(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("channels", ctypes.c_int64), ("width", ctypes.c_int64),
                ("io_dtype", ctypes.c_int32), ("silu", ctypes.c_int32)]


class SSDError(RuntimeError):
    def __init__(self, status: int, where: str = ""):
        self.status = int(status)
        msg = lib.ssd_status_string(self.status).decode()
        super().__init__(f"{where}: {msg}" if where else msg)


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build the gfx950 library first "
            "(python -c 'import __graft_entry__ as g; g.build()' or "
            "python state_space_model_amd/build.py). There is no CPU fallback.")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    L.ssd_chunk_scan.restype = i32
    L.ssd_chunk_scan.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 11 + [sz, vp]
    L.ssd_chunk_scan_timed.restype = i32
    L.ssd_chunk_scan_timed.argtypes = ([ctypes.POINTER(ScanDesc)] + [vp] * 11 + [sz, vp]
                                       + [ctypes.POINTER(vp), ctypes.c_int])
    L.ssd_chunk_scan_ablation.restype = i32
    L.ssd_chunk_scan_ablation.argtypes = ([ctypes.POINTER(ScanDesc), i32] + [vp] * 11 + [sz, vp])
    L.ssd_chunk_scan_noalloc.restype = i32
    L.ssd_chunk_scan_noalloc.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 10 + [vp]
    L.ssd_chunk_scan_workspace_bytes.restype = sz
    L.ssd_chunk_scan_workspace_bytes.argtypes = [ctypes.POINTER(ScanDesc)]
    L.ssd_chunk_scan_schedule.restype = i32
    L.ssd_chunk_scan_schedule.argtypes = [ctypes.POINTER(ScanDesc)]
    L.ssd_step.restype = i32
    L.ssd_step.argtypes = [ctypes.POINTER(StepDesc)] + [vp] * 9 + [vp]
    L.ssd_chunk_scan_backward.restype = i32
    L.ssd_chunk_scan_backward.argtypes = [ctypes.POINTER(ScanDesc)] + [vp] * 19 + [sz, vp]
    L.ssd_chunk_scan_backward_workspace_bytes.restype = sz
    L.ssd_chunk_scan_backward_workspace_bytes.argtypes = [ctypes.POINTER(ScanDesc)]
    L.ssd_conv1d.restype = i32
    L.ssd_conv1d.argtypes = [ctypes.POINTER(ConvDesc)] + [vp] * 6 + [vp]
    L.ssd_conv1d_step.restype = i32
    L.ssd_conv1d_step.argtypes = [ctypes.POINTER(ConvDesc)] + [vp] * 5 + [vp]
    L.ssd_status_string.restype = ctypes.c_char_p
    L.ssd_status_string.argtypes = [i32]
    L.ssd_abi_version.restype = i32
    L.ssd_abi_version.argtypes = []
    return L


lib = _load()


def _io_code(dtype: torch.dtype) -> int:
    if dtype == torch.float32:
        return SSD_F32
    if dtype == torch.bfloat16:
        return SSD_BF16
    raise TypeError(f"x, B, C must be float32 or bfloat16, got {dtype}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: Optional[torch.Tensor], name: str, dtype=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (got {t.device}); there is no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")


def _shape(t: Optional[torch.Tensor], name: str, shape) -> None:
    """Raise ValueError unless t is None or has exactly `shape`.  The C ABI
    receives bare pointers and cannot see a buffer's extent, so every tensor's
    shape is checked here, before any launch."""
    if t is not None and tuple(t.shape) != tuple(int(v) for v in shape):
        raise ValueError(f"{name} must have shape {tuple(int(v) for v in shape)}, "
                         f"got {tuple(t.shape)}")


def _nbytes(t: torch.Tensor) -> int:
    return t.numel() * t.element_size()


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _scan_shapes(x, dt, A, B, C, D=None, dt_bias=None, initial_state=None) -> None:
    """Shapes of a scan's inputs against (Bt, T, H, P) of x and (G, N) of B."""
    if x.dim() != 4 or B.dim() != 4:
        raise ValueError("x must be [Bt,T,H,P] and B, C [Bt,T,G,N]")
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _shape(B, "B", (Bt, T, G, N))
    _shape(C, "C", (Bt, T, G, N))
    _shape(dt, "dt", (Bt, T, H))
    for t, n in ((A, "A"), (D, "D"), (dt_bias, "dt_bias")):
        _shape(t, n, (H,))
    _shape(initial_state, "initial_state", (Bt, H, P, N))


def scan_desc(x: torch.Tensor, B: torch.Tensor, chunk: int, dt_softplus: bool,
              dt_limit: Sequence[float]) -> ScanDesc:
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    return ScanDesc(Bt, T, H, P, N, G, int(chunk), _io_code(x.dtype), int(bool(dt_softplus)),
                    float(dt_limit[0]), float(dt_limit[1]))


def ssd_chunk_scan_workspace_bytes(x: torch.Tensor, B: torch.Tensor, chunk: int = 256) -> int:
    d = scan_desc(x, B, chunk, True, (1e-4, 0.5))
    return int(lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(d)))


def ssd_chunk_scan_schedule(x: torch.Tensor, B: torch.Tensor, chunk: int = 256) -> int:
    """SSD_SCHEDULE_PHASED or SSD_SCHEDULE_CHAIN: the kernel schedule a scan of
    these shapes runs (both give bit-identical results)."""
    d = scan_desc(x, B, chunk, True, (1e-4, 0.5))
    r = int(lib.ssd_chunk_scan_schedule(ctypes.byref(d)))
    if r < 0:
        raise SSDError(-r, "ssd_chunk_scan_schedule")
    return r


def ssd_chunk_scan(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                   C: torch.Tensor, D: Optional[torch.Tensor] = None, *, chunk: int = 256,
                   dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = True,
                   dt_limit: Sequence[float] = (1e-4, 0.5),
                   initial_state: Optional[torch.Tensor] = None,
                   return_final_state: bool = True,
                   y: Optional[torch.Tensor] = None, final_state: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None,
                   phase_events: Optional[Sequence[torch.cuda.Event]] = None,
                   variant: int = SSD_VARIANT_DEFAULT
                   ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Chunked SSD scan (prefill) on the current stream.

    x [Bt,T,H,P], B/C [Bt,T,G,N] in float32 or bfloat16 (same dtype);
    dt [Bt,T,H], A/D/dt_bias [H], initial_state [Bt,H,P,N] float32.
    Returns (y [Bt,T,H,P] in x's dtype, final_state [Bt,H,P,N] float32 or None).
    Output and workspace tensors may be passed in to avoid allocation.
    `phase_events`: optional SSD_SCAN_PHASES+1 torch.cuda.Event objects
    (created with enable_timing=True) recorded around the scan's kernels.
    `variant`: SSD_VARIANT_BF16_DECAY or SSD_VARIANT_LOADED_MASK runs the
    ablation variant of the output path (ssd_chunk_scan_ablation).
    """
    _scan_shapes(x, dt, A, B, C, D, dt_bias, initial_state)
    Bt, T, H, P = x.shape
    N = B.shape[3]
    _shape(y, "y", (Bt, T, H, P))
    _shape(final_state, "final_state", (Bt, H, P, N))
    for t, n, dt_ in ((x, "x", None), (B, "B", x.dtype), (C, "C", x.dtype), (dt, "dt", torch.float32),
                      (A, "A", torch.float32), (D, "D", torch.float32),
                      (dt_bias, "dt_bias", torch.float32),
                      (initial_state, "initial_state", torch.float32)):
        _check(t, n, dt_)
    desc = scan_desc(x, B, chunk, dt_softplus, dt_limit)
    dev = x.device
    if y is None:
        y = torch.empty_like(x)
    if final_state is None and return_final_state:
        final_state = torch.empty((Bt, H, P, N), dtype=torch.float32, device=dev)
    _check(y, "y", x.dtype)
    _check(final_state, "final_state", torch.float32)
    need = int(lib.ssd_chunk_scan_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace")
    wbytes = _nbytes(workspace)
    args = (ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C),
            _ptr(D), _ptr(initial_state), _ptr(y), _ptr(final_state), _ptr(workspace),
            ctypes.c_size_t(wbytes), _stream(dev))
    if variant != SSD_VARIANT_DEFAULT:
        if phase_events is not None:
            raise ValueError("phase_events time the default variant only")
        st = lib.ssd_chunk_scan_ablation(args[0], int(variant), *args[1:])
    elif phase_events is None:
        st = lib.ssd_chunk_scan(*args)
    else:
        for e in phase_events:  # torch creates the HIP event at its first record
            if not e.cuda_event:
                e.record()
        evs = (ctypes.c_void_p * len(phase_events))(*[ctypes.c_void_p(e.cuda_event)
                                                      for e in phase_events])
        st = lib.ssd_chunk_scan_timed(*args, evs, len(phase_events))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_scan")
    return y, final_state


def ssd_chunk_scan_noalloc(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                           C: torch.Tensor, D: Optional[torch.Tensor] = None, *, chunk: int = 256,
                           dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = True,
                           dt_limit: Sequence[float] = (1e-4, 0.5),
                           initial_state: Optional[torch.Tensor] = None,
                           y: Optional[torch.Tensor] = None,
                           final_state: Optional[torch.Tensor] = None
                           ) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """ssd_chunk_scan through the allocation-free entry point: the library
    uses its static per-device scratch (at most SSD_NOALLOC_MAX_WORKSPACE
    bytes) instead of a workspace.  Pass y (and final_state, or None for no
    final state) to make the call allocate nothing here either."""
    _scan_shapes(x, dt, A, B, C, D, dt_bias, initial_state)
    Bt, T, H, P = x.shape
    N = B.shape[3]
    _shape(y, "y", (Bt, T, H, P))
    _shape(final_state, "final_state", (Bt, H, P, N))
    for t, n, dt_ in ((x, "x", None), (B, "B", x.dtype), (C, "C", x.dtype), (dt, "dt", torch.float32),
                      (A, "A", torch.float32), (D, "D", torch.float32),
                      (dt_bias, "dt_bias", torch.float32),
                      (initial_state, "initial_state", torch.float32), (y, "y", x.dtype),
                      (final_state, "final_state", torch.float32)):
        _check(t, n, dt_)
    desc = scan_desc(x, B, chunk, dt_softplus, dt_limit)
    if y is None:
        y = torch.empty_like(x)
    st = lib.ssd_chunk_scan_noalloc(ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A),
                                    _ptr(B), _ptr(C), _ptr(D), _ptr(initial_state), _ptr(y),
                                    _ptr(final_state), _stream(x.device))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_scan_noalloc")
    return y, final_state


def step_desc(state: torch.Tensor, x_t: torch.Tensor, B_t: torch.Tensor, dt_softplus: bool,
              dt_limit: Sequence[float]) -> StepDesc:
    Bt, H, P, N = state.shape
    return StepDesc(Bt, H, P, N, B_t.shape[1], _io_code(x_t.dtype), int(bool(dt_softplus)),
                    float(dt_limit[0]), float(dt_limit[1]))


def ssd_step(state: torch.Tensor, x_t: torch.Tensor, dt_t: torch.Tensor, A: torch.Tensor,
             B_t: torch.Tensor, C_t: torch.Tensor, D: Optional[torch.Tensor] = None, *,
             dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = True,
             dt_limit: Sequence[float] = (1e-4, 0.5),
             y_t: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One decode step on the current stream; `state` [Bt,H,P,N] float32 is
    updated in place.  x_t [Bt,H,P], B_t/C_t [Bt,G,N] (float32 or bfloat16),
    dt_t [Bt,H] float32.  Returns y_t [Bt,H,P] in x_t's dtype."""
    if state.dim() != 4 or B_t.dim() != 3:
        raise ValueError("state [Bt,H,P,N], x_t [Bt,H,P], B_t/C_t [Bt,G,N]")
    Bt, H, P, N = state.shape
    G = B_t.shape[1]
    _shape(x_t, "x_t", (Bt, H, P))
    _shape(dt_t, "dt_t", (Bt, H))
    _shape(B_t, "B_t", (Bt, G, N))
    _shape(C_t, "C_t", (Bt, G, N))
    for t, n in ((A, "A"), (D, "D"), (dt_bias, "dt_bias")):
        _shape(t, n, (H,))
    _shape(y_t, "y_t", (Bt, H, P))
    for t, n, dt_ in ((state, "state", torch.float32), (x_t, "x_t", None),
                      (B_t, "B_t", x_t.dtype), (C_t, "C_t", x_t.dtype),
                      (dt_t, "dt_t", torch.float32), (A, "A", torch.float32),
                      (D, "D", torch.float32), (dt_bias, "dt_bias", torch.float32)):
        _check(t, n, dt_)
    desc = step_desc(state, x_t, B_t, dt_softplus, dt_limit)
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _check(y_t, "y_t", x_t.dtype)
    st = lib.ssd_step(ctypes.byref(desc), _ptr(state), _ptr(x_t), _ptr(dt_t), _ptr(dt_bias),
                      _ptr(A), _ptr(B_t), _ptr(C_t), _ptr(D), _ptr(y_t), _stream(state.device))
    if st != SSD_OK:
        raise SSDError(st, "ssd_step")
    return y_t


def ssd_chunk_scan_backward_workspace_bytes(x: torch.Tensor, B: torch.Tensor,
                                            chunk: int = 256) -> int:
    d = scan_desc(x, B, chunk, True, (1e-4, 0.5))
    return int(lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(d)))


# shapes of the gradients ssd_chunk_scan_backward returns, in terms of (Bt, T, H, P, G, N)
_GRAD_SHAPES = {"dx": ("Bt", "T", "H", "P"), "ddt": ("Bt", "T", "H"), "dA": ("H",),
                "dB": ("Bt", "T", "G", "N"), "dC": ("Bt", "T", "G", "N"), "dD": ("H",),
                "ddt_bias": ("H",), "dinitial_state": ("Bt", "H", "P", "N")}


def ssd_chunk_scan_backward(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                            C: torch.Tensor, D: Optional[torch.Tensor] = None, *, dy: torch.Tensor,
                            dfinal_state: Optional[torch.Tensor] = None, chunk: int = 256,
                            dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = True,
                            dt_limit: Sequence[float] = (1e-4, 0.5),
                            initial_state: Optional[torch.Tensor] = None,
                            workspace: Optional[torch.Tensor] = None,
                            grads: Optional[dict] = None) -> dict:
    """Gradients of ssd_chunk_scan for L = sum(dy * y) + sum(dfinal_state *
    final_state), on the current stream.  dy has x's shape and dtype;
    dfinal_state [Bt,H,P,N] float32 or None.  Returns a dict of float32
    tensors dx, ddt, dA, dB, dC, dD, ddt_bias, dinitial_state (the last three
    always computed here)."""
    _scan_shapes(x, dt, A, B, C, D, dt_bias, initial_state)
    Bt, T, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    _shape(dy, "dy", (Bt, T, H, P))
    _shape(dfinal_state, "dfinal_state", (Bt, H, P, N))
    g = grads or {}
    unknown = set(g) - set(_GRAD_SHAPES)
    if unknown:
        raise ValueError(f"unknown gradient names {sorted(unknown)}")
    dims = dict(Bt=Bt, T=T, H=H, P=P, G=G, N=N)
    for k, v in g.items():
        _shape(v, k, tuple(dims[a] for a in _GRAD_SHAPES[k]))
    for t, n, dt_ in ((x, "x", None), (dt, "dt", torch.float32), (A, "A", torch.float32),
                      (B, "B", x.dtype), (C, "C", x.dtype), (D, "D", torch.float32),
                      (dt_bias, "dt_bias", torch.float32), (initial_state, "initial_state", torch.float32),
                      (dy, "dy", x.dtype), (dfinal_state, "dfinal_state", torch.float32)):
        _check(t, n, dt_)
    desc = scan_desc(x, B, chunk, dt_softplus, dt_limit)
    dev = x.device
    f32 = torch.float32
    out = {
        "dx": g.get("dx", torch.empty(Bt, T, H, P, device=dev, dtype=f32)),
        "ddt": g.get("ddt", torch.empty(Bt, T, H, device=dev, dtype=f32)),
        "dA": g.get("dA", torch.empty(H, device=dev, dtype=f32)),
        "dB": g.get("dB", torch.empty(Bt, T, G, N, device=dev, dtype=f32)),
        "dC": g.get("dC", torch.empty(Bt, T, G, N, device=dev, dtype=f32)),
        "dD": g.get("dD", torch.empty(H, device=dev, dtype=f32)),
        "ddt_bias": g.get("ddt_bias", torch.empty(H, device=dev, dtype=f32)),
        "dinitial_state": g.get("dinitial_state", torch.empty(Bt, H, P, N, device=dev, dtype=f32)),
    }
    for k, v in out.items():
        _check(v, k, f32)
    need = int(lib.ssd_chunk_scan_backward_workspace_bytes(ctypes.byref(desc)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(workspace, "workspace")
    st = lib.ssd_chunk_scan_backward(
        ctypes.byref(desc), _ptr(x), _ptr(dt), _ptr(dt_bias), _ptr(A), _ptr(B), _ptr(C), _ptr(D),
        _ptr(initial_state), _ptr(dy), _ptr(dfinal_state), _ptr(out["dx"]), _ptr(out["ddt"]),
        _ptr(out["dA"]), _ptr(out["dB"]), _ptr(out["dC"]), _ptr(out["dD"]), _ptr(out["ddt_bias"]),
        _ptr(out["dinitial_state"]), _ptr(workspace), ctypes.c_size_t(_nbytes(workspace)),
        _stream(dev))
    if st != SSD_OK:
        raise SSDError(st, "ssd_chunk_scan_backward")
    return out


def ssd_conv1d(x: torch.Tensor, weight: torch.Tensor, bias: Optional[torch.Tensor] = None, *,
               state: Optional[torch.Tensor] = None, silu: bool = True,
               y: Optional[torch.Tensor] = None, state_out: Optional[torch.Tensor] = None,
               return_state: bool = True) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Depthwise causal convolution over a sequence on the current stream.

    x [Bt,T,D] float32 or bfloat16; weight [D,k] float32 (weight[:, k-1]
    multiplies the current input); bias [D] float32 or None; state
    [Bt,D,k-1] in x's dtype (the k-1 inputs before x[:, 0], oldest first) or
    None for zeros.  Returns (y [Bt,T,D] in x's dtype, the outgoing window
    [Bt,D,k-1] or None when return_state is False).  state_out may be
    `state` itself (updated in place)."""
    if x.dim() != 3 or weight.dim() != 2 or weight.shape[0] != x.shape[2]:
        raise ValueError("x [Bt,T,D], weight [D,k]")
    Bt, T, Dc = x.shape
    K = weight.shape[1]
    _shape(bias, "bias", (Dc,))
    _shape(state, "state", (Bt, Dc, K - 1))
    _shape(y, "y", (Bt, T, Dc))
    _shape(state_out, "state_out", (Bt, Dc, K - 1))
    for t, n, dt_ in ((x, "x", None), (weight, "weight", torch.float32),
                      (bias, "bias", torch.float32), (state, "state", x.dtype)):
        _check(t, n, dt_)
    if y is None:
        y = torch.empty_like(x)
    if state_out is None and return_state:
        state_out = torch.empty(Bt, Dc, K - 1, dtype=x.dtype, device=x.device)
    _check(y, "y", x.dtype)
    _check(state_out, "state_out", x.dtype)
    desc = ConvDesc(Bt, T, Dc, K, _io_code(x.dtype), int(bool(silu)))
    st = lib.ssd_conv1d(ctypes.byref(desc), _ptr(x), _ptr(weight), _ptr(bias), _ptr(state),
                        _ptr(y), _ptr(state_out), _stream(x.device))
    if st != SSD_OK:
        raise SSDError(st, "ssd_conv1d")
    return y, state_out


def ssd_conv1d_step(state: torch.Tensor, x_t: torch.Tensor, weight: torch.Tensor,
                    bias: Optional[torch.Tensor] = None, *, silu: bool = True,
                    y_t: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One token of the convolution on the current stream; the window `state`
    [Bt,D,k-1] (x_t's dtype) is updated in place.  x_t [Bt,D].  Returns y_t."""
    if state.dim() != 3 or x_t.dim() != 2 or weight.dim() != 2:
        raise ValueError("state [Bt,D,k-1], x_t [Bt,D], weight [D,k]")
    Bt, Dc = x_t.shape
    K = weight.shape[1]
    _shape(weight, "weight", (Dc, K))
    _shape(state, "state", (Bt, Dc, K - 1))
    _shape(bias, "bias", (Dc,))
    _shape(y_t, "y_t", (Bt, Dc))
    for t, n, dt_ in ((state, "state", x_t.dtype), (x_t, "x_t", None),
                      (weight, "weight", torch.float32), (bias, "bias", torch.float32)):
        _check(t, n, dt_)
    if y_t is None:
        y_t = torch.empty_like(x_t)
    _check(y_t, "y_t", x_t.dtype)
    desc = ConvDesc(Bt, 1, Dc, K, _io_code(x_t.dtype), int(bool(silu)))
    st = lib.ssd_conv1d_step(ctypes.byref(desc), _ptr(state), _ptr(x_t), _ptr(weight),
                             _ptr(bias), _ptr(y_t), _stream(x_t.device))
    if st != SSD_OK:
        raise SSDError(st, "ssd_conv1d_step")
    return y_t


def abi_version() -> int:
    return int(lib.ssd_abi_version())
