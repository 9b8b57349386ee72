"""The Python binding checks every tensor's shape before anything reaches the
C ABI (which receives bare pointers and cannot see a buffer's extent).

Shapes are checked before device placement, so these run on the CPU: a
wrong shape raises ValueError naming the tensor; a well-shaped CPU tensor
still raises (there is no CPU path), so no kernel can be launched from here.
"""
import pytest
import torch

import state_space_model_amd as ssd

Bt, T, H, P, G, N = 2, 40, 4, 16, 2, 32


def scan_inputs(dtype=torch.float32):
    return dict(x=torch.zeros(Bt, T, H, P, dtype=dtype), dt=torch.zeros(Bt, T, H),
                A=-torch.ones(H), B=torch.zeros(Bt, T, G, N, dtype=dtype),
                C=torch.zeros(Bt, T, G, N, dtype=dtype), D=torch.zeros(H))


SCAN_BAD = [
    ("dt", torch.zeros(Bt, T, H + 1)),
    ("dt", torch.zeros(Bt, T - 1, H)),
    ("A", -torch.ones(H - 1)),
    ("D", torch.zeros(H, 1)),
    ("C", torch.zeros(Bt, T, G, N - 1)),
    ("C", torch.zeros(Bt - 1, T, G, N)),
    ("B", torch.zeros(Bt, T + 1, G, N)),
]


@pytest.mark.parametrize("name,bad", SCAN_BAD, ids=lambda v: v if isinstance(v, str) else "")
def test_scan_rejects_wrong_input_shapes(name, bad):
    kw = scan_inputs()
    kw[name] = bad
    if name == "B":   # B fixes (G, N); an inconsistent C is then the one reported
        kw["C"] = torch.zeros(Bt, T, G, N)
    with pytest.raises(ValueError, match="must have shape|must be \\[Bt"):
        ssd.ssd_chunk_scan(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"], chunk=32)


@pytest.mark.parametrize("opt,bad", [
    ("dt_bias", torch.zeros(H + 2)),
    ("initial_state", torch.zeros(Bt, H, P, N + 1)),
    ("y", torch.zeros(Bt, T, H, P + 1)),
    ("final_state", torch.zeros(Bt, H, P - 1, N)),
], ids=lambda v: v if isinstance(v, str) else "")
def test_scan_rejects_wrong_optional_and_output_shapes(opt, bad):
    kw = scan_inputs()
    with pytest.raises(ValueError, match=f"{opt} must have shape"):
        ssd.ssd_chunk_scan(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"], chunk=32,
                           **{opt: bad})


def test_scan_well_shaped_cpu_tensors_still_refused():
    kw = scan_inputs()
    with pytest.raises(ValueError, match="device tensor"):
        ssd.ssd_chunk_scan(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"], chunk=32)


def step_inputs():
    return dict(state=torch.zeros(Bt, H, P, N), x_t=torch.zeros(Bt, H, P),
                dt_t=torch.zeros(Bt, H), A=-torch.ones(H), B_t=torch.zeros(Bt, G, N),
                C_t=torch.zeros(Bt, G, N), D=torch.zeros(H))


@pytest.mark.parametrize("name,bad", [
    ("x_t", torch.zeros(Bt, H, P + 1)),
    ("x_t", torch.zeros(Bt + 1, H, P)),
    ("dt_t", torch.zeros(Bt, H - 1)),
    ("B_t", torch.zeros(Bt - 1, G, N)),
    ("C_t", torch.zeros(Bt, G, N + 2)),
    ("A", -torch.ones(H + 1)),
    ("D", torch.zeros(1)),
], ids=lambda v: v if isinstance(v, str) else "")
def test_step_rejects_wrong_shapes(name, bad):
    kw = step_inputs()
    kw[name] = bad
    with pytest.raises(ValueError, match="must have shape"):
        ssd.ssd_step(kw["state"], kw["x_t"], kw["dt_t"], kw["A"], kw["B_t"], kw["C_t"], kw["D"])


def test_step_rejects_wrong_output_and_bias_shapes():
    kw = step_inputs()
    with pytest.raises(ValueError, match="y_t must have shape"):
        ssd.ssd_step(kw["state"], kw["x_t"], kw["dt_t"], kw["A"], kw["B_t"], kw["C_t"], kw["D"],
                     y_t=torch.zeros(Bt, H, P - 1))
    with pytest.raises(ValueError, match="dt_bias must have shape"):
        ssd.ssd_step(kw["state"], kw["x_t"], kw["dt_t"], kw["A"], kw["B_t"], kw["C_t"], kw["D"],
                     dt_bias=torch.zeros(H * 2))


@pytest.mark.parametrize("name,bad", [
    ("dy", torch.zeros(Bt, T, H, P - 1)),
    ("dfinal_state", torch.zeros(Bt, H, P, N // 2)),
], ids=lambda v: v if isinstance(v, str) else "")
def test_backward_rejects_wrong_cotangent_shapes(name, bad):
    kw = scan_inputs()
    extra = {"dy": torch.zeros(Bt, T, H, P)}
    extra[name] = bad
    with pytest.raises(ValueError, match=f"{name} must have shape"):
        ssd.ssd_chunk_scan_backward(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"],
                                    chunk=32, **extra)


@pytest.mark.parametrize("gname,bad", [
    ("dx", torch.zeros(Bt, T, H, P + 1)),
    ("ddt", torch.zeros(Bt, T)),
    ("dA", torch.zeros(H + 1)),
    ("dB", torch.zeros(Bt, T, G, N - 1)),
    ("dC", torch.zeros(Bt, T, 1, N)),
    ("dinitial_state", torch.zeros(Bt, H, N, P)),
], ids=lambda v: v if isinstance(v, str) else "")
def test_backward_rejects_wrong_gradient_buffers(gname, bad):
    kw = scan_inputs()
    with pytest.raises(ValueError, match=f"{gname} must have shape"):
        ssd.ssd_chunk_scan_backward(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"],
                                    dy=torch.zeros(Bt, T, H, P), chunk=32, grads={gname: bad})
    with pytest.raises(ValueError, match="unknown gradient"):
        ssd.ssd_chunk_scan_backward(kw["x"], kw["dt"], kw["A"], kw["B"], kw["C"], kw["D"],
                                    dy=torch.zeros(Bt, T, H, P), chunk=32,
                                    grads={"d_x": torch.zeros(1)})


def test_conv_rejects_wrong_shapes():
    Dc, K = 24, 4
    x = torch.zeros(Bt, T, Dc)
    w = torch.zeros(Dc, K)
    for kw, name in ((dict(bias=torch.zeros(Dc + 1)), "bias"),
                     (dict(state=torch.zeros(Bt, Dc, K)), "state"),
                     (dict(y=torch.zeros(Bt, T - 1, Dc)), "y"),
                     (dict(state_out=torch.zeros(Bt + 1, Dc, K - 1)), "state_out")):
        with pytest.raises(ValueError, match=f"{name} must have shape"):
            ssd.ssd_conv1d(x, w, **kw)
    st = torch.zeros(Bt, Dc, K - 1)
    with pytest.raises(ValueError, match="state must have shape"):
        ssd.ssd_conv1d_step(torch.zeros(Bt, Dc, K - 2), torch.zeros(Bt, Dc), w)
    with pytest.raises(ValueError, match="weight must have shape"):
        ssd.ssd_conv1d_step(st, torch.zeros(Bt, Dc), torch.zeros(Dc + 1, K))
    with pytest.raises(ValueError, match="y_t must have shape"):
        ssd.ssd_conv1d_step(st, torch.zeros(Bt, Dc), w, y_t=torch.zeros(Bt, Dc + 4))
