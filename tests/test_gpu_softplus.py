"""The device's Delta activation against its definition: softplus(z) =
max(z, 0) + log1p(exp(-|z|)) in float64 ([SSD] Implementation: einsum
shaping names the softplus).  Delta is read back exactly through ssd_step:
with a zero state, x = 1 in head channel 0, B = C = the first unit vector and
no skip term, one step gives y = C . (Delta x B) = Delta (products with 1).
The clip range is opened so that the raw softplus shows.
"""
import numpy as np
import pytest
import torch

from gpu_util import announce, need_gpu

pytestmark = pytest.mark.gpu


def test_delta_softplus_matches_its_definition():
    need_gpu()
    import state_space_model_amd as ssd
    z = np.concatenate([np.linspace(-40.0, 40.0, 8001), [0.0, 1e-6, -1e-6, 1e-3, -1e-3, 16.0,
                                                          17.0, 18.0, -16.0, -17.0, -18.0]])
    z = z.astype(np.float32)
    Bt, H, P, N = len(z), 1, 16, 16
    dev = "cuda"
    state = torch.zeros(Bt, H, P, N, device=dev)
    x = torch.zeros(Bt, H, P, device=dev)
    x[:, 0, 0] = 1.0
    Bv = torch.zeros(Bt, 1, N, device=dev)
    Bv[:, 0, 0] = 1.0
    dt = torch.from_numpy(z).reshape(Bt, 1).to(dev)
    announce("device softplus through ssd_step")
    y = ssd.ssd_step(state, x, dt, -torch.ones(H, device=dev), Bv, Bv.clone(), None,
                     dt_limit=(0.0, 1e30))
    torch.cuda.synchronize()
    got = y[:, 0, 0].double().cpu().numpy()
    zd = z.astype(np.float64)
    ref = np.maximum(zd, 0.0) + np.log1p(np.exp(-np.abs(zd)))
    rel = np.abs(got - ref) / ref
    # the exponent -|z| log2(e) is rounded to float32 before the hardware exp2:
    # a relative error of about |z| 2^-24 on exp(-|z|); a few ulps otherwise
    bound = 4.0 * 2.0 ** -24 * (1.0 + np.abs(zd)) + 4.0 * 2.0 ** -24
    worst = int(np.argmax(rel / bound))
    print(f"softplus: max rel err {rel.max():.3e}; worst against its bound at z={z[worst]} "
          f"({rel[worst]:.3e} <= {bound[worst]:.3e})")
    assert np.all(rel <= bound), (z[worst], rel[worst], bound[worst])
