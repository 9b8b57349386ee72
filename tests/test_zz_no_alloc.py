"""ssd_chunk_scan_noalloc: the allocation-free entry point (its workspace is
the library's static per-device scratch) against ssd_chunk_scan, through the
C ABI, on two calls in a row, the second smaller than the first: the results
must be bitwise those of ssd_chunk_scan with a caller workspace (the same
kernels on the same inputs), and the second call must not see the first
call's leftovers.  A problem beyond the scratch is refused before launch.
"""
import pytest
import torch

from gpu_util import TOL, announce, need_gpu, oracle_scan, state_err, to_dev, y_err
from ssd_inputs import make_inputs, make_tiny

pytestmark = pytest.mark.gpu


def scan_both(ssd, w):
    inp = make_inputs(w, with_initial_state=True)
    d = to_dev(inp)
    kw = dict(chunk=w.chunk, dt_bias=d["dt_bias"], dt_limit=(w.dt_min, w.dt_max),
              initial_state=d["h0"])
    y_ref, f_ref = ssd.ssd_chunk_scan(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], **kw)
    y = torch.empty_like(d["x"])
    fin = torch.empty_like(f_ref)
    y_na, f_na = ssd.ssd_chunk_scan_noalloc(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                            y=y, final_state=fin, **kw)
    torch.cuda.synchronize()
    return inp, (y_ref, f_ref), (y_na, f_na)


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_noalloc_matches_scan_on_two_calls(io):
    need_gpu()
    import state_space_model_amd as ssd
    # the 2.7B-shaped 4096-token layer (bf16: 67 MB of scratch), then a smaller, ragged one
    first = make_tiny(1, 4096, 80 if io == "bf16" else 24, 64, 128, 1, 256, io, seed=4600)
    second = make_tiny(2, 777, 8, 64, 128, 2, 128, io, seed=4601)
    for k, w in enumerate((first, second)):
        announce(f"noalloc call {k} {io} {w.name}")
        inp, (y_ref, f_ref), (y_na, f_na) = scan_both(ssd, w)
        assert torch.equal(y_na, y_ref) and torch.equal(f_na, f_ref), (k, io)
        if k == 1:
            yo, fo = oracle_scan(inp, w)
            assert y_err(y_na, yo) <= TOL[io] and state_err(f_na, fo) <= TOL[io]


def test_noalloc_refuses_a_problem_beyond_its_scratch():
    need_gpu()
    import state_space_model_amd as ssd
    announce("noalloc refuses 16 x 16384 x 64 heads")
    x = torch.zeros(16, 16384, 64, 64, device="cuda", dtype=torch.bfloat16)
    B = torch.zeros(16, 16384, 1, 128, device="cuda", dtype=torch.bfloat16)
    dt = torch.zeros(16, 16384, 64, device="cuda")
    A = -torch.ones(64, device="cuda")
    with pytest.raises(ssd.SSDError, match="WORKSPACE"):
        ssd.ssd_chunk_scan_noalloc(x, dt, A, B, B, chunk=256)
