"""quat_cumprod_bwd_noalloc (the backward whose workspace is the library's
fixed device array, for callers that cannot allocate) against
quat_cumprod_bwd on the same inputs, through the C ABI.  Same kernels and the
same association of every sum, so the outputs must agree bit for bit; both
are also held to the oracle's float32 bar.  Two calls in a row, the second on
a smaller input, and a call without saved boundary state (which puts the
re-derived state in the array too)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.inputs import make_config, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def to_dev(arr):
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def both(inp, use_ckpt):
    q, init, d = to_dev(inp.q), to_dev(inp.init), to_dev(inp.d_cum)
    ck = capi.new_ckpt(q) if use_ckpt else None
    capi.quat_cumprod_fwd(q, init, ckpt=ck)
    ref_dq, ref_di = capi.quat_cumprod_bwd(q, init, d, ck)
    d_q, d_init = torch.empty_like(q), torch.empty_like(init)
    status = torch.full((1,), -1, dtype=torch.int32, device=DEV)
    capi.quat_cumprod_bwd_noalloc(q, init, d, d_q, d_init, ckpt=ck, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert capi.default_workspace.status(q.device) == 0
    return (d_q, d_init), (ref_dq, ref_di)


@pytest.mark.parametrize("use_ckpt", [True, False], ids=["saved-state", "leaves-only"])
def test_noalloc_matches_allocating_backward_twice(use_ckpt):
    first = make_config("headline")
    second = make_inputs(2, 3000, 4, 8, "unit", "f32", seed=77)
    for inp in (first, second):
        print(f"[noalloc b={inp.b} s={inp.s} h={inp.h} j={inp.j} ckpt={use_ckpt}]", flush=True)
        (d_q, d_init), (r_dq, r_di) = both(inp, use_ckpt)
        assert torch.equal(d_q, r_dq) and torch.equal(d_init, r_di)
        o_dq, o_di = oracle.bwd(inp.q64, inp.init64, inp.d_cum64)
        for got, ref in ((d_q, o_dq), (d_init, o_di)):
            err = np.abs(got.cpu().numpy().astype(np.float64) - ref)
            assert float(err.max()) <= 1e-4
            assert not (err > 2.0 ** -23 * np.abs(ref) + 1e-9 * np.abs(ref).max()).any()


def test_noalloc_reports_a_zero_step_in_status():
    inp = make_inputs(1, 500, 2, 4, "unit", "f32", seed=78)
    inp.q[0, 200, 1, 1] = 0.0
    q, init, d = to_dev(inp.q), to_dev(inp.init), to_dev(inp.d_cum)
    d_q, d_init = torch.empty_like(q), torch.empty_like(init)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    capi.quat_cumprod_bwd_noalloc(q, init, d, d_q, d_init, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 2                      # QC_STATUS_ZERO
    good = make_inputs(1, 500, 2, 4, "unit", "f32", seed=79)
    q2, i2, dd2 = to_dev(good.q), to_dev(good.init), to_dev(good.d_cum)
    capi.quat_cumprod_bwd_noalloc(q2, i2, dd2, d_q, d_init, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0                      # the array's status word was cleared


def test_noalloc_rejects_shapes_beyond_its_array():
    lib = capi.load()
    p = ctypes.c_void_p(1 << 30)
    rc = lib.quat_cumprod_bwd_noalloc(p, ctypes.c_void_p(1 << 31), ctypes.c_void_p(1 << 32), None, 0,
                                      ctypes.c_void_p(1 << 33), None, 64, 4096, 32, 32, 0, None, None)
    assert rc == -6
