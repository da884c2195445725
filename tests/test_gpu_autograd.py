"""The torch.autograd node (quaternion_cumprod_autodiff_amd.autograd) against
the float64 oracle (needs an MI355X).

Gradients of scalar losses L = sum(w * cum) (+ sum(w2 * final_carry)) are
compared with oracle.bwd at d_cum = dL/dcum, to the same tolerances as the
C-ABI parity tests.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.autograd import QuatCumprodFunction, quat_cumprod, quat_cumprod_with_final
from quaternion_cumprod_autodiff_amd.inputs import make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def dev(arr, dtype="f32", grad=False):
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)
    return t.requires_grad_(grad)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def close(got, ref, dtype="f32"):
    err = float(np.abs(got - ref).max())
    scale = float(np.abs(ref).max())
    if dtype == "f32":
        assert err <= 1e-4, (err, scale)
    else:
        assert err / scale <= 2e-2, (err, scale)


@pytest.mark.parametrize("saved", ["boundary", "final", "none"])
def test_gradients_match_oracle(saved):
    inp = make_inputs(2, 700, 4, 8, "unit", "f32", seed=21)
    w = np.random.default_rng(22).standard_normal(inp.q.shape).astype(np.float32)
    q, init = dev(inp.q, grad=True), dev(inp.init, grad=True)
    cum = quat_cumprod(q, init, saved=saved)
    (cum * dev(w)).sum().backward()
    r_cum = oracle.fwd(inp.q64, inp.init64)
    r_dq, r_di = oracle.bwd(inp.q64, inp.init64, w.astype(np.float64))
    close(f64(cum), r_cum)
    close(f64(q.grad), r_dq)
    close(f64(init.grad), r_di)


@pytest.mark.parametrize("saved", ["boundary", "final"])
def test_final_carry_gradient_is_folded(saved):
    """The final carry is a slice of cum: its gradient lands in d_cum[:, -1]."""
    inp = make_inputs(3, 300, 2, 4, "unit", "f32", seed=23)
    rng = np.random.default_rng(24)
    w = rng.standard_normal(inp.q.shape).astype(np.float32)
    w2 = rng.standard_normal(inp.init.shape).astype(np.float32)
    q, init = dev(inp.q, grad=True), dev(inp.init, grad=True)
    cum, final = quat_cumprod_with_final(q, init, saved=saved)
    ((cum * dev(w)).sum() + (final * dev(w2)).sum()).backward()
    d = w.astype(np.float64)
    d[:, -1] += w2
    r_dq, r_di = oracle.bwd(inp.q64, inp.init64, d)
    close(f64(q.grad), r_dq)
    close(f64(init.grad), r_di)


@pytest.mark.parametrize("which", ["q", "init"])
def test_only_tracked_inputs_get_gradients(which):
    inp = make_inputs(1, 200, 2, 8, "unit", "f32", seed=25)
    w = np.random.default_rng(26).standard_normal(inp.q.shape).astype(np.float32)
    q, init = dev(inp.q, grad=which == "q"), dev(inp.init, grad=which == "init")
    (quat_cumprod(q, init) * dev(w)).sum().backward()
    r_dq, r_di = oracle.bwd(inp.q64, inp.init64, w.astype(np.float64))
    if which == "q":
        assert init.grad is None
        close(f64(q.grad), r_dq)
    else:
        assert q.grad is None
        close(f64(init.grad), r_di)


def test_untracked_call_runs_forward_only():
    inp = make_inputs(2, 150, 2, 2, "unit", "f32", seed=27)
    q, init = dev(inp.q, grad=True), dev(inp.init, grad=True)
    with torch.no_grad():
        cum = quat_cumprod(q, init)
    assert cum.grad_fn is None
    assert torch.equal(cum, capi.quat_cumprod_fwd(q.detach(), init.detach()))


def test_segments_chained_through_autograd():
    """Feeding one segment's final carry as the next segment's init: autograd
    routes the second segment's d_init into the first's final carry."""
    inp = make_inputs(2, 500, 2, 4, "unit", "f32", seed=28)
    w = np.random.default_rng(29).standard_normal(inp.q.shape).astype(np.float32)
    q, init = dev(inp.q, grad=True), dev(inp.init, grad=True)
    head, carry = quat_cumprod_with_final(q[:, :200], init)
    tail = quat_cumprod(q[:, 200:], carry)
    (torch.cat([head, tail], 1) * dev(w)).sum().backward()
    r_dq, r_di = oracle.bwd(inp.q64, inp.init64, w.astype(np.float64))
    np.testing.assert_allclose(f64(q.grad), r_dq, rtol=0, atol=1e-4)
    np.testing.assert_allclose(f64(init.grad), r_di, rtol=0, atol=1e-4)


def test_bf16_gradients():
    """bf16 storage: the loss weights are the recipe's bf16 d_cum, so the
    cotangent reaching the node is exactly d_cum."""
    inp = make_inputs(2, 400, 4, 4, "drift", "bf16", seed=30)
    q, init = dev(inp.q, "bf16", grad=True), dev(inp.init, "bf16", grad=True)
    wd = dev(inp.d_cum, "bf16")
    for saved in ("boundary", "final"):
        q.grad = init.grad = None
        cum = QuatCumprodFunction.apply(q, init, saved, "deferred")
        (cum.float() * wd.float()).sum().backward()
        r_dq, r_di = oracle.bwd(inp.q64, inp.init64, inp.d_cum64)
        close(f64(q.grad), r_dq, "bf16")
        close(f64(init.grad), r_di, "bf16")


@pytest.mark.parametrize("saved", ["boundary", "final", "none"])
def test_zero_step_raises_from_backward(saved):
    """A zero step makes the backward's prefix products zero: with
    status_check="sync" the backward itself raises, instead of handing
    non-finite gradients to the optimiser."""
    inp = make_inputs(2, 300, 2, 4, "unit", "f32", seed=31)
    inp.q[1, 120, 0, 3] = 0.0
    q, init = dev(inp.q, grad=True), dev(inp.init, grad=True)
    cum = quat_cumprod(q, init, saved=saved, status_check="sync")
    with pytest.raises(capi.QuatCumprodStatusError) as ei:
        cum.sum().backward()
    assert ei.value.bits == 2
    capi.check_status()                       # reported once, then cleared


def test_zero_step_raises_at_next_call_when_deferred():
    """Deferred mode (the default): the status copy is queued after the
    backward, and the next call through the node (or capi.check_status())
    raises."""
    inp = make_inputs(1, 200, 2, 2, "unit", "f32", seed=32)
    inp.q[0, 50, 1, 1] = 0.0
    q, init = dev(inp.q, grad=True), dev(inp.init, grad=True)
    quat_cumprod(q, init).sum().backward()
    torch.cuda.synchronize()
    with pytest.raises(capi.QuatCumprodStatusError):
        quat_cumprod(q.detach(), init.detach())
    capi.check_status()
    good = make_inputs(1, 200, 2, 2, "unit", "f32", seed=33)
    q2, i2 = dev(good.q, grad=True), dev(good.init, grad=True)
    quat_cumprod(q2, i2).sum().backward()
    capi.check_status()


def test_two_streams_share_the_default_workspace():
    """Two streams run leaves-only forward + backward through the autograd
    node concurrently on the default workspace: it keeps a buffer per stream,
    so neither the carry slots nor the re-derived boundary state are shared,
    and both match the oracle."""
    shapes = [(4, 2048, 16, 16, "unit", 41), (2, 6000, 4, 8, "drift", 42)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for (b, s, h, j, recipe, seed), st in zip(shapes, streams):
        inp = make_inputs(b, s, h, j, recipe, "f32", seed=seed)
        w = np.random.default_rng(seed + 100).standard_normal(inp.q.shape).astype(np.float32)
        runs.append(dict(inp=inp, w=w, st=st, grads=[]))
    torch.cuda.synchronize()
    for it in range(3):
        for rn in runs:
            with torch.cuda.stream(rn["st"]):
                q, init = dev(rn["inp"].q, grad=True), dev(rn["inp"].init, grad=True)
                (quat_cumprod(q, init, saved="none") * dev(rn["w"])).sum().backward()
                rn["grads"].append((q.grad, init.grad))
    torch.cuda.synchronize()
    capi.check_status()
    for rn in runs:
        inp = rn["inp"]
        r_dq, r_di = oracle.bwd(inp.q64, inp.init64, rn["w"].astype(np.float64))
        print(f"[default workspace, stream of b={inp.b} s={inp.s}]", flush=True)
        for gq, gi in rn["grads"]:
            close(f64(gq), r_dq)
            close(f64(gi), r_di)
