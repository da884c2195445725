"""The generic scan as an autograd node (autograd.scan / ScanFunction) against
the float64 oracle (oracle/generic_scan.py), through the C ABI (needs an
MI355X).  Loss = sum of W * ys for a fixed random W, so the upstream
cotangent of every saved carry is W.

Tolerances as in test_gpu_scan.py: 2^-23 |ref| + 1e-9 max|ref| per element for
the snapshot VJP (carries recomputed in float64), plus 2^-21 of the element's
vector norm for the trajectory VJP (it reads float32-rounded carries); max
abs <= 1e-4 for both.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd.autograd import scan

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def inputs(body, b, s, m, seed):
    rng = np.random.default_rng(seed)
    w = oracle.SCAN_BODIES[body]
    xs = rng.standard_normal((b, s, m, w)).astype(np.float32)
    init = rng.standard_normal((b, m, w)).astype(np.float32)
    if body == "quat":
        xs /= np.linalg.norm(xs, axis=-1, keepdims=True)
        init /= np.linalg.norm(init, axis=-1, keepdims=True)
    wts = rng.standard_normal((b, s, m, w)).astype(np.float32)
    return xs, init, wts


def check(name, got, ref, rel_norm):
    err = np.abs(got - ref)
    worst = float(err.max())
    assert worst <= 1e-4, f"{name}: max abs err {worst:.3e}"
    norm = np.linalg.norm(ref, axis=-1, keepdims=True)
    bad = err > 2.0 ** -23 * np.abs(ref) + rel_norm * norm + 1e-9 * float(np.abs(ref).max())
    assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond the bound; worst {worst:.3e}"


@pytest.mark.parametrize("body", ["add", "quat"])
@pytest.mark.parametrize("k", [0, 1, 4])
def test_gradients_match_oracle(body, k):
    b, s, m = 2, 129, 40
    print(f"[scan autograd {body} k={k}]", flush=True)
    xs, init, wts = inputs(body, b, s, m, seed=31 + k)
    X = torch.from_numpy(xs).to(DEV).requires_grad_()
    I = torch.from_numpy(init).to(DEV).requires_grad_()
    W = torch.from_numpy(wts).to(DEV)
    ys = scan(body, X, I, num_checkpoints=k)
    (ys * W).sum().backward()
    torch.cuda.synchronize()
    r_dx, r_di = oracle.scan_bwd(body, xs, init, wts)
    rel_norm = 2.0 ** -21 if k == 0 else 0.0
    check("xs.grad", X.grad.cpu().numpy().astype(np.float64), r_dx, rel_norm)
    check("init.grad", I.grad.cpu().numpy().astype(np.float64), r_di, rel_norm)
    check("ys", ys.detach().cpu().numpy().astype(np.float64), oracle.scan_fwd(body, xs, init), 0.0)


def test_second_backward_through_a_checkpointed_graph():
    """The snapshot VJP overwrites the snapshots the forward took; a second
    backward (retain_graph) recomputes them from init and gives the same
    gradients bit for bit."""
    xs, init, wts = inputs("quat", 1, 300, 64, seed=5)
    X = torch.from_numpy(xs).to(DEV).requires_grad_()
    I = torch.from_numpy(init).to(DEV).requires_grad_()
    W = torch.from_numpy(wts).to(DEV)
    loss = (scan("quat", X, I, num_checkpoints=3) * W).sum()
    loss.backward(retain_graph=True)
    g1 = (X.grad.clone(), I.grad.clone())
    X.grad = None
    I.grad = None
    loss.backward()
    torch.cuda.synchronize()
    assert torch.equal(X.grad, g1[0]) and torch.equal(I.grad, g1[1])


def test_only_tracked_inputs_get_gradients_and_untracked_runs_forward_only():
    xs, init, wts = inputs("quat", 1, 50, 16, seed=6)
    X = torch.from_numpy(xs).to(DEV).requires_grad_()
    I = torch.from_numpy(init).to(DEV)
    ys = scan("quat", X, I, num_checkpoints=2)
    (ys * torch.from_numpy(wts).to(DEV)).sum().backward()
    assert X.grad is not None and I.grad is None
    with torch.no_grad():
        y2 = scan("quat", X, I)
    assert y2.grad_fn is None and torch.equal(y2, ys.detach())
