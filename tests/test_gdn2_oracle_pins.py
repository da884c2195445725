"""Pins of the float64 Gated DeltaNet-2 oracle (oracle/gdn2.py) to things
other than itself (no GPU):

* a step worked by hand (tests/golden/gdn2_one_step.txt);
* closed forms of special cases of the recurrence of the burn_gdn source page
  "src/chunk_wy/custom_backward.rs" (forward_impl): decay only (zero keys),
  linear attention (no erase, no decay), and the delta rule's defining
  property (erase 1, no decay, unit key: the new state reads the written value
  back exactly);
* the VJP against torch.autograd of the direct graph in float64 (the page
  checks its custom backward against the autodiff of that graph), and central
  finite differences for all seven cotangents.
"""
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "gdn2_one_step.txt")


def rand_inputs(B, H, T, L, D, seed, decay=(-1.2, -0.2)):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, T, L))
    k = rng.standard_normal((B, H, T, L)) / np.sqrt(L)
    v = rng.standard_normal((B, H, T, D))
    b = rng.uniform(0.0, 1.0, (B, H, T, L))
    w = rng.uniform(0.0, 1.0, (B, H, T, D))
    g = rng.uniform(decay[0], decay[1], (B, H, T, L))
    s0 = rng.standard_normal((B, H, L, D))
    return q, k, v, b, w, g, s0


def test_step_worked_by_hand():
    vals = {}
    for ln in open(GOLDEN):
        if "=" in ln and not ln.startswith("#"):
            key, val = ln.split("=")
            vals[key.strip()] = [float(x) for x in val.split()]
    s0 = np.array([[1.0], [2.0]])[None, None]
    args = (np.array([1.0, 0.0]), np.array([0.6, 0.8]), np.array([3.0]), np.array([0.5, 0.5]), np.array([2.0]),
            np.array([0.0, np.log(0.5)]))
    q, k, v, b, w, g = (x[None, None, None] for x in args)
    ctx, state = oracle.gdn2_fwd(q, k, v, b, w, g, s0)
    np.testing.assert_allclose(state.ravel(), vals["state"], rtol=1e-14)
    np.testing.assert_allclose(ctx.ravel(), vals["context"], rtol=1e-14)


def test_decay_only_closed_form():
    q, k, v, b, w, g, s0 = rand_inputs(2, 2, 7, 5, 3, seed=1)
    k[:] = 0.0
    ctx, state = oracle.gdn2_fwd(q, k, v, b, w, g, s0)
    cum = np.cumsum(g, axis=2)                                      # [B, H, T, L]
    S = np.exp(cum)[..., None] * s0[:, :, None]                     # S_t = diag(exp(sum g)) S0
    want_ctx = np.einsum("bhtld,bhtl->bhtd", S, q) / np.sqrt(5)
    np.testing.assert_allclose(ctx, want_ctx, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(state, S[:, :, -1], rtol=1e-12, atol=1e-13)


def test_linear_attention_closed_form():
    q, k, v, b, w, g, s0 = rand_inputs(1, 3, 9, 4, 6, seed=2)
    b[:] = 0.0
    g[:] = 0.0
    ctx, state = oracle.gdn2_fwd(q, k, v, b, w, g, s0)
    outer = k[..., :, None] * (w * v)[..., None, :]                 # [B, H, T, L, D]
    S = s0[:, :, None] + np.cumsum(outer, axis=2)
    np.testing.assert_allclose(ctx, np.einsum("bhtld,bhtl->bhtd", S, q) / 2.0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(state, S[:, :, -1], rtol=1e-12, atol=1e-12)


def test_delta_rule_reads_back_the_written_value():
    """erase = 1, no decay, unit key: S_t^T k_t = w_t * v_t after every step."""
    q, k, v, b, w, g, s0 = rand_inputs(1, 2, 6, 8, 5, seed=3)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    b[:] = 1.0
    g[:] = 0.0
    _, states = oracle.gdn2_states(q, k, v, b, w, g, s0)
    for t in range(6):
        read = np.einsum("bhld,bhl->bhd", states[:, :, t + 1], k[:, :, t])
        np.testing.assert_allclose(read, w[:, :, t] * v[:, :, t], rtol=1e-12, atol=1e-12)


def torch_direct_graph(q, k, v, b, w, g, s0):
    """The page's direct graph, step by step, in torch float64 (matrix form)."""
    L = q.shape[-1]
    S = s0
    outs = []
    for t in range(q.shape[2]):
        decayed = torch.exp(g[:, :, t]).unsqueeze(-1) * S
        erased = torch.matmul((b[:, :, t] * k[:, :, t]).unsqueeze(-2), decayed).squeeze(-2)
        update = w[:, :, t] * v[:, :, t] - erased
        S = decayed + torch.matmul(k[:, :, t].unsqueeze(-1), update.unsqueeze(-2))
        outs.append(torch.matmul(q[:, :, t].unsqueeze(-2), S).squeeze(-2) / L ** 0.5)
    return torch.stack(outs, dim=2), S


@pytest.mark.parametrize("geom", [(1, 2, 5, 3, 4), (1, 2, 9, 5, 37), (2, 3, 12, 16, 8)])
@pytest.mark.parametrize("with_state_grad", [False, True])
def test_vjp_matches_torch_autograd(geom, with_state_grad):
    B, H, T, L, D = geom
    arrays = rand_inputs(B, H, T, L, D, seed=sum(geom))
    rng = np.random.default_rng(7)
    d_ctx = rng.standard_normal((B, H, T, D))
    d_state = rng.standard_normal((B, H, L, D)) if with_state_grad else None
    ts = [torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in arrays]
    ctx, state = torch_direct_graph(*ts)
    loss = (ctx * torch.from_numpy(d_ctx)).sum()
    if with_state_grad:
        loss = loss + (state * torch.from_numpy(d_state)).sum()
    loss.backward()
    got = oracle.gdn2_bwd(*arrays, d_ctx, d_state)
    want_ctx, want_state = oracle.gdn2_fwd(*arrays)
    np.testing.assert_allclose(ctx.detach().numpy(), want_ctx, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(state.detach().numpy(), want_state, rtol=1e-12, atol=1e-12)
    for name, mine, t in zip(oracle.gdn2.NAMES, got, ts):
        np.testing.assert_allclose(mine, t.grad.numpy(), rtol=1e-10, atol=1e-11, err_msg=name)


def test_vjp_matches_central_differences():
    B, H, T, L, D = 1, 2, 5, 3, 4
    arrays = list(rand_inputs(B, H, T, L, D, seed=11))
    rng = np.random.default_rng(12)
    d_ctx = rng.standard_normal((B, H, T, D))
    d_state = rng.standard_normal((B, H, L, D))

    def loss(arrs):
        c, s = oracle.gdn2_fwd(*arrs)
        return float(np.sum(c * d_ctx) + np.sum(s * d_state))

    grads = oracle.gdn2_bwd(*arrays, d_ctx, d_state)
    h = 1e-6
    for i, name in enumerate(oracle.gdn2.NAMES):
        fd = np.zeros_like(arrays[i])
        for idx in np.ndindex(arrays[i].shape):
            plus = [a.copy() for a in arrays]
            minus = [a.copy() for a in arrays]
            plus[i][idx] += h
            minus[i][idx] -= h
            fd[idx] = (loss(plus) - loss(minus)) / (2 * h)
        np.testing.assert_allclose(grads[i], fd, rtol=1e-6, atol=1e-7, err_msg=name)
