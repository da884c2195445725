"""Pins of the float64 oracle against facts that do not come from the oracle.

Sources:
  * burn-mamba source page "burn_mamba/mamba3/quat_scan/backward.rs", module
    doc "Gradient math" (scan definition, per-factor VJPs, reverse recurrence,
    unit-quaternion closed form);
  * Hamilton's relations (tests/golden/hamilton_basis.txt);
  * independent re-derivations: complex numbers (numpy/torch cumprod), the
    2x2 complex-matrix representation of the quaternions with torch autograd,
    finite differences, the forward-mode (tangent) recurrence.

A plausible slip in the oracle (a flipped sign in the product, swapped operand
order, an off-by-one step index in the backward, a dropped d_init term) fails
at least one of these.
"""
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
UNITS = {"1": (1.0, 0.0, 0.0, 0.0), "i": (0.0, 1.0, 0.0, 0.0),
         "j": (0.0, 0.0, 1.0, 0.0), "k": (0.0, 0.0, 0.0, 1.0)}


def _unit(tok: str) -> np.ndarray:
    sign = -1.0 if tok.startswith("-") else 1.0
    return sign * np.array(UNITS[tok.lstrip("-")])


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


def _unit_quats(rng, shape):
    v = rng.standard_normal(tuple(shape) + (4,))
    return v / np.linalg.norm(v, axis=-1, keepdims=True)


# ---------------------------------------------------------------- the product

def test_basis_table():
    rows = _rows("hamilton_basis.txt")
    assert len(rows) == 16
    for a, b, p in rows:
        np.testing.assert_array_equal(oracle.qmul(_unit(a), _unit(b)), _unit(p))


def test_norm_multiplicative_associative_conjugate():
    rng = np.random.default_rng(1)
    for _ in range(50):
        a, b, c = rng.standard_normal((3, 4)) * rng.uniform(0.1, 3.0, size=(3, 1))
        ab = oracle.qmul(a, b)
        assert abs(np.linalg.norm(ab) - np.linalg.norm(a) * np.linalg.norm(b)) < 1e-12 * (1 + np.linalg.norm(ab))
        np.testing.assert_allclose(oracle.qmul(ab, c), oracle.qmul(a, oracle.qmul(b, c)), rtol=0, atol=1e-12)
        conj = np.array([1.0, -1.0, -1.0, -1.0])
        np.testing.assert_allclose(ab * conj, oracle.qmul(b * conj, a * conj), rtol=0, atol=1e-12)


# ---------------------------------------------------------------- the scan

def test_order_example():
    rows = _rows("order_example.txt")
    vals = {(r[0], int(r[1])): np.array([float(x) for x in r[2:]]) for r in rows}
    q = np.stack([vals[("q", 0)], vals[("q", 1)]])[None, :, None, :]
    init = vals[("init", -1)][None, None, :]
    cum = oracle.fwd(q, init)
    np.testing.assert_array_equal(cum[0, 0, 0], vals[("cum", 0)])
    np.testing.assert_array_equal(cum[0, 1, 0], vals[("cum", 1)])


def test_commuting_rotations_closed_form():
    # Rotations about one fixed axis commute; angles add:
    # cum[t] = (cos(((t+1) th + ph)/2), sin(((t+1) th + ph)/2) u).
    rng = np.random.default_rng(2)
    s, m = 300, 5
    u = rng.standard_normal((m, 3))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    th = rng.uniform(-0.3, 0.3, size=m)
    ph = rng.uniform(-3, 3, size=m)
    q = np.zeros((1, s, m, 4))
    q[..., 0] = np.cos(th / 2)
    q[..., 1:] = np.sin(th / 2)[:, None] * u
    init = np.zeros((1, m, 4))
    init[..., 0] = np.cos(ph / 2)
    init[..., 1:] = np.sin(ph / 2)[:, None] * u
    cum = oracle.fwd(q, init)
    ang = (np.arange(1, s + 1)[:, None] * th[None, :] + ph[None, :]) / 2
    want = np.zeros((s, m, 4))
    want[..., 0] = np.cos(ang)
    want[..., 1:] = np.sin(ang)[..., None] * u[None]
    np.testing.assert_allclose(cum[0], want, rtol=0, atol=1e-12)


def _complex_case(rng, b, s, m):
    q = np.zeros((b, s, m, 4))
    q[..., :2] = rng.standard_normal((b, s, m, 2)) * 0.5 + np.array([0.8, 0.0])
    init = np.zeros((b, m, 4))
    init[..., :2] = rng.standard_normal((b, m, 2))
    d = np.zeros((b, s, m, 4))
    d[..., :2] = rng.standard_normal((b, s, m, 2))
    return q, init, d


def test_complex_subspace_forward():
    # y = z = 0 is the complex plane w + x i; the scan is a complex cumprod.
    rng = np.random.default_rng(3)
    q, init, _ = _complex_case(rng, 2, 40, 3)
    cum = oracle.fwd(q, init)
    zq = q[..., 0] + 1j * q[..., 1]
    zi = init[..., 0] + 1j * init[..., 1]
    want = np.cumprod(zq, axis=1) * zi[:, None, :]
    np.testing.assert_allclose(cum[..., 0], want.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(cum[..., 1], want.imag, rtol=0, atol=1e-12)
    assert np.all(cum[..., 2:] == 0.0)


def test_complex_subspace_backward_torch_autograd():
    rng = np.random.default_rng(4)
    q, init, d = _complex_case(rng, 2, 40, 3)
    d_q, d_init = oracle.bwd(q, init, d)
    qw = torch.tensor(q[..., 0], requires_grad=True)
    qx = torch.tensor(q[..., 1], requires_grad=True)
    iw = torch.tensor(init[..., 0], requires_grad=True)
    ix = torch.tensor(init[..., 1], requires_grad=True)
    cum = torch.cumprod(torch.complex(qw, qx), dim=1) * torch.complex(iw, ix)[:, None, :]
    loss = (torch.tensor(d[..., 0]) * cum.real + torch.tensor(d[..., 1]) * cum.imag).sum()
    loss.backward()
    np.testing.assert_allclose(d_q[..., 0], qw.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(d_q[..., 1], qx.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(d_init[..., 0], iw.grad.numpy(), rtol=0, atol=1e-11)
    np.testing.assert_allclose(d_init[..., 1], ix.grad.numpy(), rtol=0, atol=1e-11)
    assert np.abs(d_q[..., 2:]).max() < 1e-12 and np.abs(d_init[..., 2:]).max() < 1e-12


# ------------------------------------------- independent matrix representation

def _su2(v: torch.Tensor) -> torch.Tensor:
    """q = w + x i + y j + z k  ->  [[w + x i, y + z i], [-y + z i, w - x i]]."""
    w, x, y, z = v.unbind(-1)
    a = torch.complex(w, x)
    b = torch.complex(y, z)
    return torch.stack([torch.stack([a, b], -1), torch.stack([-b.conj(), a.conj()], -1)], -2)


def _from_su2(mat: torch.Tensor) -> torch.Tensor:
    return torch.stack([mat[..., 0, 0].real, mat[..., 0, 0].imag,
                        mat[..., 0, 1].real, mat[..., 0, 1].imag], -1)


def _su2_scan(q: torch.Tensor, init: torch.Tensor) -> torch.Tensor:
    c = _su2(init)
    out = []
    for t in range(q.shape[1]):
        c = _su2(q[:, t]) @ c
        out.append(_from_su2(c))
    return torch.stack(out, 1)


def test_su2_representation_is_hamilton():
    # The test's matrix representation must itself satisfy the basis table.
    for a, b, p in _rows("hamilton_basis.txt"):
        got = _from_su2(_su2(torch.tensor(_unit(a))) @ _su2(torch.tensor(_unit(b))))
        np.testing.assert_array_equal(got.numpy(), _unit(p))


@pytest.mark.parametrize("case", ["unit", "scaled", "with_zero_step", "single_step"])
def test_su2_autograd_forward_and_backward(case):
    rng = np.random.default_rng(5)
    b, s, m = 2, (1 if case == "single_step" else 37), 3
    q = _unit_quats(rng, (b, s, m))
    if case == "scaled":
        q *= rng.uniform(0.5, 1.5, size=(b, s, m, 1))
    if case == "with_zero_step":
        q[0, 11, 1] = 0.0
        q[1, 0, 2] = 0.0
    init = _unit_quats(rng, (b, m)) * rng.uniform(0.5, 2.0, size=(b, m, 1))
    d = rng.standard_normal((b, s, m, 4))

    qt = torch.tensor(q, requires_grad=True)
    it = torch.tensor(init, requires_grad=True)
    cum_t = _su2_scan(qt, it)
    (cum_t * torch.tensor(d)).sum().backward()

    cum = oracle.fwd(q, init)
    d_q, d_init = oracle.bwd(q, init, d)
    np.testing.assert_allclose(cum, cum_t.detach().numpy(), rtol=0, atol=1e-12)
    np.testing.assert_allclose(d_q, qt.grad.numpy(), rtol=0, atol=1e-10)
    np.testing.assert_allclose(d_init, it.grad.numpy(), rtol=0, atol=1e-10)


# ------------------------------------------------ statements on the page itself

def test_per_factor_vjp_finite_differences():
    # o = a (x) b, cotangent g: grad_a = g (x) conj(b), grad_b = conj(a) (x) g.
    rng = np.random.default_rng(6)
    conj = np.array([1.0, -1.0, -1.0, -1.0])
    h = 1e-6
    for _ in range(20):
        a, b, g = rng.standard_normal((3, 4))
        fd_a = np.array([(g @ oracle.qmul(a + h * e, b) - g @ oracle.qmul(a - h * e, b)) / (2 * h)
                         for e in np.eye(4)])
        fd_b = np.array([(g @ oracle.qmul(a, b + h * e) - g @ oracle.qmul(a, b - h * e)) / (2 * h)
                         for e in np.eye(4)])
        np.testing.assert_allclose(oracle.qmul(g, b * conj), fd_a, rtol=0, atol=1e-8)
        np.testing.assert_allclose(oracle.qmul(a * conj, g), fd_b, rtol=0, atol=1e-8)


@pytest.mark.parametrize("s", [1, 2, 64, 513])
def test_closed_form_matches_recurrence_for_unit_quaternions(s):
    rng = np.random.default_rng(7)
    q = _unit_quats(rng, (2, s, 5))
    init = _unit_quats(rng, (2, 5))
    d = rng.standard_normal((2, s, 5, 4))
    dq_r, di_r = oracle.bwd(q, init, d)
    for normalise in (False, True):
        dq_c, di_c = oracle.bwd_closed_form(q, init, d, normalise)
        np.testing.assert_allclose(dq_c, dq_r, rtol=0, atol=1e-11)
        np.testing.assert_allclose(di_c, di_r, rtol=0, atol=1e-11)


def test_closed_form_needs_normalisation_off_the_unit_sphere():
    # The page states the closed form for unit quaternions only.  Off the unit
    # sphere G[t] = P_t (x) S[t] / |P_t|^2 is exact; without the division it is not.
    rng = np.random.default_rng(8)
    q = _unit_quats(rng, (1, 48, 4)) * rng.uniform(0.5, 1.5, size=(1, 48, 4, 1))
    init = _unit_quats(rng, (1, 4))
    d = rng.standard_normal((1, 48, 4, 4))
    dq_r, di_r = oracle.bwd(q, init, d)
    dq_n, di_n = oracle.bwd_closed_form(q, init, d, True)
    dq_u, di_u = oracle.bwd_closed_form(q, init, d, False)
    scale = np.abs(dq_r).max()
    np.testing.assert_allclose(dq_n, dq_r, rtol=0, atol=1e-10 * scale)
    np.testing.assert_allclose(di_n, di_r, rtol=0, atol=1e-10 * np.abs(di_r).max())
    np.testing.assert_allclose(di_u, di_r, rtol=0, atol=1e-10 * np.abs(di_r).max())  # d_init = S[0] always
    assert np.abs(dq_u - dq_r).max() > 1e-3 * scale


@pytest.mark.parametrize("s", [1, 3, 8])
def test_central_finite_differences(s):
    rng = np.random.default_rng(9)
    b, m = 2, 3
    q = _unit_quats(rng, (b, s, m)) * rng.uniform(0.7, 1.3, size=(b, s, m, 1))
    init = _unit_quats(rng, (b, m))
    d = rng.standard_normal((b, s, m, 4))
    d_q, d_init = oracle.bwd(q, init, d)
    h = 1e-6

    def loss(qq, ii):
        return float(np.sum(d * oracle.fwd(qq, ii)))

    fd_q = np.zeros_like(q)
    for idx in np.ndindex(*q.shape):
        e = np.zeros_like(q)
        e[idx] = h
        fd_q[idx] = (loss(q + e, init) - loss(q - e, init)) / (2 * h)
    fd_i = np.zeros_like(init)
    for idx in np.ndindex(*init.shape):
        e = np.zeros_like(init)
        e[idx] = h
        fd_i[idx] = (loss(q, init + e) - loss(q, init - e)) / (2 * h)
    np.testing.assert_allclose(d_q, fd_q, rtol=0, atol=1e-8)
    np.testing.assert_allclose(d_init, fd_i, rtol=0, atol=1e-8)


def _su2_np(v):
    a = v[..., 0] + 1j * v[..., 1]
    b = v[..., 2] + 1j * v[..., 3]
    return np.stack([np.stack([a, b], -1), np.stack([-np.conj(b), np.conj(a)], -1)], -2)


def _from_su2_np(mat):
    return np.stack([mat[..., 0, 0].real, mat[..., 0, 0].imag,
                     mat[..., 0, 1].real, mat[..., 0, 1].imag], -1)


def test_dot_product_adjoint_identity():
    # <d_cum, J dq> = <d_q, dq> + <d_init, dinit>, with the tangent propagated by
    # dcum[t] = dq_t (x) cum[t-1] + q_t (x) dcum[t-1]  (product rule), here in the
    # 2x2 complex representation.
    rng = np.random.default_rng(10)
    b, s, m = 3, 200, 4
    q = _unit_quats(rng, (b, s, m)) * rng.uniform(0.9, 1.1, size=(b, s, m, 1))
    init = _unit_quats(rng, (b, m))
    d = rng.standard_normal((b, s, m, 4))
    tq = rng.standard_normal(q.shape)
    ti = rng.standard_normal(init.shape)
    c = _su2_np(init)
    dc = _su2_np(ti)
    lhs = 0.0
    for t in range(s):
        mq = _su2_np(q[:, t])
        dc = _su2_np(tq[:, t]) @ c + mq @ dc
        c = mq @ c
        lhs += np.sum(d[:, t] * _from_su2_np(dc))
    d_q, d_init = oracle.bwd(q, init, d)
    rhs = np.sum(d_q * tq) + np.sum(d_init * ti)
    assert abs(lhs - rhs) <= 1e-10 * (abs(lhs) + 1.0)


def test_unit_norm_preserved():
    rng = np.random.default_rng(11)
    q = _unit_quats(rng, (2, 5000, 3))
    init = _unit_quats(rng, (2, 3))
    cum = oracle.fwd(q, init)
    assert np.abs(np.linalg.norm(cum, axis=-1) - 1.0).max() < 1e-12


def test_segment_chaining():
    # fwd(q, init) = fwd(q[s1:], cum[s1-1]) on the tail; backward: the tail's
    # d_init flows into the head's last cotangent (the final_carry convention).
    rng = np.random.default_rng(12)
    b, s, m, s1 = 2, 90, 3, 37
    q = _unit_quats(rng, (b, s, m))
    init = _unit_quats(rng, (b, m))
    d = rng.standard_normal((b, s, m, 4))
    cum = oracle.fwd(q, init)
    head = oracle.fwd(q[:, :s1], init)
    tail = oracle.fwd(q[:, s1:], head[:, -1])
    np.testing.assert_allclose(np.concatenate([head, tail], 1), cum, rtol=0, atol=1e-12)
    d_q, d_init = oracle.bwd(q, init, d)
    dq_tail, di_tail = oracle.bwd(q[:, s1:], head[:, -1], d[:, s1:])
    d_head = d[:, :s1].copy()
    d_head[:, -1] += di_tail
    dq_head, di_head = oracle.bwd(q[:, :s1], init, d_head)
    np.testing.assert_allclose(np.concatenate([dq_head, dq_tail], 1), d_q, rtol=0, atol=1e-10)
    np.testing.assert_allclose(di_head, d_init, rtol=0, atol=1e-10)


def test_threads_do_not_change_results():
    rng = np.random.default_rng(13)
    q = _unit_quats(rng, (3, 100, 7))
    init = _unit_quats(rng, (3, 7))
    d = rng.standard_normal((3, 100, 7, 4))
    a = oracle.bwd(q, init, d, nthreads=1)
    bb = oracle.bwd(q, init, d, nthreads=4)
    np.testing.assert_array_equal(a[0], bb[0])
    np.testing.assert_array_equal(a[1], bb[1])
    np.testing.assert_array_equal(oracle.fwd(q, init, 1), oracle.fwd(q, init, 4))
