"""Pins of the generic-scan oracle (oracle/generic_scan.py).

Sources of truth, none of them the generic oracle itself:
  * numpy's cumsum for the "add" body, the body of the scan tests on the
    rlx-autodiff source page "src/decompose_backward.rs" (Add of the carry and
    x_t): its forward is a running sum and its VJP a reverse running sum;
  * the quaternion oracle (oracle/quat_oracle.c, pinned on its own in
    test_oracle_pins.py), which uses conjugates where the generic oracle uses
    transposed 4x4 Jacobians;
  * central finite differences of sum_t <u[t], ys[t]> on tiny inputs.

A slip in the generic oracle (a Jacobian not transposed, L and R swapped, the
upstream cotangent added one step late, a dropped init term) fails one of them.
"""
import numpy as np
import pytest

import oracle


def _inputs(body, b, s, m, seed, unit=False):
    rng = np.random.default_rng(seed)
    w = oracle.SCAN_BODIES[body]
    xs = rng.standard_normal((b, s, m, w))
    init = rng.standard_normal((b, m, w))
    if unit and body == "quat":
        xs /= np.linalg.norm(xs, axis=-1, keepdims=True)
        init /= np.linalg.norm(init, axis=-1, keepdims=True)
    up = rng.standard_normal((b, s, m, w))
    return xs, init, up


def test_add_body_forward_is_a_running_sum():
    xs, init, _ = _inputs("add", 3, 50, 7, 1)
    ys = oracle.scan_fwd("add", xs, init)
    np.testing.assert_allclose(ys, init[:, None] + np.cumsum(xs, axis=1), rtol=0, atol=1e-12)


def test_add_body_vjp_is_a_reverse_running_sum():
    xs, init, up = _inputs("add", 2, 40, 5, 2)
    d_xs, d_init = oracle.scan_bwd("add", xs, init, up)
    rev = np.cumsum(up[:, ::-1], axis=1)[:, ::-1]
    np.testing.assert_allclose(d_xs, rev, rtol=0, atol=1e-12)
    np.testing.assert_allclose(d_init, up.sum(axis=1), rtol=0, atol=1e-12)


@pytest.mark.parametrize("unit", [True, False])
def test_quat_body_matches_the_quaternion_oracle(unit):
    xs, init, up = _inputs("quat", 2, 64, 6, 3, unit=unit)
    ys = oracle.scan_fwd("quat", xs, init)
    np.testing.assert_allclose(ys, oracle.fwd(xs, init), rtol=1e-12, atol=1e-12)
    d_xs, d_init = oracle.scan_bwd("quat", xs, init, up)
    ref_dq, ref_di = oracle.bwd(xs, init, up)
    scale = np.abs(ref_dq).max()
    np.testing.assert_allclose(d_xs, ref_dq, rtol=0, atol=1e-12 * scale)
    np.testing.assert_allclose(d_init, ref_di, rtol=0, atol=1e-12 * scale)


@pytest.mark.parametrize("body", ["add", "quat"])
def test_vjp_matches_finite_differences(body):
    xs, init, up = _inputs(body, 1, 5, 2, 4)
    d_xs, d_init = oracle.scan_bwd(body, xs, init, up)

    def loss(x, i):
        return float(np.sum(up * oracle.scan_fwd(body, x, i)))

    h = 1e-6
    num_xs = np.zeros_like(xs)
    for idx in np.ndindex(xs.shape):
        p, q = xs.copy(), xs.copy()
        p[idx] += h
        q[idx] -= h
        num_xs[idx] = (loss(p, init) - loss(q, init)) / (2 * h)
    num_init = np.zeros_like(init)
    for idx in np.ndindex(init.shape):
        p, q = init.copy(), init.copy()
        p[idx] += h
        q[idx] -= h
        num_init[idx] = (loss(xs, p) - loss(xs, q)) / (2 * h)
    np.testing.assert_allclose(d_xs, num_xs, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(d_init, num_init, rtol=1e-6, atol=1e-7)


def test_single_step_and_shapes():
    xs, init, up = _inputs("quat", 1, 1, 3, 5)
    d_xs, d_init = oracle.scan_bwd("quat", xs, init, up)
    # s = 1: d_x = g (x) conj(init), d_init = conj(x) (x) g, with g = u[0].
    conj = np.array([1.0, -1.0, -1.0, -1.0])
    for k in range(3):
        np.testing.assert_allclose(d_xs[0, 0, k], oracle.qmul(up[0, 0, k], init[0, k] * conj), atol=1e-14)
        np.testing.assert_allclose(d_init[0, k], oracle.qmul(xs[0, 0, k] * conj, up[0, 0, k]), atol=1e-14)
    with pytest.raises(ValueError):
        oracle.scan_fwd("quat", np.zeros((1, 2, 3, 1)), np.zeros((1, 3, 1)))
    with pytest.raises(ValueError):
        oracle.scan_fwd("mul", np.zeros((1, 2, 3, 1)), np.zeros((1, 3, 1)))
