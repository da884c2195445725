"""float64 oracle for a generic scan and its VJP (plain numpy, sequential in t).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this module; the device library and
its Python binding never import it.

The scan follows the Scan / ScanBackward / ScanBackwardXs ops of the
rlx-autodiff source page "src/decompose_backward.rs" (the lowering of
ScanBackward and ScanBackwardXs, and its tests "decompose_scan_backward_length_129"
and "decompose_scan_backward_griewank"): a body maps (carry, x_t) to the next
carry, the forward saves the trajectory of carries, and the backward takes the
initial carry, the trajectory, an upstream cotangent for every saved carry
and the per-step inputs, and returns the cotangents of the initial carry and
of the inputs.  Written out:

    c[-1] = init,   c[t] = f(c[t-1], x[t]),   t = 0 .. s-1,   ys[t] = c[t]
    g[s-1] = u[s-1];   for t = s-1 .. 0:
        d_x[t]  = J_x(c[t-1], x[t])^T g[t]
        g[t-1]  = u[t-1] + J_c(c[t-1], x[t])^T g[t]        (u[-1] = 0)
    d_init = g[-1]

This is the plain definition of the VJP of a scan whose every carry is an
output; checkpointing changes where c[t-1] comes from, never the result, so
the oracle always keeps the whole trajectory.

Bodies (carry width w):
  * "add" (w = 1): f(c, x) = c + x, the body of the page's scan tests
    (a binary Add of the carry and x_t).  Both Jacobians are the identity.
  * "quat" (w = 4): f(c, x) = x (x) c, the quaternion cumulative product of
    the burn-mamba source page "burn_mamba/mamba3/quat_scan/backward.rs"
    (module documentation, "Gradient math").  Here the Jacobians are written
    as explicit 4x4 matrices: x (x) c = L(x) c = R(c) x, so
    J_c = L(x) and J_x = R(c), and the VJPs are their transposes applied to g.

Arrays: xs, ys, upstream, d_xs are [b, s, m, w]; init, d_init are [b, m, w].
"""
from __future__ import annotations

import numpy as np

BODIES = {"add": 1, "quat": 4}


def _lmat(a: np.ndarray) -> np.ndarray:
    """L(a) with a (x) b = L(a) b, Hamilton product, scalar first: [..., 4, 4]."""
    w, x, y, z = a[..., 0], a[..., 1], a[..., 2], a[..., 3]
    return np.stack([np.stack([w, -x, -y, -z], -1),
                     np.stack([x, w, -z, y], -1),
                     np.stack([y, z, w, -x], -1),
                     np.stack([z, -y, x, w], -1)], -2)


def _rmat(b: np.ndarray) -> np.ndarray:
    """R(b) with a (x) b = R(b) a: [..., 4, 4]."""
    w, x, y, z = b[..., 0], b[..., 1], b[..., 2], b[..., 3]
    return np.stack([np.stack([w, -x, -y, -z], -1),
                     np.stack([x, w, z, -y], -1),
                     np.stack([y, -z, w, x], -1),
                     np.stack([z, y, -x, w], -1)], -2)


def _matvec(mat: np.ndarray, v: np.ndarray) -> np.ndarray:
    return np.einsum("...ij,...j->...i", mat, v)


def _step(body: str, c: np.ndarray, x: np.ndarray) -> np.ndarray:
    if body == "add":
        return c + x
    return _matvec(_lmat(x), c)


def _step_vjp(body: str, c: np.ndarray, x: np.ndarray, g: np.ndarray):
    """(J_c^T g, J_x^T g) at (c, x)."""
    if body == "add":
        return g.copy(), g.copy()
    lt = np.swapaxes(_lmat(x), -1, -2)
    rt = np.swapaxes(_rmat(c), -1, -2)
    return _matvec(lt, g), _matvec(rt, g)


def _check(body: str, xs: np.ndarray, init: np.ndarray):
    if body not in BODIES:
        raise ValueError(f"unknown body {body!r}")
    w = BODIES[body]
    if xs.ndim != 4 or xs.shape[-1] != w or init.shape != (xs.shape[0], xs.shape[2], w):
        raise ValueError(f"shapes: xs {xs.shape}, init {init.shape}, width {w}")


def scan_fwd(body: str, xs, init) -> np.ndarray:
    """ys[t] = c[t] for every t (the whole trajectory)."""
    xs = np.asarray(xs, np.float64)
    init = np.asarray(init, np.float64)
    _check(body, xs, init)
    ys = np.empty_like(xs)
    c = init.copy()
    for t in range(xs.shape[1]):
        c = _step(body, c, xs[:, t])
        ys[:, t] = c
    return ys


def scan_bwd(body: str, xs, init, upstream):
    """(d_xs, d_init) of sum_t <upstream[t], ys[t]>, by the reverse sweep above."""
    xs = np.asarray(xs, np.float64)
    init = np.asarray(init, np.float64)
    upstream = np.asarray(upstream, np.float64)
    _check(body, xs, init)
    if upstream.shape != xs.shape:
        raise ValueError("upstream must have the shape of xs")
    ys = scan_fwd(body, xs, init)
    s = xs.shape[1]
    d_xs = np.empty_like(xs)
    g = np.zeros_like(init)
    for t in range(s - 1, -1, -1):
        g = g + upstream[:, t]
        c_prev = ys[:, t - 1] if t > 0 else init
        g, d_xs[:, t] = _step_vjp(body, c_prev, xs[:, t], g)
    return d_xs, g
