"""Parity of the generic scan kernels (include/qc_scan.h) against the float64
oracle (oracle/generic_scan.py), through the C ABI (needs an MI355X).

Tolerances (float32 storage, float64 arithmetic inside):
  * forward, and the VJP from snapshots (carries recomputed in float64):
    |gpu - ref| <= 2^-23 |ref| + 1e-9 max|ref| per element, and max abs
    <= 1e-4 (the stated float32 bound);
  * VJP from the saved trajectory: the carries it reads are the float32
    outputs of the forward, rounded component by component (relative error
    2^-24 of each component, so at most 2^-24 of the carry's norm).  For the
    quaternion body d_x[t] = g (x) conj(c[t-1]) then errs by at most
    2^-24 |g| |c| = 2^-24 |d_x[t]| (norms), while g itself never reads a
    carry (J_c^T g = conj(x) (x) g), so nothing accumulates; with a factor 4 of
    margin, |gpu - ref| <= 2^-23 |ref| + 2^-21 ||ref|| + 1e-9 max|ref|, where
    ||ref|| is the norm of the element's whole vector, and max abs <= 1e-4.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def make(body, b, s, m, seed):
    """xs unit quaternions (quat) or N(0, 1) (add); init likewise; upstream N(0, 1)."""
    rng = np.random.default_rng(seed)
    w = oracle.SCAN_BODIES[body]
    xs = rng.standard_normal((b, s, m, w)).astype(np.float32)
    init = rng.standard_normal((b, m, w)).astype(np.float32)
    if body == "quat":
        xs /= np.linalg.norm(xs, axis=-1, keepdims=True)
        init /= np.linalg.norm(init, axis=-1, keepdims=True)
    up = rng.standard_normal((b, s, m, w)).astype(np.float32)
    return xs, init, up


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def host(t):
    return t.cpu().numpy().astype(np.float64)


def check(name, got, ref, rel, rel_norm=0.0):
    err = np.abs(got - ref)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    worst = float(err.max()) if err.size else 0.0
    assert worst <= 1e-4, f"{name}: max abs err {worst:.3e}"
    norm = np.linalg.norm(ref, axis=-1, keepdims=True)
    bad = err > rel * np.abs(ref) + rel_norm * norm + 1e-9 * scale
    assert not bad.any(), f"{name}: {int(bad.sum())} elements beyond the bound; worst {worst:.3e}"


SHAPES = [(1, 1, 5), (1, 7, 3), (2, 300, 37), (3, 1000, 200), (1, 257, 300)]


@pytest.mark.parametrize("body", ["add", "quat"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "b%ds%dm%d" % s)
def test_forward_and_trajectory_vjp(body, shape):
    b, s, m = shape
    print(f"[scan traj {body} {shape}]", flush=True)
    xs, init, up = make(body, b, s, m, seed=s + m)
    X, I, U = dev(xs), dev(init), dev(up)
    ys = capi.scan_fwd(body, X, I)
    d_xs, d_init = capi.scan_bwd_trajectory(body, X, I, ys, U)
    torch.cuda.synchronize()
    check("ys", host(ys), oracle.scan_fwd(body, xs, init), 2.0 ** -23)
    r_dx, r_di = oracle.scan_bwd(body, xs, init, up)
    check("d_xs", host(d_xs), r_dx, 2.0 ** -23, 2.0 ** -21)
    check("d_init", host(d_init), r_di, 2.0 ** -23, 2.0 ** -21)


@pytest.mark.parametrize("body", ["add", "quat"])
@pytest.mark.parametrize("s,k", [(1, 1), (64, 1), (300, 2), (300, 3), (1000, 8), (1000, 40), (50, 60)])
def test_checkpointed_vjp(body, s, k):
    b, m = 2, 45
    print(f"[scan ckpt {body} s={s} k={k}]", flush=True)
    xs, init, up = make(body, b, s, m, seed=7 * s + k)
    X, I, U = dev(xs), dev(init), dev(up)
    sch = capi.ScanSchedule(s, k)
    snaps = capi.new_snapshots(body, X, k)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    d_xs, d_init = capi.scan_bwd_checkpointed(body, X, I, U, sch, snaps, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    r_dx, r_di = oracle.scan_bwd(body, xs, init, up)
    check("d_xs", host(d_xs), r_dx, 2.0 ** -23)
    check("d_init", host(d_init), r_di, 2.0 ** -23)

    # The forward sweep's part done by the forward (snapshots as its output):
    # the same float64 arithmetic, so bitwise the same result.
    snaps2 = capi.new_snapshots(body, X, k)
    ys = capi.scan_fwd(body, X, I, schedule=sch, snaps=snaps2)
    d_xs2, d_init2 = capi.scan_bwd_checkpointed(body, X, I, U, sch, snaps2, after_forward=True, status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    assert torch.equal(d_xs2, d_xs) and torch.equal(d_init2, d_init)
    check("ys", host(ys), oracle.scan_fwd(body, xs, init), 2.0 ** -23)
    # Snapshots only (no ys).
    snaps3 = capi.new_snapshots(body, X, k)
    assert capi.scan_fwd(body, X, I, schedule=sch, snaps=snaps3, want_ys=False) is None
    d_xs3, _ = capi.scan_bwd_checkpointed(body, X, I, U, sch, snaps3, after_forward=True)
    torch.cuda.synchronize()
    assert torch.equal(d_xs3, d_xs)


def test_quat_body_agrees_with_the_chunked_scan():
    """The quaternion body of the generic scan and the chunked quaternion
    library compute the same thing; both within float32 rounding of the oracle
    and of each other."""
    b, s, m = 2, 700, 64
    xs, init, up = make("quat", b, s, m, seed=11)
    X, I, U = dev(xs), dev(init), dev(up)
    ys = capi.scan_fwd("quat", X, I)
    q5, i5, u5 = X.view(b, s, 1, m, 4), I.view(b, 1, m, 4), U.view(b, s, 1, m, 4)
    cum = capi.quat_cumprod_fwd(q5, i5, path="chunked")
    d_q, d_i = capi.quat_cumprod_bwd(q5, i5, u5, path="chunked")
    sch = capi.ScanSchedule(s, 6)
    d_xs, d_init = capi.scan_bwd_checkpointed("quat", X, I, U, sch, capi.new_snapshots("quat", X, 6))
    torch.cuda.synchronize()
    assert float((ys - cum.view_as(ys)).abs().max()) <= 2e-6
    assert float((d_xs - d_q.view_as(d_xs)).abs().max()) <= 1e-4
    assert float((d_init - d_i.view_as(d_init)).abs().max()) <= 1e-4


def test_optional_outputs():
    b, s, m = 1, 100, 70
    xs, init, up = make("quat", b, s, m, seed=3)
    X, I, U = dev(xs), dev(init), dev(up)
    ys = capi.scan_fwd("quat", X, I)
    full = capi.scan_bwd_trajectory("quat", X, I, ys, U)
    d_init_only = torch.full_like(I, float("nan"))
    rc = capi.load().qc_scan_bwd_trajectory(1, X.data_ptr(), I.data_ptr(), ys.data_ptr(), U.data_ptr(), None,
                                            d_init_only.data_ptr(), b, s, m, None)
    torch.cuda.synchronize()
    assert rc == 0 and torch.equal(d_init_only, full[1])


def test_bad_record_sets_status_and_stops():
    """A record out of range (a snapshot slot >= k, set from the host) is
    refused on the device: the kernel flags it and every column stops before
    touching memory through it."""
    b, s, m, k = 1, 50, 64, 3
    xs, init, up = make("add", b, s, m, seed=5)
    X, I, U = dev(xs), dev(init), dev(up)
    sch = capi.ScanSchedule(s, k)
    acts = sch.actions.clone()
    stores = (acts[:, 0] == 1).nonzero().flatten()
    acts[stores[-1], 1] = k + 5
    bad = acts.to(DEV)
    snaps = capi.new_snapshots("add", X, k)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    d_xs, d_init = torch.zeros_like(X), torch.zeros_like(I)
    rc = capi.load().qc_scan_bwd_checkpointed(0, X.data_ptr(), I.data_ptr(), U.data_ptr(), d_xs.data_ptr(),
                                              d_init.data_ptr(), b, s, m, bad.data_ptr(), sch.n_actions, 0,
                                              snaps.data_ptr(), k, status.data_ptr(), None)
    torch.cuda.synchronize()
    assert rc == 0 and int(status.item()) == 1
    assert float(d_init.abs().max()) == 0.0   # stopped before the end


def test_many_columns_sampled():
    """A large launch (65,536 columns in 256 blocks per batch entry pair),
    checked on sampled columns against the oracle."""
    b, s, m = 2, 512, 32768
    g = torch.Generator(device=DEV).manual_seed(9)
    X = torch.randn((b, s, m, 4), device=DEV, generator=g)
    X = X / X.norm(dim=-1, keepdim=True)
    I = torch.randn((b, m, 4), device=DEV, generator=g)
    I = I / I.norm(dim=-1, keepdim=True)
    U = torch.randn((b, s, m, 4), device=DEV, generator=g)
    ys = capi.scan_fwd("quat", X, I)
    d_xs, d_init = capi.scan_bwd_trajectory("quat", X, I, ys, U)
    sch = capi.ScanSchedule(s, 10)
    c_xs, c_init = capi.scan_bwd_checkpointed("quat", X, I, U, sch, capi.new_snapshots("quat", X, 10))
    torch.cuda.synchronize()
    cols = np.array([0, 1, 255, 256, 4097, 32767])
    xs_s, init_s, up_s = host(X[:, :, cols]), host(I[:, cols]), host(U[:, :, cols])
    check("ys", host(ys[:, :, cols]), oracle.scan_fwd("quat", xs_s, init_s), 2.0 ** -23)
    r_dx, r_di = oracle.scan_bwd("quat", xs_s, init_s, up_s)
    check("d_xs traj", host(d_xs[:, :, cols]), r_dx, 2.0 ** -23, 2.0 ** -21)
    check("d_init traj", host(d_init[:, cols]), r_di, 2.0 ** -23, 2.0 ** -21)
    check("d_xs ckpt", host(c_xs[:, :, cols]), r_dx, 2.0 ** -23)
    check("d_init ckpt", host(c_init[:, cols]), r_di, 2.0 ** -23)


@pytest.mark.parametrize("k", [0, 1, 2, 5])
def test_page_length_129_sum_of_carries(k):
    """The rlx-autodiff page's length-129 scan test: an add body over a carry of
    2 values, loss = the sum of every saved carry, so the upstream cotangent is
    all ones.  Then x[t] reaches the carries t .. 128, so d_x[t] = 129 - t
    exactly, d_init = 129, and ys is a running sum.  k = 0 reads the saved
    trajectory; k > 0 recomputes from k snapshots."""
    b, s, m = 1, 129, 2
    rng = np.random.default_rng(129)
    xs = rng.standard_normal((b, s, m, 1)).astype(np.float32)
    init = rng.standard_normal((b, m, 1)).astype(np.float32)
    X, I, U = dev(xs), dev(init), torch.ones((b, s, m, 1), dtype=torch.float32, device=DEV)
    ys = capi.scan_fwd("add", X, I)
    if k == 0:
        d_xs, d_init = capi.scan_bwd_trajectory("add", X, I, ys, U)
    else:
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        d_xs, d_init = capi.scan_bwd_checkpointed("add", X, I, U, capi.ScanSchedule(s, k),
                                                  capi.new_snapshots("add", X, k), status=status)
    torch.cuda.synchronize()
    want = np.broadcast_to((s - np.arange(s, dtype=np.float64))[None, :, None, None], (b, s, m, 1))
    assert np.array_equal(host(d_xs), want)
    assert np.array_equal(host(d_init), np.full((b, m, 1), float(s)))
    running = init.astype(np.float64)[:, None] + np.cumsum(xs.astype(np.float64), axis=1)
    check("ys", host(ys), running, 2.0 ** -23)
    if k:
        assert int(status.item()) == 0


@pytest.mark.parametrize("after_forward", [False, True])
def test_page_griewank_length_4_two_snapshots(after_forward):
    """The page's Griewank case: body carry + 1 (here x[t] = 1), a carry of 2
    values, length 4, k = 2 snapshots, an arbitrary upstream.  Closed form:
    ys[t] = init + t + 1, d_init = sum over t of upstream[t], d_x[t] = the sum
    of upstream over u >= t."""
    b, s, m, k = 1, 4, 2, 2
    rng = np.random.default_rng(4)
    init = rng.standard_normal((b, m, 1)).astype(np.float32)
    up = rng.standard_normal((b, s, m, 1)).astype(np.float32)
    X, I, U = torch.ones((b, s, m, 1), dtype=torch.float32, device=DEV), dev(init), dev(up)
    sch = capi.ScanSchedule(s, k)
    snaps = capi.new_snapshots("add", X, k)
    status = torch.zeros(1, dtype=torch.int32, device=DEV)
    ys = capi.scan_fwd("add", X, I, schedule=sch if after_forward else None,
                       snaps=snaps if after_forward else None)
    d_xs, d_init = capi.scan_bwd_checkpointed("add", X, I, U, sch, snaps, after_forward=after_forward,
                                              status=status)
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    u64 = up.astype(np.float64)
    check("ys", host(ys), init.astype(np.float64)[:, None] + np.arange(1, s + 1)[None, :, None, None], 2.0 ** -23)
    check("d_xs", host(d_xs), np.cumsum(u64[:, ::-1], axis=1)[:, ::-1], 2.0 ** -23)
    check("d_init", host(d_init), u64.sum(axis=1), 2.0 ** -23)


def test_random_shapes_and_snapshot_counts():
    """A seeded sweep of 24 random (body, b, s, m, k) cases, k = 0 meaning the
    trajectory VJP, each against the oracle.  s spans 1 .. 2000 (odd lengths,
    partial load groups), m spans 1 .. 300 (partial blocks), k 0 .. 40."""
    rng = np.random.default_rng(2024)
    for case in range(24):
        body = ["add", "quat"][int(rng.integers(2))]
        b = int(rng.integers(1, 4))
        s = int(rng.choice([1, 2, 7, 8, 9, 63, 129, 500, 1001, 2000]))
        m = int(rng.integers(1, 301))
        k = int(rng.choice([0, 0, 1, 2, 5, 17, 40]))
        print(f"[scan sweep {case}: {body} b={b} s={s} m={m} k={k}]", flush=True)
        xs, init, up = make(body, b, s, m, seed=1000 + case)
        X, I, U = dev(xs), dev(init), dev(up)
        r_dx, r_di = oracle.scan_bwd(body, xs, init, up)
        if k == 0:
            ys = capi.scan_fwd(body, X, I)
            d_xs, d_init = capi.scan_bwd_trajectory(body, X, I, ys, U)
            torch.cuda.synchronize()
            check("ys", host(ys), oracle.scan_fwd(body, xs, init), 2.0 ** -23)
            check("d_xs", host(d_xs), r_dx, 2.0 ** -23, 2.0 ** -21)
            check("d_init", host(d_init), r_di, 2.0 ** -23, 2.0 ** -21)
        else:
            sch = capi.ScanSchedule(s, k)
            snaps = capi.new_snapshots(body, X, k)
            status = torch.zeros(1, dtype=torch.int32, device=DEV)
            ys = capi.scan_fwd(body, X, I, schedule=sch, snaps=snaps)
            d_xs, d_init = capi.scan_bwd_checkpointed(body, X, I, U, sch, snaps, after_forward=True, status=status)
            torch.cuda.synchronize()
            assert int(status.item()) == 0
            check("ys", host(ys), oracle.scan_fwd(body, xs, init), 2.0 ** -23)
            check("d_xs", host(d_xs), r_dx, 2.0 ** -23)
            check("d_init", host(d_init), r_di, 2.0 ** -23)


@pytest.mark.parametrize("k", [0, 8])
def test_bench_workload_sampled_columns(k):
    """The scan bench's launch configuration (quaternion body, b1 s129 m2^20,
    trajectory or 8 snapshots) on sampled columns against the oracle; columns
    are independent, so a column's oracle result is exact."""
    import bench
    from quaternion_cumprod_autodiff_amd.inputs import make_generic_scan_inputs_device
    b, s, m = bench.SCAN_WORKLOADS["quat"]
    X, I, U = make_generic_scan_inputs_device("quat", b, s, m, 0, DEV)
    if k == 0:
        ys = capi.scan_fwd("quat", X, I)
        d_xs, d_init = capi.scan_bwd_trajectory("quat", X, I, ys, U)
        rel_norm = 2.0 ** -21
    else:
        sch = capi.ScanSchedule(s, k)
        snaps = capi.new_snapshots("quat", X, k)
        status = torch.zeros(1, dtype=torch.int32, device=DEV)
        ys = capi.scan_fwd("quat", X, I, schedule=sch, snaps=snaps)
        d_xs, d_init = capi.scan_bwd_checkpointed("quat", X, I, U, sch, snaps, after_forward=True, status=status)
        rel_norm = 0.0
    torch.cuda.synchronize()
    if k:
        assert int(status.item()) == 0
    cols = np.array([0, 1, 255, 256, 65537, 524287, 524288, m - 1])
    xs_s, init_s, up_s = host(X[:, :, cols]), host(I[:, cols]), host(U[:, :, cols])
    check("ys", host(ys[:, :, cols]), oracle.scan_fwd("quat", xs_s, init_s), 2.0 ** -23)
    r_dx, r_di = oracle.scan_bwd("quat", xs_s, init_s, up_s)
    check("d_xs", host(d_xs[:, :, cols]), r_dx, 2.0 ** -23, rel_norm)
    check("d_init", host(d_init[:, cols]), r_di, 2.0 ** -23, rel_norm)
