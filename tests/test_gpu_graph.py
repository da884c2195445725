"""Forward + backward captured in a HIP graph and replayed (needs an MI355X).

A captured launch keeps its arguments for every replay, so the library cannot
hand the chunked kernels a fresh host-chosen launch epoch; it captures a
one-thread kernel that bumps a counter in the workspace header instead, and
the kernels read their epoch from there.  These tests replay one graph several
times on new inputs, with eager launches on the same workspace between the
replays, and check every replay against the oracle and, bitwise, against an
eager run of the same inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.inputs import make_inputs
from test_gpu_parity import FINAL, check, new_state, to_dev, to_f64

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# (b, s, h, j, recipe, dtype, path, use_ckpt): chunked with saved boundary
# state, chunked leaves-only (forward prepass inside the backward), bfloat16,
# a few long chains (tall tiles), the per-column path, the reduce-then-scan
# passes, and each look-back scheme forced ("fenwick", "grouped": the chunked
# path with that scheme; AUTO takes the grouped one for the first and the
# long-chain shapes); then the backward from the final carry alone.
CASES = [
    (2, 4096, 4, 8, "unit", "f32", "chunked", True),
    (2, 4096, 4, 8, "unit", "f32", "chunked", False),
    (2, 3000, 4, 8, "unit", "bf16", "chunked", True),
    (1, 20000, 1, 4, "drift", "f32", "chunked", True),
    (4, 700, 8, 8, "unit", "f32", "column", True),
    (1, 30000, 2, 8, "unit", "f32", "rscan", True),
    (1, 30000, 2, 8, "unit", "f32", "rscan", False),
    (1, 30000, 2, 8, "unit", "f32", "fenwick", True),
    (3, 5000, 2, 3, "unit", "bf16", "grouped", False),
    (2, 4096, 4, 8, "unit", "f32", "chunked", FINAL),
    (1, 30000, 2, 8, "unit", "f32", "fenwick", FINAL),
    (3, 5000, 2, 3, "unit", "bf16", "grouped", FINAL),
]
REPLAYS = 4


def _opts(path):
    return dict(path="chunked", lookback=path) if path in ("fenwick", "grouped") else dict(path=path)


def _eager(q, init, d, path, use_ckpt, ws):
    ck = new_state(q, use_ckpt)
    cum = capi.quat_cumprod_fwd(q, init, ckpt=ck, workspace=ws, **_opts(path))
    d_q, d_init = capi.quat_cumprod_bwd(q, init, d, ck, workspace=ws, **_opts(path))
    return cum, d_q, d_init


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"b{c[0]}s{c[1]}h{c[2]}j{c[3]}-{c[4]}-{c[5]}-{c[6]}"
                         + ("-final" if c[7] == FINAL else "" if c[7] else "-leaves"))
def test_graph_replays_match_eager_and_oracle(case):
    b, s, h, j, recipe, dtype, path, use_ckpt = case
    print(f"[graph {case}]", flush=True)
    first = make_inputs(b, s, h, j, recipe, dtype, seed=500)
    q, init, d = to_dev(first.q, dtype), to_dev(first.init, dtype), to_dev(first.d_cum, dtype)
    cum, d_q, d_init = torch.empty_like(q), torch.empty_like(q), torch.empty_like(init)
    ck = new_state(q, use_ckpt)
    ws = capi.Workspace()
    eager_ws = capi.Workspace()

    # Warm-up on the capture workspace (allocates and zeroes it outside the capture).
    capi.quat_cumprod_fwd(q, init, cum, ck, workspace=ws, **_opts(path))
    capi.quat_cumprod_bwd(q, init, d, ck, d_q=d_q, d_init=d_init, workspace=ws, **_opts(path))
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        capi.quat_cumprod_fwd(q, init, cum, ck, workspace=ws, **_opts(path))
        capi.quat_cumprod_bwd(q, init, d, ck, d_q=d_q, d_init=d_init, workspace=ws, **_opts(path))
    torch.cuda.synchronize()

    for r in range(REPLAYS):
        inp = make_inputs(b, s, h, j, recipe, dtype, seed=501 + r)
        q.copy_(to_dev(inp.q, dtype))
        init.copy_(to_dev(inp.init, dtype))
        d.copy_(to_dev(inp.d_cum, dtype))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (cum, d_q, d_init)]
        assert ws.status(q.device) == 0, f"replay {r}: status bits set"

        # Eager work between replays, on the capture workspace (host epochs)
        # and on a workspace of its own (the bitwise reference).
        other = make_inputs(b, s, h, j, recipe, dtype, seed=900 + r)
        _eager(to_dev(other.q, dtype), to_dev(other.init, dtype), to_dev(other.d_cum, dtype), path, use_ckpt, ws)
        ref_dev = _eager(q, init, d, path, use_ckpt, eager_ws)
        torch.cuda.synchronize()
        assert ws.status(q.device) == 0 and eager_ws.status(q.device) == 0

        for name, gt, et in zip(("cum", "d_q", "d_init"), got, ref_dev):
            assert torch.equal(gt.view(torch.int16) if dtype == "bf16" else gt.view(torch.int32),
                               et.view(torch.int16) if dtype == "bf16" else et.view(torch.int32)), \
                f"replay {r}: {name} differs from the eager run"
        ref = (oracle.fwd(inp.q64, inp.init64),) + tuple(oracle.bwd(inp.q64, inp.init64, inp.d_cum64))
        for name, gt, rr in zip(("cum", "d_q", "d_init"), got, ref):
            check(name, to_f64(gt), rr, dtype, s)
    del g


def test_gdn2_graph_replays_match_eager():
    """Gated DeltaNet-2 forward + VJP (two blocks per head, so the summing
    kernel runs too) captured once and replayed on new inputs, with eager
    calls between the replays; every replay equals an eager run bit for bit
    and the first also matches the oracle within the page's tolerance."""
    from quaternion_cumprod_autodiff_amd.inputs import make_gdn2_random_inputs
    names = capi.GDN2_INPUTS
    B, H, T, L, D, chunk = 1, 2, 60, 32, 100, 8
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=20)
    ins = [torch.from_numpy(arrays[n]).to(DEV) for n in names]
    d_ctx = torch.randn((B, H, T, D), device=DEV, generator=torch.Generator(device=DEV).manual_seed(21))
    ctx0, _, bnd0 = capi.gdn2_fwd(*ins, chunk=chunk)   # warm-up outside the capture
    capi.gdn2_bwd(*ins[:6], bnd0, d_ctx, chunk=chunk)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ctx, state, bnd = capi.gdn2_fwd(*ins, chunk=chunk)
        grads = capi.gdn2_bwd(*ins[:6], bnd, d_ctx, chunk=chunk)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        new = make_gdn2_random_inputs(B, H, T, L, D, seed=30 + r)
        for t, n in zip(ins, names):
            t.copy_(torch.from_numpy(new[n]).to(DEV))
        d_ctx.copy_(torch.randn((B, H, T, D), device=DEV, generator=torch.Generator(device=DEV).manual_seed(40 + r)))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (ctx, state) + tuple(grads)]
        e_ctx, e_state, e_bnd = capi.gdn2_fwd(*ins, chunk=chunk)
        e_grads = capi.gdn2_bwd(*ins[:6], e_bnd, d_ctx, chunk=chunk)
        torch.cuda.synchronize()
        for x, y in zip(got, (e_ctx, e_state) + tuple(e_grads)):
            assert torch.equal(x, y), f"replay {r} differs from the eager run"
        if r == 0:
            r_ctx, _ = oracle.gdn2_fwd(*[new[n] for n in names])
            r_grads = oracle.gdn2_bwd(*[new[n] for n in names], d_ctx.cpu().numpy())
            for gt, rr in zip([got[0]] + got[2:], [r_ctx] + list(r_grads)):
                err = float(np.abs(gt.cpu().numpy().astype(np.float64) - rr).max())
                assert err <= 3e-3 + 3e-3 * float(np.abs(rr).max())
    del g


def test_generic_scan_graph_replays_match_eager():
    """The generic scan's forward and both VJPs (trajectory, and 5 snapshots
    after the forward) captured once and replayed on new inputs; every replay
    equals an eager run bit for bit."""
    b, s, m, k = 2, 300, 70, 5
    rng = np.random.default_rng(50)
    X = torch.nn.functional.normalize(torch.from_numpy(rng.standard_normal((b, s, m, 4)).astype(np.float32)),
                                      dim=-1).to(DEV)
    I = torch.nn.functional.normalize(torch.from_numpy(rng.standard_normal((b, m, 4)).astype(np.float32)),
                                      dim=-1).to(DEV)
    U = torch.from_numpy(rng.standard_normal((b, s, m, 4)).astype(np.float32)).to(DEV)
    sch = capi.ScanSchedule(s, k)
    sch.device(DEV)                                   # device copy made outside the capture
    snaps = capi.new_snapshots("quat", X, k)
    ys = capi.scan_fwd("quat", X, I, schedule=sch, snaps=snaps)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ys = capi.scan_fwd("quat", X, I, schedule=sch, snaps=snaps)
        t_dx, t_di = capi.scan_bwd_trajectory("quat", X, I, ys, U)
        c_dx, c_di = capi.scan_bwd_checkpointed("quat", X, I, U, sch, snaps, after_forward=True)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        X.copy_(torch.nn.functional.normalize(torch.randn(X.shape, device=DEV), dim=-1))
        U.copy_(torch.randn(U.shape, device=DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (ys, t_dx, t_di, c_dx, c_di)]
        e_snaps = capi.new_snapshots("quat", X, k)
        e_ys = capi.scan_fwd("quat", X, I, schedule=sch, snaps=e_snaps)
        e_t = capi.scan_bwd_trajectory("quat", X, I, e_ys, U)
        e_c = capi.scan_bwd_checkpointed("quat", X, I, U, sch, e_snaps, after_forward=True)
        torch.cuda.synchronize()
        for x, y in zip(got, (e_ys,) + e_t + e_c):
            assert torch.equal(x, y), f"replay {r} differs from the eager run"
    del g
