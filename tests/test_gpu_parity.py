"""Parity of the HIP library against the float64 oracle (needs an MI355X).

Every test calls the device library through the C ABI (ctypes binding in
quaternion_cumprod_autodiff_amd.capi) and compares element by element with
oracle/ on the same seeded inputs (quaternion_cumprod_autodiff_amd.inputs).

Tolerances, per output tensor (cum, d_q, d_init):
  float32 storage
    * stated bound: max |gpu - ref| <= 1e-4 for s <= 65536;
    * derived bound (every s): the library computes in float64 and rounds
      once to float32, so |gpu - ref| <= 2^-23 |ref| + 1e-9 max|ref| per
      element (half an ulp of the result, plus float64 reassociation noise).
  bfloat16 storage (float32 arithmetic inside): normwise relative error
      max |gpu - ref| / max |ref| <= 2e-2, the reference being the float64
      oracle on the bfloat16-rounded inputs.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.inputs import CONFIGS, make_config, make_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32_ABS_TOL = 1e-4
BF16_NORMWISE_TOL = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    capi.load()
    yield
    torch.cuda.synchronize()


def to_dev(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(DEV)


def to_f64(t):
    return t.float().cpu().numpy().astype(np.float64) if t is not None else None


# Backward modes without saved state, forced: the forward pre-pass over q, or
# the co-resident single pass.
LEAVES_MODES = ("prepass", "coresident")


def path_options(path):
    """A test's path name as binding options: "fenwick" and "grouped" are the
    look-back path with that carry scheme forced, "prepass" and "coresident"
    the look-back path with that leaves-only backward forced (they matter only
    without saved state)."""
    if path in ("fenwick", "grouped"):
        return dict(path="chunked", lookback=path), {}
    if path in LEAVES_MODES:
        return dict(path="chunked"), dict(leaves=path)
    return dict(path=path), {}


# use_ckpt: True (the saved boundary state), False (leaves only) or FINAL (the
# forward saves only its final carry, and the backward runs from it).
FINAL = "final"


def new_state(q, use_ckpt):
    if use_ckpt == FINAL:
        return capi.new_ckpt(q, "final")
    return capi.new_ckpt(q) if use_ckpt else None


def run_device(inp, path=None, use_ckpt=True, want_dq=True, want_dinit=True, stream=None):
    q, init, d = to_dev(inp.q, inp.dtype), to_dev(inp.init, inp.dtype), to_dev(inp.d_cum, inp.dtype)
    ck = new_state(q, use_ckpt)
    opts, bwd_only = path_options(path)
    cum = capi.quat_cumprod_fwd(q, init, ckpt=ck, stream=stream, **opts)
    d_q, d_init = capi.quat_cumprod_bwd(q, init, d, ckpt=ck, want_dq=want_dq, want_dinit=want_dinit,
                                        stream=stream, **opts, **bwd_only)
    assert capi.default_workspace.status(q.device, stream) == 0, "a cross-block wait hit its spin limit"
    return cum, d_q, d_init


def reference(inp):
    cum = oracle.fwd(inp.q64, inp.init64)
    d_q, d_init = oracle.bwd(inp.q64, inp.init64, inp.d_cum64)
    return cum, d_q, d_init


def check(name, got, ref, dtype, s, report=None):
    err = np.abs(got - ref)
    scale = float(np.abs(ref).max()) if ref.size else 0.0
    max_err = float(err.max()) if err.size else 0.0
    if report is not None:
        report[name] = (max_err, scale)
    if dtype == "f32":
        if s <= 65536:
            assert max_err <= F32_ABS_TOL, f"{name}: max abs err {max_err:.3e} > {F32_ABS_TOL}"
        bound = 2.0 ** -23 * np.abs(ref) + 1e-9 * scale
        bad = err > bound
        assert not bad.any(), (f"{name}: {int(bad.sum())} elements beyond the float32 rounding bound; "
                               f"worst err {max_err:.3e} (max|ref| {scale:.3e})")
    else:
        rel = max_err / scale if scale > 0 else max_err
        assert rel <= BF16_NORMWISE_TOL, f"{name}: normwise rel err {rel:.3e} > {BF16_NORMWISE_TOL}"


def compare(inp, path=None, use_ckpt=True, ref=None):
    cum, d_q, d_init = run_device(inp, path=path, use_ckpt=use_ckpt)
    r_cum, r_dq, r_di = ref if ref is not None else reference(inp)
    rep = {}
    check("cum", to_f64(cum), r_cum, inp.dtype, inp.s, rep)
    check("d_q", to_f64(d_q), r_dq, inp.dtype, inp.s, rep)
    check("d_init", to_f64(d_init), r_di, inp.dtype, inp.s, rep)
    print(" ".join(f"{k}: err {v[0]:.2e} max|ref| {v[1]:.2e}" for k, v in rep.items()), flush=True)
    return cum, d_q, d_init


# --------------------------------------------------------------- the configs

_config_cache = {}


def config_and_reference(name):
    """Inputs and oracle results of one named workload, kept for the next
    test of the same workload only (the full-size arrays are large)."""
    if name not in _config_cache:
        _config_cache.clear()
        inp = make_config(name)
        _config_cache[name] = (inp, reference(inp))
    return _config_cache[name]


@pytest.mark.parametrize("use_ckpt", [True, False, FINAL], ids=["saved-state", "leaves-only", "final-carry"])
@pytest.mark.parametrize("name", list(CONFIGS))
def test_config_full_parity(name, use_ckpt):
    """Every named workload at full size, in the launch configuration the
    benchmark times (default path, saved boundary state), in the
    page-faithful leaves-only mode (the backward re-derives the boundary
    state from q), and with only the forward's final carry saved."""
    mode = {True: "saved state", False: "leaves only", FINAL: "final carry"}[use_ckpt]
    print(f"[config {name} {mode}]", flush=True)
    inp, ref = config_and_reference(name)
    compare(inp, use_ckpt=use_ckpt, ref=ref)


@pytest.mark.parametrize("name", ["tiny", "medium"])
@pytest.mark.parametrize("path,use_ckpt", [("chunked", False), ("column", True), ("column", False),
                                           ("rscan", True), ("rscan", False), ("fenwick", True),
                                           ("fenwick", False), ("grouped", True), ("prepass", False),
                                           ("coresident", False), ("chunked", FINAL), ("fenwick", FINAL),
                                           ("grouped", FINAL), ("column", FINAL)])
def test_config_other_paths(name, path, use_ckpt):
    print(f"[config {name} path={path} ckpt={use_ckpt}]", flush=True)
    compare(make_config(name), path=path, use_ckpt=use_ckpt)


# ------------------------------------------------------------------ edge cases

EDGE_S = [1, 2, 3, 63, 64, 65, 127, 128, 129, 255, 257, 1000]
EDGE_HJ = [(1, 1), (1, 3), (4, 4), (4, 8), (8, 8), (5, 13), (10, 10)]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["chunked", "column", "rscan", "fenwick", "grouped", "prepass", "coresident",
                                  "final", "final-grouped"])
def test_edge_shapes(dtype, path):
    use_ckpt = path not in LEAVES_MODES
    if path.startswith("final"):
        path, use_ckpt = ("grouped" if path == "final-grouped" else "chunked"), FINAL
    for s in EDGE_S:
        for (h, j) in EDGE_HJ:
            for b in (1, 3):
                inp = make_inputs(b, s, h, j, "unit", dtype, seed=s * 131 + h * 7 + j + b)
                print(f"[edge b={b} s={s} h={h} j={j} {dtype} {path} ckpt={use_ckpt}]", flush=True)
                compare(inp, path=path, use_ckpt=use_ckpt)


def test_random_shapes():
    """A seeded sweep of shapes, dtypes, paths and saved-state modes, drawn to
    reach the combinations the grids above do not (partial column groups of
    every width, the wide forward groups, one to thousands of tiles)."""
    rng = np.random.default_rng(2024)
    for it in range(40):
        b = int(rng.choice([1, 2, 3, 5, 8, 33, 70]))
        h, j = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        if b >= 33:
            h, j = int(rng.integers(8, 17)), int(rng.integers(5, 9))   # 64-column forward groups
        s = int(rng.integers(1, 3000 if b * h * j < 400 else 300))
        dtype = "bf16" if rng.random() < 0.3 else "f32"
        path = "column" if rng.random() < 0.2 else "chunked"
        use_ckpt = bool(rng.random() < 0.7)
        if not use_ckpt and path == "chunked":
            path = LEAVES_MODES[it % 2]
        inp = make_inputs(b, s, h, j, "unit", dtype, seed=1000 + it)
        print(f"[random {it}: b={b} s={s} h={h} j={j} {dtype} {path} ckpt={use_ckpt}]", flush=True)
        compare(inp, path=path, use_ckpt=use_ckpt)


def test_random_shapes_final_carry():
    """The same kind of sweep for the backward from the final carry alone,
    over both look-backs (forced and AUTO) and both dtypes."""
    rng = np.random.default_rng(2025)
    for it in range(30):
        b = int(rng.choice([1, 2, 3, 5, 8, 33]))
        h, j = int(rng.integers(1, 12)), int(rng.integers(1, 12))
        s = int(rng.integers(1, 4000 if b * h * j < 400 else 300))
        dtype = "bf16" if rng.random() < 0.3 else "f32"
        path = ("chunked", "fenwick", "grouped")[it % 3]
        inp = make_inputs(b, s, h, j, "unit", dtype, seed=3000 + it)
        print(f"[random final {it}: b={b} s={s} h={h} j={j} {dtype} {path}]", flush=True)
        compare(inp, path=path, use_ckpt=FINAL)


@pytest.mark.parametrize("s,hj", [(2048, (1, 1)), (4100, (1, 2)), (8191, (2, 2)), (12345, (1, 64)),
                                  (3000, (33, 3))])
def test_many_tiles_ragged(s, hj):
    """Chains of many tiles (deep carry trees) with ragged tails and partial column groups."""
    inp = make_inputs(2, s, hj[0], hj[1], "unit", "f32", seed=s)
    print(f"[ragged s={s} hj={hj}]", flush=True)
    ref = reference(inp)
    for path in ("chunked", "rscan", "fenwick", "grouped"):
        compare(inp, path=path, ref=ref)
        compare(inp, path=path, use_ckpt=False, ref=ref)
        if path != "rscan":
            compare(inp, path=path, use_ckpt=FINAL, ref=ref)
    for path in LEAVES_MODES:
        compare(inp, path=path, use_ckpt=False, ref=ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("b,s,h,j", [(64, 300, 5, 13), (32, 129, 8, 16), (128, 65, 1, 64)])
def test_wide_forward_groups(dtype, b, s, h, j):
    """Many chains switch the forward to 64-column groups with half-height
    tiles: partial groups (h*j not a multiple of 64) and ragged tails."""
    inp = make_inputs(b, s, h, j, "unit", dtype, seed=b + s + h * j)
    print(f"[wide b={b} s={s} h={h} j={j} {dtype}]", flush=True)
    ref = reference(inp)
    compare(inp, ref=ref)
    compare(inp, use_ckpt=False, ref=ref)
    compare(inp, use_ckpt=FINAL, ref=ref)
    compare(inp, path="rscan", ref=ref)
    compare(inp, path="grouped", ref=ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_non_unit_steps(dtype):
    """Off the unit sphere the division by |P_t|^2 keeps the closed form exact."""
    inp = make_inputs(2, 400, 4, 8, "scaled", dtype, seed=3)
    print(f"[scaled {dtype}]", flush=True)
    compare(inp)
    compare(inp, path="column")
    # From the final carry, cum is rebuilt backwards through q_t^-1 = conj(q_t) / |q_t|^2.
    compare(inp, use_ckpt=FINAL)
    compare(inp, path="grouped", use_ckpt=FINAL)


def test_drift_bf16_column_path():
    inp = make_config("drift_bf16")
    print("[drift_bf16 column]", flush=True)
    compare(inp, path="column")


# ------------------------------------------------------------- API semantics

def test_checkpoint_and_prepass_leaves_only_agree_bitwise():
    """The pre-pass (the default leaves-only backward) writes exactly the
    boundary state the forward saves, so that leaves-only backward equals the
    saved-state one bit for bit.  The co-resident pass combines the tiles'
    products in another order: it matches to rounding, and the oracle."""
    inp = make_config("medium")
    a = run_device(inp, use_ckpt=True)
    b = run_device(inp, path="prepass", use_ckpt=False)
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    ref = reference(inp)
    c = run_device(inp, path="coresident", use_ckpt=False)
    for name, x, y, r in zip(("cum", "d_q", "d_init"), a, c, ref):
        check(name, to_f64(y), r, inp.dtype, inp.s)
        assert torch.allclose(x, y, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("use_ckpt", [True, FINAL])
def test_optional_gradients(use_ckpt):
    inp = make_inputs(2, 300, 4, 8, "unit", "f32", seed=5)
    _, dq_full, di_full = run_device(inp, use_ckpt=use_ckpt)
    _, dq_only, none1 = run_device(inp, want_dinit=False, use_ckpt=use_ckpt)
    _, none2, di_only = run_device(inp, want_dq=False, use_ckpt=use_ckpt)
    assert none1 is None and none2 is None
    assert torch.equal(dq_full, dq_only)
    assert torch.equal(di_full, di_only)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("path", ["chunked", "column"])
def test_final_carry_state_is_the_last_cum(dtype, path):
    """The final-carry state is cum[:, s-1] in the internal precision (float64
    for float32 storage, float32 for bfloat16), whichever forward path wrote
    it; and a state from the per-column forward serves the chunked backward."""
    inp = make_inputs(3, 777, 3, 5, "unit", dtype, seed=8)
    q, init, d = to_dev(inp.q, dtype), to_dev(inp.init, dtype), to_dev(inp.d_cum, dtype)
    ck = capi.new_ckpt(q, "final")
    capi.quat_cumprod_fwd(q, init, ckpt=ck, path=path)
    ct = torch.float64 if dtype == "f32" else torch.float32
    got = ck.view(ct).reshape(3, 3, 5, 4).cpu().numpy().astype(np.float64)
    ref = oracle.fwd(inp.q64, inp.init64)[:, -1]
    tol = 1e-12 if dtype == "f32" else 1e-5
    assert float(np.abs(got - ref).max()) <= tol * max(1.0, float(np.abs(ref).max()))
    d_q, d_init = capi.quat_cumprod_bwd(q, init, d, ck, path="chunked")
    assert capi.default_workspace.status(q.device) == 0
    _, r_dq, r_di = reference(inp)
    check("d_q", to_f64(d_q), r_dq, dtype, inp.s)
    check("d_init", to_f64(d_init), r_di, dtype, inp.s)


def test_final_carry_refused_by_rscan_and_noalloc():
    """The reduce-then-scan backward has no pair carries, and the allocation-free
    entry point takes no options: both refuse a final-carry state."""
    inp = make_inputs(1, 100, 2, 2, "unit", "f32", seed=6)
    q, init, d = to_dev(inp.q, "f32"), to_dev(inp.init, "f32"), to_dev(inp.d_cum, "f32")
    ck = capi.new_ckpt(q, "final")
    capi.quat_cumprod_fwd(q, init, ckpt=ck)
    with pytest.raises(capi.QuatCumprodError, match="option"):
        capi.quat_cumprod_bwd(q, init, d, ck, path="rscan")
    with pytest.raises(ValueError, match="boundary"):
        capi.quat_cumprod_bwd_noalloc(q, init, d, torch.empty_like(q), torch.empty_like(init), ck)


@pytest.mark.parametrize("use_ckpt,path", [(True, None), (FINAL, None), (FINAL, "fenwick")])
def test_determinism_repeated_runs(use_ckpt, path):
    """Every combine has a fixed association, so repeated runs agree bit for
    bit, with either saved state and either look-back."""
    inp = make_config("medium")
    first = run_device(inp, path=path, use_ckpt=use_ckpt)
    q, init, d = to_dev(inp.q, "f32"), to_dev(inp.init, "f32"), to_dev(inp.d_cum, "f32")
    ck = new_state(q, use_ckpt)
    opts, _ = path_options(path)
    for it in range(100):
        cum = capi.quat_cumprod_fwd(q, init, ckpt=ck, **opts)
        d_q, d_init = capi.quat_cumprod_bwd(q, init, d, ckpt=ck, **opts)
        assert torch.equal(cum, first[0]) and torch.equal(d_q, first[1]) and torch.equal(d_init, first[2]), it
    assert capi.default_workspace.status(q.device) == 0


def test_side_stream_and_workspace_reuse_across_shapes():
    s1 = torch.cuda.Stream()
    for shape in [(1, 300, 2, 8), (3, 129, 4, 4), (1, 5000, 1, 1), (2, 64, 8, 8)]:
        inp = make_inputs(*shape, "unit", "f32", seed=sum(shape))
        with torch.cuda.stream(s1):
            cum, d_q, d_init = run_device(inp, stream=s1)
        s1.synchronize()
        r = reference(inp)
        for name, g, rr in zip(("cum", "d_q", "d_init"), (cum, d_q, d_init), r):
            check(name, to_f64(g), rr, "f32", inp.s)


def test_concurrent_streams_with_separate_workspaces():
    """Two streams run interleaved forward + backward passes on different
    inputs at the same time, each with its own workspace (the documented rule
    for concurrent calls); both must match the oracle."""
    shapes = [(4, 2048, 16, 16, "unit", "f32", 101), (2, 6000, 4, 8, "drift", "f32", 102)]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    runs = []
    for (b, s, h, j, recipe, dtype, seed), st in zip(shapes, streams):
        inp = make_inputs(b, s, h, j, recipe, dtype, seed=seed)
        q, init, d = to_dev(inp.q, dtype), to_dev(inp.init, dtype), to_dev(inp.d_cum, dtype)
        runs.append(dict(inp=inp, q=q, init=init, d=d, st=st, ws=capi.Workspace(), out=[]))
    torch.cuda.synchronize()
    for it in range(3):
        for rn in runs:
            with torch.cuda.stream(rn["st"]):
                ck = capi.new_ckpt(rn["q"])
                cum = capi.quat_cumprod_fwd(rn["q"], rn["init"], ckpt=ck, stream=rn["st"], workspace=rn["ws"])
                d_q, d_init = capi.quat_cumprod_bwd(rn["q"], rn["init"], rn["d"], ck, stream=rn["st"],
                                                    workspace=rn["ws"])
                rn["out"].append((cum, d_q, d_init))
    torch.cuda.synchronize()
    for rn in runs:
        assert rn["ws"].status(rn["q"].device, rn["st"]) == 0
        ref = reference(rn["inp"])
        print(f"[concurrent b={rn['inp'].b} s={rn['inp'].s}]", flush=True)
        for outs in rn["out"]:
            for name, g, r in zip(("cum", "d_q", "d_init"), outs, ref):
                check(name, to_f64(g), r, "f32", rn["inp"].s)


def test_segment_chaining_on_device():
    """The final carry of one segment is the init of the next; the backward of
    the tail hands d_init back into the head's last cotangent."""
    inp = make_inputs(2, 700, 4, 4, "unit", "f32", seed=9)
    q, init, d = to_dev(inp.q, "f32"), to_dev(inp.init, "f32"), to_dev(inp.d_cum, "f32")
    s1 = 300
    full = capi.quat_cumprod_fwd(q, init)
    head = capi.quat_cumprod_fwd(q[:, :s1].contiguous(), init)
    tail = capi.quat_cumprod_fwd(q[:, s1:].contiguous(), head[:, -1].contiguous())
    np.testing.assert_allclose(to_f64(torch.cat([head, tail], 1)), to_f64(full), rtol=0, atol=2e-6)
    dq, di = capi.quat_cumprod_bwd(q, init, d)
    dq_t, di_t = capi.quat_cumprod_bwd(q[:, s1:].contiguous(), head[:, -1].contiguous(), d[:, s1:].contiguous())
    d_head = d[:, :s1].clone()
    d_head[:, -1] += di_t
    dq_h, di_h = capi.quat_cumprod_bwd(q[:, :s1].contiguous(), init, d_head)
    np.testing.assert_allclose(to_f64(torch.cat([dq_h, dq_t], 1)), to_f64(dq), rtol=0, atol=1e-4)
    np.testing.assert_allclose(to_f64(di_h), to_f64(di), rtol=0, atol=1e-4)


def test_workspace_reuse_small_then_large_shapes():
    """Regression: the carry slots of one shape overlap other parts of the
    workspace of another; slots left by earlier launches must never be
    accepted as this launch's carries."""
    seq = [make_config("medium"), make_config("tiny"), make_config("medium"),
           make_inputs(1, 3000, 2, 8, "unit", "f32", seed=4), make_config("medium")]
    for inp in seq:
        print(f"[reuse b={inp.b} s={inp.s} h={inp.h} j={inp.j}]", flush=True)
        compare(inp, path="chunked", use_ckpt=False)
        # The final-carry backward's pair slots are larger: slots of other
        # kinds and shapes lie at other offsets under them.
        compare(inp, path="chunked", use_ckpt=FINAL)


@pytest.mark.parametrize("path", ["chunked", "column", "rscan", "grouped", "coresident", "final", "final-grouped"])
def test_zero_step_is_reported(path):
    """A step that is exactly zero makes every later prefix product zero: the
    forward stays exact, and the backward (whose exact form divides by |P_t|^2)
    raises the status bit instead of failing silently."""
    inp = make_inputs(2, 300, 2, 4, "unit", "f32", seed=77)
    inp.q[1, 170, 1, 2] = 0.0
    inp.q64[1, 170, 1, 2] = 0.0
    q, init, d = to_dev(inp.q, "f32"), to_dev(inp.init, "f32"), to_dev(inp.d_cum, "f32")
    print(f"[zero step {path}]", flush=True)
    ws = capi.Workspace()
    if path.startswith("final"):
        path, ck = ("grouped" if path == "final-grouped" else "chunked"), capi.new_ckpt(q, "final")
    else:
        ck = None if path in LEAVES_MODES else capi.new_ckpt(q)
    opts, bwd_only = path_options(path)
    cum = capi.quat_cumprod_fwd(q, init, ckpt=ck, workspace=ws, **opts)
    assert ws.status(q.device) == 0
    check("cum", to_f64(cum), oracle.fwd(inp.q64, inp.init64), "f32", inp.s)
    capi.quat_cumprod_bwd(q, init, d, ck, workspace=ws, **opts, **bwd_only)
    assert ws.status(q.device) == 2            # QC_STATUS_ZERO, and cleared by the read
    assert ws.status(q.device) == 0


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_rscan_and_lookback_agree_on_long_chains(dtype):
    """Few long chains (the long-sequence shape, scaled down): the
    reduce-then-scan passes and the one-pass look-back give the same results
    to rounding, and both match the oracle, with and without saved state."""
    for (b, s, h, j) in [(1, 70000, 2, 8), (2, 40000, 1, 3), (3, 33333, 1, 1)]:
        inp = make_inputs(b, s, h, j, "unit", dtype, seed=s + h * j)
        print(f"[long chains b={b} s={s} h={h} j={j} {dtype}]", flush=True)
        ref = reference(inp)
        for path in ("rscan", "chunked", "fenwick", "grouped"):
            for use_ckpt in (True, False):
                compare(inp, path=path, use_ckpt=use_ckpt, ref=ref)
            if path != "rscan":
                compare(inp, path=path, use_ckpt=FINAL, ref=ref)
        for path in LEAVES_MODES:
            compare(inp, path=path, use_ckpt=False, ref=ref)
