"""Parity of the Gated DeltaNet-2 kernels (include/gdn2.h) with the float64
oracle (oracle/gdn2.py), through the C ABI (needs an MI355X).

Tolerances, per output tensor (the context, the final state and all seven
cotangents), both asserted:
  * the burn_gdn page's own test bound, max |gpu - ref| <= 3e-3 + 3e-3
    max|ref| (its assert_close);
  * a float32 bound derived from the arithmetic: normwise
    max |gpu - ref| / max |ref| <= 1e-5.  Every output is a sum of at most
    L + D + chunk products per step, in float32 (unit roundoff 2^-24), and
    the decays (<= 0.82 on these inputs) forget a rounding error after a few
    steps, so the probabilistic rounding model gives about
    sqrt(6 (L + D + chunk)) 2^-24 <= 5e-6 at the largest sizes here; the
    bound leaves a factor 2 above that.
The device computes in float32 from float32 inputs; the oracle takes the
same float32 values widened to float64.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.inputs import make_gdn2_page_inputs, make_gdn2_random_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = capi.GDN2_INPUTS
NORMWISE_TOL = 1e-5


def close(label, got, ref):
    got = got.detach().cpu().numpy().astype(np.float64)
    scale = float(np.abs(ref).max())
    err = float(np.abs(got - ref).max())
    assert err <= 3e-3 + 3e-3 * scale, f"{label}: max diff {err:.3e} (ref max {scale:.3e})"
    rel = err / max(scale, 1e-30)
    assert rel <= NORMWISE_TOL, f"{label}: normwise error {rel:.3e} > {NORMWISE_TOL} (ref max {scale:.3e})"
    return rel


def run_case(arrays, chunk, d_ctx, d_state=None):
    dev = {n: torch.from_numpy(arrays[n]).to(DEV) for n in NAMES}
    ctx, state, bnd = capi.gdn2_fwd(*[dev[n] for n in NAMES], chunk=chunk)
    D_ctx = torch.from_numpy(d_ctx).to(DEV)
    D_st = torch.from_numpy(d_state).to(DEV) if d_state is not None else None
    grads = capi.gdn2_bwd(*[dev[n] for n in NAMES[:6]], bnd, D_ctx, D_st, chunk=chunk)
    torch.cuda.synchronize()
    r_ctx, r_state = oracle.gdn2_fwd(*[arrays[n] for n in NAMES])
    r_grads = oracle.gdn2_bwd(*[arrays[n] for n in NAMES], d_ctx, d_state)
    rel = {"context": close("context", ctx, r_ctx), "state": close("state", state, r_state)}
    for n, g, r in zip(NAMES, grads, r_grads):
        rel["d_" + n] = close("d_" + n, g, r)
    return rel


# The page's test geometries (batch, heads, time, latent, dense, chunk) and data.
PAGE = [(1, 2, 5, 3, 4, 2), (1, 2, 9, 5, 37, 4), (1, 4, 12, 64, 128, 6), (1, 2, 64, 16, 32, 64)]


@pytest.mark.parametrize("geom", PAGE, ids=lambda g: "b%dh%dt%dl%dd%dc%d" % g)
def test_page_geometries_and_data(geom):
    B, H, T, L, D, chunk = geom
    print(f"[gdn2 page {geom}]", flush=True)
    arrays = make_gdn2_page_inputs(B, H, T, L, D)
    rel = run_case(arrays, chunk, arrays["output_weight"])
    print("  relative max errors:", {k: f"{v:.1e}" for k, v in rel.items()}, flush=True)


@pytest.mark.parametrize("geom", [(2, 3, 50, 7, 100, 8), (1, 1, 200, 64, 128, 32), (3, 2, 33, 33, 65, 1),
                                  (1, 2, 40, 1, 1, 7), (2, 1, 17, 16, 100, 100), (1, 3, 128, 64, 64, 16),
                                  (1, 2, 50, 32, 300, 16), (1, 1, 1, 4, 4, 1), (1, 1, 3, 64, 1024, 2),
                                  (2, 1, 9, 64, 65, 4), (1, 1, 20, 64, 1, 3), (1, 2, 45, 64, 96, 8),
                                  (1, 1, 24, 16, 70, 8), (1, 1, 19, 32, 40, 8)],
                         ids=lambda g: "b%dh%dt%dl%dd%dc%d" % g)
def test_random_shapes_with_final_state_cotangent(geom):
    B, H, T, L, D, chunk = geom
    print(f"[gdn2 random {geom}]", flush=True)
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=sum(geom))
    rng = np.random.default_rng(1)
    d_ctx = rng.standard_normal((B, H, T, D)).astype(np.float32)
    d_state = rng.standard_normal((B, H, L, D)).astype(np.float32)
    rel = run_case(arrays, chunk, d_ctx, d_state)
    print("  relative max errors:", {k: f"{v:.1e}" for k, v in rel.items()}, flush=True)


@pytest.mark.parametrize("shape,chunks", [((1, 2, 90, 16, 48), (1, 7, 8, 30, 90, 500)),
                                          ((1, 1, 42, 64, 96), (8, 13, 42))],
                         ids=["l16", "l64"])
def test_chunk_size_does_not_change_results_beyond_rounding(shape, chunks):
    """The chunk only sets where boundary states are saved: the forward is the
    same arithmetic for every chunk (bitwise), and the backward recomputes
    the same states (bitwise too, since each chunk restarts from a state the
    forward stored exactly).  Chunk 8 keeps whole chunks' states in registers
    and its ragged last chunk in the scratch; the others use the scratch."""
    B, H, T, L, D = shape
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=4)
    dev = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    d_ctx = torch.randn((B, H, T, D), device=DEV, generator=torch.Generator(device=DEV).manual_seed(2))
    outs = []
    for chunk in chunks:
        ctx, state, bnd = capi.gdn2_fwd(*dev, chunk=chunk)
        grads = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=chunk)
        outs.append((ctx, state) + grads)
    torch.cuda.synchronize()
    for o in outs[1:]:
        for x, y in zip(outs[0], o):
            assert torch.equal(x, y)


def test_optional_outputs_and_determinism():
    arrays = make_gdn2_random_inputs(2, 2, 30, 8, 70, seed=5)
    dev = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    d_ctx = torch.randn((2, 2, 30, 70), device=DEV, generator=torch.Generator(device=DEV).manual_seed(3))
    ctx, state, bnd = capi.gdn2_fwd(*dev, chunk=4)
    ctx2, _, none = capi.gdn2_fwd(*dev, chunk=4, want_boundary=False)
    full = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=4)
    again = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=4)
    part = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=4, want=("key", "initial_state"))
    zero_state = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, torch.zeros_like(state), chunk=4)
    torch.cuda.synchronize()
    assert none is None and torch.equal(ctx, ctx2)
    for x, y, z in zip(full, again, zero_state):
        assert torch.equal(x, y) and torch.equal(x, z)
    for n, x, p in zip(NAMES, full, part):
        if n in ("key", "initial_state"):
            assert torch.equal(x, p)
        else:
            assert p is None


def test_autograd_node_against_oracle():
    """autograd.gated_deltanet2: a loss on both outputs (context and final
    state); gradients for all seven inputs, then for a tracked subset only."""
    from quaternion_cumprod_autodiff_amd.autograd import gated_deltanet2
    B, H, T, L, D = 2, 2, 40, 12, 24
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=8)
    rng = np.random.default_rng(9)
    wc = rng.standard_normal((B, H, T, D)).astype(np.float32)
    ws = rng.standard_normal((B, H, L, D)).astype(np.float32)
    ts = [torch.from_numpy(arrays[n]).to(DEV).requires_grad_() for n in NAMES]
    context, state = gated_deltanet2(*ts, chunk=7)
    ((context * torch.from_numpy(wc).to(DEV)).sum() + (state * torch.from_numpy(ws).to(DEV)).sum()).backward()
    torch.cuda.synchronize()
    ref = oracle.gdn2_bwd(*[arrays[n] for n in NAMES], wc, ws)
    for n, t, r in zip(NAMES, ts, ref):
        close("grad " + n, t.grad, r)
    # Only key and initial_state tracked: the others get no gradient.
    ts2 = [torch.from_numpy(arrays[n]).to(DEV).requires_grad_(n in ("key", "initial_state")) for n in NAMES]
    context2, _ = gated_deltanet2(*ts2, chunk=7)
    (context2 * torch.from_numpy(wc).to(DEV)).sum().backward()
    ref2 = oracle.gdn2_bwd(*[arrays[n] for n in NAMES], wc)
    for n, t, r in zip(NAMES, ts2, ref2):
        if n in ("key", "initial_state"):
            close("grad " + n, t.grad, r)
        else:
            assert t.grad is None
    with torch.no_grad():
        c3, s3 = gated_deltanet2(*ts, chunk=7)
    assert c3.grad_fn is None and torch.equal(c3, context.detach()) and torch.equal(s3, state.detach())


@pytest.mark.parametrize("chunk", [16, 32])
def test_no_grad_forward_paths_chunk_wy(chunk):
    """autograd.gated_deltanet2 without gradients: the default runs the factor
    and strip kernels through a temporary boundary buffer, equal bit for bit to
    the forward the autograd node runs; low_memory=True runs the fused kernel.
    Both against the oracle."""
    from quaternion_cumprod_autodiff_amd.autograd import gated_deltanet2
    B, H, T, L, D = 1, 3, 77, 20, 52
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=21)
    ts = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    r_ctx, r_state = oracle.gdn2_fwd(*[arrays[n] for n in NAMES])
    with torch.no_grad():
        c_fast, s_fast = gated_deltanet2(*ts, chunk=chunk)
        c_low, s_low = gated_deltanet2(*ts, chunk=chunk, low_memory=True)
    c_node, s_node, _ = capi.gdn2_fwd(*ts, chunk=chunk)
    torch.cuda.synchronize()
    assert torch.equal(c_fast, c_node) and torch.equal(s_fast, s_node)
    for label, c, st in (("default", c_fast, s_fast), ("low_memory", c_low, s_low)):
        close(label + " context", c, r_ctx)
        close(label + " state", st, r_state)


def test_bench_workload_sampled_heads():
    """The bench's launch configuration (8 x 16 heads, 2048 steps, latent 64,
    dense 128, chunk 8: the register path), checked on sampled heads: heads are independent, so
    the oracle on a head's inputs alone gives that head's exact outputs."""
    import bench
    B, H, T, L, D, _ = bench.GDN2_WORKLOAD
    chunk = 8
    g = torch.Generator(device=DEV).manual_seed(0)
    ins = [torch.randn((B, H, T, L), device=DEV, generator=g),
           torch.randn((B, H, T, L), device=DEV, generator=g) / L ** 0.5,
           torch.randn((B, H, T, D), device=DEV, generator=g),
           torch.rand((B, H, T, L), device=DEV, generator=g),
           torch.rand((B, H, T, D), device=DEV, generator=g),
           torch.rand((B, H, T, L), device=DEV, generator=g) - 1.2,
           torch.randn((B, H, L, D), device=DEV, generator=g)]
    d_ctx = torch.randn((B, H, T, D), device=DEV, generator=g)
    ctx, state, bnd = capi.gdn2_fwd(*ins, chunk=chunk)
    grads = capi.gdn2_bwd(*ins[:6], bnd, d_ctx, chunk=chunk)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1), (3, 7)):
        print(f"[gdn2 bench workload, head ({b}, {h})]", flush=True)
        host = [x[b:b + 1, h:h + 1].cpu().numpy() for x in ins]
        dc = d_ctx[b:b + 1, h:h + 1].cpu().numpy()
        r_ctx, r_state = oracle.gdn2_fwd(*host)
        r_grads = oracle.gdn2_bwd(*host, dc)
        close("context", ctx[b:b + 1, h:h + 1], r_ctx)
        close("state", state[b:b + 1, h:h + 1], r_state)
        for n, gr, r in zip(NAMES, grads, r_grads):
            close("d_" + n, gr[b:b + 1, h:h + 1], r)


def test_latent_tensors_only_4_byte_aligned():
    """Tensors that are 4- but not 16-byte aligned (views one float into a
    buffer; the API asks for 4) give the same results bit for bit."""
    arrays = make_gdn2_random_inputs(1, 2, 30, 16, 20, seed=12)
    base = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    shifted = []
    for n, t in zip(NAMES, base):
        if n in ("query", "key", "erase", "log_decay"):
            buf = torch.empty(t.numel() + 1, dtype=torch.float32, device=DEV)
            v = buf[1:].view(t.shape)
            v.copy_(t)
            assert v.data_ptr() % 16 != 0
            shifted.append(v)
        else:
            shifted.append(t)
    d_ctx = torch.randn((1, 2, 30, 20), device=DEV, generator=torch.Generator(device=DEV).manual_seed(4))
    c1, s1, b1 = capi.gdn2_fwd(*base, chunk=8)
    c2, s2, b2 = capi.gdn2_fwd(*shifted, chunk=8)
    g1 = capi.gdn2_bwd(*base[:6], b1, d_ctx, chunk=8)
    g2 = capi.gdn2_bwd(*shifted[:6], b2, d_ctx, chunk=8)
    torch.cuda.synchronize()
    assert torch.equal(c1, c2) and torch.equal(s1, s2)
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("chunk", [16, 32])
def test_chunk_wy_outputs_only_4_byte_aligned(chunk):
    """Context and final state written through the C ABI at addresses one
    float past 16-byte alignment (the API asks for 4), with D a multiple of 4
    (where aligned outputs take 16-byte stores): bit-equal to aligned ones."""
    B, H, T, L, D = 1, 3, 70, 40, 96
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=31)
    ins = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    c1, s1, b1 = capi.gdn2_fwd(*ins, chunk=chunk)
    lib = capi.load()
    cbuf = torch.empty(B * H * T * D + 1, dtype=torch.float32, device=DEV)
    sbuf = torch.empty(B * H * L * D + 1, dtype=torch.float32, device=DEV)
    b2 = torch.empty_like(b1)
    assert (cbuf.data_ptr() + 4) % 16 != 0 and (sbuf.data_ptr() + 4) % 16 != 0
    rc = lib.gdn2_fwd(*[x.data_ptr() for x in ins], cbuf.data_ptr() + 4, sbuf.data_ptr() + 4, b2.data_ptr(),
                      B, H, T, L, D, chunk, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(c1.flatten(), cbuf[1:]) and torch.equal(s1.flatten(), sbuf[1:])


@pytest.mark.parametrize("chunk", [16, 32])
def test_chunk_wy_backward_dense_only_4_byte_aligned(chunk):
    """The VJP through the C ABI with d_context and every cotangent one float
    past 16-byte alignment, D and L multiples of 4 (where aligned tensors take
    16-byte loads and stores): bit-equal to aligned tensors."""
    B, H, T, L, D = 1, 3, 70, 40, 96
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=32)
    ins = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    d_ctx = torch.randn((B, H, T, D), device=DEV, generator=torch.Generator(device=DEV).manual_seed(8))
    _, _, bnd = capi.gdn2_fwd(*ins, chunk=chunk)
    ref = capi.gdn2_bwd(*ins[:6], bnd, d_ctx, chunk=chunk)

    def shifted(n):   # a view one float into a fresh buffer
        buf = torch.empty(n + 1, dtype=torch.float32, device=DEV)
        assert (buf.data_ptr() + 4) % 16 != 0
        return buf[1:]

    dc = shifted(d_ctx.numel())
    dc.copy_(d_ctx.flatten())
    outs = [shifted(x.numel()) for x in ref]
    lib = capi.load()
    nscr = int(lib.gdn2_scratch_bytes(B, H, T, L, D, chunk))
    scratch = torch.empty(nscr // 4, dtype=torch.float32, device=DEV)
    rc = lib.gdn2_bwd(*[x.data_ptr() for x in ins[:6]], bnd.data_ptr(), dc.data_ptr(), None,
                      *[o.data_ptr() for o in outs], scratch.data_ptr(), nscr, B, H, T, L, D, chunk,
                      torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    for n, r, o in zip(NAMES, ref, outs):
        assert torch.equal(r.flatten(), o), n


@pytest.mark.parametrize("geom", [(1, 2, 60, 32, 100, 8), (1, 1, 37, 64, 65, 5), (2, 1, 21, 16, 70, 4)],
                         ids=lambda g: "b%dh%dt%dl%dd%dc%d" % g)
def test_backward_ignores_scratch_contents(geom):
    """Dense sizes that leave a head's last block partly empty (so lanes past
    D exist) with several blocks per head: the backward's results do not
    depend on what its scratch held before the call (NaN-filled against
    zero-filled, bit for bit), and match the oracle."""
    B, H, T, L, D, chunk = geom
    print(f"[gdn2 scratch {geom}]", flush=True)
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=7 + sum(geom))
    dev = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    d_ctx = torch.randn((B, H, T, D), device=DEV, generator=torch.Generator(device=DEV).manual_seed(5))
    ctx, _, bnd = capi.gdn2_fwd(*dev, chunk=chunk)
    nscr = int(capi.load().gdn2_scratch_bytes(B, H, T, L, D, chunk))
    runs = []
    for fill in (float("nan"), 0.0):
        scratch = torch.full((nscr // 4,), fill, dtype=torch.float32, device=DEV)
        runs.append(capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=chunk, scratch=scratch))
    torch.cuda.synchronize()
    for n, x, y in zip(NAMES, *runs):
        assert torch.equal(x, y), f"d_{n} depends on the scratch's previous contents"
    r_grads = oracle.gdn2_bwd(*[arrays[n] for n in NAMES], d_ctx.cpu().numpy())
    for n, g, r in zip(NAMES, runs[0], r_grads):
        close("d_" + n, g, r)


@pytest.mark.parametrize("T", [8, 9, 16, 17, 31])
@pytest.mark.parametrize("L,D", [(64, 64), (5, 20)])
def test_register_chunk_orderings(T, L, D):
    """Chunk 8 around its boundaries: one register chunk alone (T = 8), a
    ragged scratch chunk followed by a register chunk (9, 17), register chunks
    handing their next chunk's inputs over (16, 31), against the oracle, with
    two heads so the hand-over's indexing is per head."""
    B, H = 1, 2
    print(f"[gdn2 register chunks T={T} L={L} D={D}]", flush=True)
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=100 + T + L)
    rng = np.random.default_rng(T)
    d_ctx = rng.standard_normal((B, H, T, D)).astype(np.float32)
    d_state = rng.standard_normal((B, H, L, D)).astype(np.float32)
    run_case(arrays, 8, d_ctx, d_state)


# ----------------------------------------------------------- chunk-WY path
# Chunks of 16 or 32 steps select the chunk-WY kernels (float32 MFMA); the
# result does not depend on the chunk, so the page's geometries and data run
# through them at those chunks too.

@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("geom", PAGE, ids=lambda g: "b%dh%dt%dl%dd%dc%d" % g)
def test_page_geometries_and_data_chunk_wy(geom, chunk):
    B, H, T, L, D, _ = geom
    print(f"[gdn2 wy page {geom} chunk {chunk}]", flush=True)
    arrays = make_gdn2_page_inputs(B, H, T, L, D)
    rel = run_case(arrays, chunk, arrays["output_weight"])
    print("  relative max errors:", {k: f"{v:.1e}" for k, v in rel.items()}, flush=True)


@pytest.mark.parametrize("chunk", [16, 32])
@pytest.mark.parametrize("geom", [(2, 3, 50, 7, 100, 0), (1, 1, 200, 64, 128, 0), (3, 2, 33, 33, 65, 0),
                                  (1, 2, 40, 1, 1, 0), (2, 1, 17, 16, 100, 0), (1, 3, 128, 64, 64, 0),
                                  (1, 2, 50, 32, 300, 0), (1, 1, 1, 4, 4, 0), (1, 1, 3, 64, 1024, 0),
                                  (2, 1, 9, 64, 65, 0), (1, 1, 20, 64, 1, 0), (1, 2, 45, 64, 96, 0),
                                  (1, 1, 31, 17, 31, 0), (1, 1, 97, 48, 33, 0)],
                         ids=lambda g: "b%dh%dt%dl%dd%d" % g[:5])
def test_random_shapes_chunk_wy(geom, chunk):
    """Ragged last chunks (T not a multiple of the chunk, T below it), latent
    sizes that pad to 16, 32 or 64 rows, dense sizes that leave the last
    32-column tile partly empty, and a final-state cotangent."""
    B, H, T, L, D, _ = geom
    print(f"[gdn2 wy random {geom[:5]} chunk {chunk}]", flush=True)
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=sum(geom) + chunk)
    rng = np.random.default_rng(chunk)
    d_ctx = rng.standard_normal((B, H, T, D)).astype(np.float32)
    d_state = rng.standard_normal((B, H, L, D)).astype(np.float32)
    rel = run_case(arrays, chunk, d_ctx, d_state)
    print("  relative max errors:", {k: f"{v:.1e}" for k, v in rel.items()}, flush=True)


@pytest.mark.parametrize("chunk", [16, 32])
def test_chunk_wy_more_chunks_than_resident_blocks(chunk):
    """More (head, chunk) items than the gradient kernel's resident grid (two
    blocks per compute unit: 512 on MI355X), and not a multiple of it, so its
    blocks loop over two or three items each and the last round is ragged:
    15 heads x 75 chunks of 16 (1125 items) or x 38 chunks of 32 (570), with
    a ragged last chunk, latent 40 and dense 70."""
    B, H, T, L, D = 3, 5, 1190, 40, 70
    items = B * H * -(-T // chunk)
    resident = torch.cuda.get_device_properties(0).multi_processor_count * 2
    assert items > resident and items % resident != 0
    print(f"[gdn2 wy {items} items over {resident} resident blocks, chunk {chunk}]", flush=True)
    arrays = make_gdn2_random_inputs(B, H, T, L, D, seed=77)
    d_ctx = np.random.default_rng(1).standard_normal((B, H, T, D)).astype(np.float32)
    rel = run_case(arrays, chunk, d_ctx)
    print("  relative max errors:", {k: f"{v:.1e}" for k, v in rel.items()}, flush=True)


def test_chunk_wy_optional_outputs_and_determinism():
    arrays = make_gdn2_random_inputs(2, 2, 70, 20, 40, seed=15)
    dev = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    d_ctx = torch.randn((2, 2, 70, 40), device=DEV, generator=torch.Generator(device=DEV).manual_seed(6))
    ctx, state, bnd = capi.gdn2_fwd(*dev, chunk=32)
    ctx2, state2, none = capi.gdn2_fwd(*dev, chunk=32, want_boundary=False)
    full = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=32)
    again = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=32)
    part = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, chunk=32, want=("log_decay", "initial_state"))
    zero_state = capi.gdn2_bwd(*dev[:6], bnd, d_ctx, torch.zeros_like(state), chunk=32)
    torch.cuda.synchronize()
    # Without a boundary buffer the forward builds each chunk's factors itself
    # in another kernel, whose sums round in another order.
    assert none is None
    for x, y in ((ctx, ctx2), (state, state2)):
        assert float((x - y).abs().max()) <= NORMWISE_TOL * float(x.abs().max())
    for x, y, z in zip(full, again, zero_state):
        assert torch.equal(x, y) and torch.equal(x, z)
    for n, x, p in zip(NAMES, full, part):
        if n in ("log_decay", "initial_state"):
            assert torch.equal(x, p)
        else:
            assert p is None


def test_bench_workload_sampled_heads_chunk_wy():
    """The bench's launch configuration (8 x 16 heads, 2048 steps, latent 64,
    dense 128, chunk-WY at its chunk), checked on sampled heads against the
    oracle on that head's inputs alone."""
    import bench
    B, H, T, L, D, chunk = bench.GDN2_WORKLOAD
    assert chunk in (16, 32)
    g = torch.Generator(device=DEV).manual_seed(0)
    ins = [torch.randn((B, H, T, L), device=DEV, generator=g),
           torch.randn((B, H, T, L), device=DEV, generator=g) / L ** 0.5,
           torch.randn((B, H, T, D), device=DEV, generator=g),
           torch.rand((B, H, T, L), device=DEV, generator=g),
           torch.rand((B, H, T, D), device=DEV, generator=g),
           torch.rand((B, H, T, L), device=DEV, generator=g) - 1.2,
           torch.randn((B, H, L, D), device=DEV, generator=g)]
    d_ctx = torch.randn((B, H, T, D), device=DEV, generator=g)
    ctx, state, bnd = capi.gdn2_fwd(*ins, chunk=chunk)
    grads = capi.gdn2_bwd(*ins[:6], bnd, d_ctx, chunk=chunk)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (B - 1, H - 1), (5, 2)):
        print(f"[gdn2 wy bench workload, head ({b}, {h})]", flush=True)
        host = [x[b:b + 1, h:h + 1].cpu().numpy() for x in ins]
        dc = d_ctx[b:b + 1, h:h + 1].cpu().numpy()
        r_ctx, r_state = oracle.gdn2_fwd(*host)
        r_grads = oracle.gdn2_bwd(*host, dc)
        rel = {"context": close("context", ctx[b:b + 1, h:h + 1], r_ctx),
               "state": close("state", state[b:b + 1, h:h + 1], r_state)}
        for n, gr, r in zip(NAMES, grads, r_grads):
            rel["d_" + n] = close("d_" + n, gr[b:b + 1, h:h + 1], r)
        print("  relative max errors:", {k: f"{v:.1e}" for k, v in rel.items()}, flush=True)


def test_boundary_of_another_chunk_is_refused():
    """The saved state is tagged with the chunk that wrote it: chunks 4 and 5
    at T = 11 give states of the same size, and the backward must not take
    one for the other."""
    arrays = make_gdn2_random_inputs(1, 2, 11, 8, 16, seed=3)
    dev = [torch.from_numpy(arrays[n]).to(DEV) for n in NAMES]
    d_ctx = torch.ones((1, 2, 11, 16), device=DEV)
    _, _, bnd4 = capi.gdn2_fwd(*dev, chunk=4)
    assert bnd4.numel() == capi.load().gdn2_boundary_bytes(1, 2, 11, 8, 16, 5) // 4
    with pytest.raises(ValueError, match="chunk 4"):
        capi.gdn2_bwd(*dev[:6], bnd4, d_ctx, chunk=5)
    capi.gdn2_bwd(*dev[:6], bnd4, d_ctx, chunk=4)
    torch.cuda.synchronize()
