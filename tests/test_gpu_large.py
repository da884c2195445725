"""Index arithmetic beyond 32 bits (needs an MI355X with >= 160 GB free).

bfloat16 storage, b=1, s=2^22+64, h*j=1024: 4,295,032,832 quaternions, so
element indices pass 2^32 and byte offsets pass 2^35.  Inputs are drawn on
the device from a seeded torch generator (unit quaternions, N(0,1)
cotangents) and rounded to bfloat16; eight sampled columns are copied back
and checked, end to end, against the float64 oracle run on exactly those
columns (the columns are independent, so this is the exact reference for
the sampled outputs).  Tolerance: normwise relative 2e-2 per output, as for
every bfloat16 workload.  The backward runs twice: from the saved boundary
state, then from the forward's final carry alone.
"""
import numpy as np
import pytest
import torch

import oracle
from quaternion_cumprod_autodiff_amd import capi

pytestmark = pytest.mark.gpu

B, S, H, J = 1, (1 << 22) + 64, 32, 32
M = H * J
COLS = [0, 1, 31, 32, 513, 700, M - 2, M - 1]


def _unit_bf16(shape, gen, chunk_rows):
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    flat = out.view(-1, 4)
    for r0 in range(0, flat.shape[0], chunk_rows):
        n = min(chunk_rows, flat.shape[0] - r0)
        x = torch.randn(n, 4, dtype=torch.float32, device="cuda:0", generator=gen)
        flat[r0:r0 + n] = (x / x.norm(dim=1, keepdim=True)).to(torch.bfloat16)
    return out


def _normal_bf16(shape, gen, chunk_rows):
    out = torch.empty(shape, dtype=torch.bfloat16, device="cuda:0")
    flat = out.view(-1, 4)
    for r0 in range(0, flat.shape[0], chunk_rows):
        n = min(chunk_rows, flat.shape[0] - r0)
        flat[r0:r0 + n] = torch.randn(n, 4, dtype=torch.float32, device="cuda:0", generator=gen).to(torch.bfloat16)
    return out


def _col(t, m):
    """[S, 4] float64 host copy of column m of a [1, S, H, J, 4] tensor."""
    return t.view(B, S, M, 4)[0, :, m].float().cpu().numpy().astype(np.float64)


def test_beyond_32bit_indices_sampled_columns():
    torch.cuda.empty_cache()
    free, _ = torch.cuda.mem_get_info(0)
    need = 4 * B * S * M * 8 + (B * S * M // 64) * 16 + (4 << 30)
    if free < need:
        pytest.skip(f"needs {need / 2**30:.0f} GiB of free device memory, {free / 2**30:.0f} available")
    assert B * S * M > (1 << 32)
    gen = torch.Generator(device="cuda:0").manual_seed(4242)
    chunk = 1 << 26
    print(f"[large b={B} s={S} h={H} j={J} bf16: {B * S * M} quaternions]", flush=True)
    q = _unit_bf16((B, S, H, J, 4), gen, chunk)
    init = _unit_bf16((B, H, J, 4), gen, chunk)
    d = _normal_bf16((B, S, H, J, 4), gen, chunk)
    ck = capi.new_ckpt(q)
    ws = capi.Workspace()
    cum = capi.quat_cumprod_fwd(q, init, ckpt=ck, workspace=ws)
    d_q, d_init = capi.quat_cumprod_bwd(q, init, d, ck, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status(q.device) == 0
    print("[large] device done, checking sampled columns", flush=True)

    nc = len(COLS)
    q64 = np.stack([_col(q, m) for m in COLS], axis=1).reshape(1, S, nc, 1, 4)
    d64 = np.stack([_col(d, m) for m in COLS], axis=1).reshape(1, S, nc, 1, 4)
    i64 = init.view(B, M, 4)[0, COLS].float().cpu().numpy().astype(np.float64).reshape(1, nc, 1, 4)
    r_cum = oracle.fwd(q64, i64)
    r_dq, r_di = oracle.bwd(q64, i64, d64)
    got_cum = np.stack([_col(cum, m) for m in COLS], axis=1).reshape(r_cum.shape)
    got_dq = np.stack([_col(d_q, m) for m in COLS], axis=1).reshape(r_dq.shape)
    got_di = d_init.view(B, M, 4)[0, COLS].float().cpu().numpy().astype(np.float64).reshape(r_di.shape)
    for name, g, r in (("cum", got_cum, r_cum), ("d_q", got_dq, r_dq), ("d_init", got_di, r_di)):
        rel = float(np.abs(g - r).max() / np.abs(r).max())
        print(f"[large] {name}: normwise rel err {rel:.2e}", flush=True)
        assert np.isfinite(g).all(), name
        assert rel <= 2e-2, f"{name}: normwise rel err {rel:.3e}"

    # The backward from the final carry alone, same inputs, into the same buffers.
    print("[large] final-carry backward", flush=True)
    fin = capi.new_ckpt(q, "final")
    capi.quat_cumprod_fwd(q, init, cum, ckpt=fin, workspace=ws)
    capi.quat_cumprod_bwd(q, init, d, fin, d_q=d_q, d_init=d_init, workspace=ws)
    torch.cuda.synchronize()
    assert ws.status(q.device) == 0
    got_dq = np.stack([_col(d_q, m) for m in COLS], axis=1).reshape(r_dq.shape)
    got_di = d_init.view(B, M, 4)[0, COLS].float().cpu().numpy().astype(np.float64).reshape(r_di.shape)
    for name, g, r in (("d_q (final carry)", got_dq, r_dq), ("d_init (final carry)", got_di, r_di)):
        rel = float(np.abs(g - r).max() / np.abs(r).max())
        print(f"[large] {name}: normwise rel err {rel:.2e}", flush=True)
        assert np.isfinite(g).all(), name
        assert rel <= 2e-2, f"{name}: normwise rel err {rel:.3e}"
    del q, d, cum, d_q, ck, fin, ws
    torch.cuda.empty_cache()
