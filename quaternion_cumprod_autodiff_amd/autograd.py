"""torch.autograd node for the quaternion cumulative-product scan.

Mirrors the custom autodiff node of the burn-mamba source page
"burn_mamba/mamba3/quat_scan/backward.rs" (the ``Autodiff`` implementation
of ``quat_cumprod`` and its ``Backward`` node):

* the node keeps only its leaves q and init, never scan intermediates; here it
  may also keep a small state the forward writes, so that the backward reads
  q and d_cum once: ``saved="boundary"`` (default) the prefix products every
  64 steps, O(N/64); ``saved="final"`` only the final carry of every column,
  O(b*h*j), from which the backward rebuilds cum backwards; ``saved="none"``
  keeps the leaves only, and the backward re-derives the boundary products
  from q (one more read of q);
* the backward recomputes the prefix products and returns the VJP;
* a gradient is produced only for an input that requires one;
* the final carry is a slice of cum, so its gradient reaches the node folded
  into the last position of d_cum (autograd's slice backward does the fold);
* without tracked inputs the forward runs alone.

All arithmetic runs in the HIP library through :mod:`.capi`.
"""
from __future__ import annotations

import torch

from . import capi


_STATUS_MODES = ("deferred", "sync")
_SAVED_MODES = ("boundary", "final", "none")


class QuatCumprodFunction(torch.autograd.Function):
    """cum = quat_cumprod(q, init); backward = the recompute-based VJP.

    Device-side conditions (a cross-block wait at its spin limit, a zero
    prefix product in the backward) are read from the workspace's status word
    without stalling the stream: each call queues an asynchronous copy of the
    word, and the next call through this node raises QuatCumprodStatusError
    for any copy that has completed with a bit set (capi.check_status() waits
    for all of them: a synchronisation point).  status_check="sync" waits
    after the backward instead and raises from it."""

    @staticmethod
    def forward(ctx, q: torch.Tensor, init: torch.Tensor, saved: str, status_check: str):
        capi.default_workspace.poll()
        q = q.contiguous()
        init = init.contiguous()
        ckpt = None if saved == "none" else capi.new_ckpt(q, saved)
        cum = capi.quat_cumprod_fwd(q, init, ckpt=ckpt)
        capi.default_workspace.watch(q.device, None, "quat_cumprod forward")
        ctx.save_for_backward(q, init, ckpt)
        ctx.saved_kind = saved
        ctx.status_check = status_check
        return cum

    @staticmethod
    def backward(ctx, d_cum: torch.Tensor):
        q, init, ckpt = ctx.saved_tensors
        want_dq, want_dinit = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (want_dq or want_dinit):
            return None, None, None, None
        capi.default_workspace.poll()
        d_q, d_init = capi.quat_cumprod_bwd(q, init, d_cum.contiguous(), ckpt, want_dq=want_dq,
                                            want_dinit=want_dinit,
                                            saved=None if ckpt is None else ctx.saved_kind)
        capi.default_workspace.watch(q.device, None, "quat_cumprod backward")
        if ctx.status_check == "sync":
            capi.default_workspace.poll(wait=True)
        return d_q, d_init, None, None


def quat_cumprod(q: torch.Tensor, init: torch.Tensor, *, saved: str = "boundary",
                 status_check: str = "deferred") -> torch.Tensor:
    """cum[t] = q_t (x) cum[t-1] with cum[-1] = init, differentiable in q and init.

    q: [b, s, h, j, 4], init: [b, h, j, 4], float32 or bfloat16, on the GPU.
    saved: what the node keeps beside q and init for its backward, "boundary"
    (default), "final" or "none" (see the module docstring).
    status_check: "deferred" (default) raises a device-side failure at the
    next call or at capi.check_status(); "sync" raises it from the backward.
    """
    if status_check not in _STATUS_MODES:
        raise ValueError(f"status_check must be one of {_STATUS_MODES}")
    if saved not in _SAVED_MODES:
        raise ValueError(f"saved must be one of {_SAVED_MODES}")
    if torch.is_grad_enabled() and (q.requires_grad or init.requires_grad):
        return QuatCumprodFunction.apply(q, init, saved, status_check)
    capi.default_workspace.poll()
    cum = capi.quat_cumprod_fwd(q.contiguous(), init.contiguous())
    capi.default_workspace.watch(q.device, None, "quat_cumprod forward")
    return cum


def quat_cumprod_with_final(q: torch.Tensor, init: torch.Tensor, *, saved: str = "boundary",
                            status_check: str = "deferred"):
    """(cum, final_carry) with final_carry = cum[:, -1], a view whose gradient
    autograd folds into the last position of cum's gradient."""
    cum = quat_cumprod(q, init, saved=saved, status_check=status_check)
    return cum, cum[:, -1]


# ---------------------------------------------------------------------------
# Generic scan (include/qc_scan.h) as an autograd node, after the Scan op of the
# rlx-autodiff source page "src/decompose_backward.rs": the forward returns
# every carry (its save_trajectory case); the backward is the scan VJP, read
# from the saved trajectory (num_checkpoints = 0) or from k snapshots that the
# forward takes on the way, recomputing the carries between them (its
# num_checkpoints = k, "Griewank", case).

_schedules: dict = {}


def _schedule(s: int, k: int) -> capi.ScanSchedule:
    key = (int(s), int(k))
    if key not in _schedules:
        _schedules[key] = capi.ScanSchedule(s, k)
    return _schedules[key]


class ScanFunction(torch.autograd.Function):
    """ys = scan(body, xs, init); backward = the VJP of every saved carry."""

    @staticmethod
    def forward(ctx, body: str, xs: torch.Tensor, init: torch.Tensor, num_checkpoints: int):
        xs = xs.contiguous()
        init = init.contiguous()
        ctx.body = body
        ctx.k = int(num_checkpoints)
        if ctx.k > 0:
            sched = _schedule(xs.shape[1], ctx.k)
            snaps = capi.new_snapshots(body, xs, ctx.k)
            ys = capi.scan_fwd(body, xs, init, schedule=sched, snaps=snaps)
            ctx.sched = sched
            ctx.fresh_snapshots = True
            ctx.save_for_backward(xs, init, snaps)
        else:
            ys = capi.scan_fwd(body, xs, init)
            ctx.save_for_backward(xs, init, ys)
        return ys

    @staticmethod
    def backward(ctx, d_ys: torch.Tensor):
        xs, init, saved = ctx.saved_tensors
        want_dxs, want_dinit = ctx.needs_input_grad[1], ctx.needs_input_grad[2]
        if not (want_dxs or want_dinit):
            return None, None, None, None
        d_ys = d_ys.contiguous()
        if ctx.k > 0:
            # The VJP overwrites the snapshots; a second backward through the
            # same graph (retain_graph) starts again from init.  A schedule
            # record the device refuses stops its column and sets `status`,
            # watched like the scan's workspace status (raised at the next
            # call or at capi.check_status()).
            capi.default_workspace.poll()
            status = torch.zeros(1, dtype=torch.int32, device=xs.device)
            d_xs, d_init = capi.scan_bwd_checkpointed(ctx.body, xs, init, d_ys, ctx.sched, saved,
                                                      after_forward=ctx.fresh_snapshots, status=status)
            capi.default_workspace.watch(xs.device, None, "scan checkpointed backward", word=status)
            ctx.fresh_snapshots = False
        else:
            d_xs, d_init = capi.scan_bwd_trajectory(ctx.body, xs, init, saved, d_ys)
        return None, (d_xs if want_dxs else None), (d_init if want_dinit else None), None


def scan(body: str, xs: torch.Tensor, init: torch.Tensor, *, num_checkpoints: int = 0) -> torch.Tensor:
    """Every carry of c[t] = f(c[t-1], xs[t]), c[-1] = init, differentiable in
    xs and init.  body: "add" (f = c + x, width 1) or "quat" (f = x (x) c,
    width 4).  xs: [b, s, m, w], init: [b, m, w], float32, on the GPU.
    num_checkpoints = 0 saves the whole trajectory for the backward; k > 0
    keeps k snapshots and recomputes the rest (binomial checkpointing)."""
    if num_checkpoints < 0:
        raise ValueError("num_checkpoints must be >= 0")
    if torch.is_grad_enabled() and (xs.requires_grad or init.requires_grad):
        return ScanFunction.apply(body, xs, init, num_checkpoints)
    return capi.scan_fwd(body, xs.contiguous(), init.contiguous())


# ---------------------------------------------------------------------------
# Gated DeltaNet-2 (include/gdn2.h) as an autograd node, after the custom
# backward node of the burn_gdn source page "src/chunk_wy/custom_backward.rs":
# the forward returns the context and the final state and keeps the inputs and
# the boundary states; the backward recomputes in-chunk states from them and
# returns a cotangent for each tracked input only.  Here the final state's
# cotangent is used too when the loss reaches the state.

class GatedDeltaNet2Function(torch.autograd.Function):
    @staticmethod
    def forward(ctx, query, key, value, erase, write, log_decay, initial_state, chunk: int):
        ins = [t.contiguous() for t in (query, key, value, erase, write, log_decay, initial_state)]
        context, state, boundary = capi.gdn2_fwd(*ins, chunk=chunk)
        ctx.chunk = int(chunk)
        ctx.save_for_backward(*ins[:6], boundary)
        return context, state

    @staticmethod
    def backward(ctx, d_context, d_state):
        *ins, boundary = ctx.saved_tensors
        want = tuple(n for n, need in zip(capi.GDN2_INPUTS, ctx.needs_input_grad[:7]) if need)
        if not want:
            return (None,) * 8
        if d_context is None:
            d_context = torch.zeros_like(ins[2])
        grads = capi.gdn2_bwd(*ins, boundary, d_context.contiguous(),
                              None if d_state is None else d_state.contiguous(), chunk=ctx.chunk, want=want)
        return (*grads, None)


def gated_deltanet2(query, key, value, erase, write, log_decay, initial_state, *, chunk: int = 32,
                    low_memory: bool = False):
    """(context [B, H, T, D], final state [B, H, L, D]) of the gated delta-rule
    recurrence, differentiable in all seven inputs; float32 tensors on the GPU
    (query, key, erase, log_decay [B, H, T, L]; value, write [B, H, T, D];
    initial_state [B, H, L, D]).

    Without gradients to track, chunks of 16 and 32 run the factor and strip
    kernels through a temporary boundary buffer (gdn2_boundary_bytes), the
    faster forward; low_memory=True runs the kernel that needs no memory
    beyond the outputs instead."""
    ins = (query, key, value, erase, write, log_decay, initial_state)
    if torch.is_grad_enabled() and any(t.requires_grad for t in ins):
        return GatedDeltaNet2Function.apply(*ins, chunk)
    context, state, _ = capi.gdn2_fwd(*[t.contiguous() for t in ins], chunk=chunk, want_boundary=not low_memory)
    return context, state
