"""torch.autograd node for the quaternion cumulative-product scan.

Mirrors the custom autodiff node of the burn-mamba source page
"burn_mamba/mamba3/quat_scan/backward.rs" (the ``Autodiff`` implementation
of ``quat_cumprod`` and its ``Backward`` node):

* the node keeps only its leaves q and init, never scan intermediates; here it
  may also keep the O(N/64) saved boundary state the forward writes, so the
  backward reads q and d_cum once (``save_boundary_state=False`` keeps the
  leaves only, and the backward re-derives that state from q);
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


class QuatCumprodFunction(torch.autograd.Function):
    """cum = quat_cumprod(q, init); backward = the recompute-based VJP."""

    @staticmethod
    def forward(ctx, q: torch.Tensor, init: torch.Tensor, save_boundary_state: bool):
        q = q.contiguous()
        init = init.contiguous()
        ckpt = capi.new_ckpt(q) if save_boundary_state else None
        cum = capi.quat_cumprod_fwd(q, init, ckpt=ckpt)
        ctx.save_for_backward(q, init, ckpt)
        return cum

    @staticmethod
    def backward(ctx, d_cum: torch.Tensor):
        q, init, ckpt = ctx.saved_tensors
        want_dq, want_dinit = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (want_dq or want_dinit):
            return None, None, None
        d_q, d_init = capi.quat_cumprod_bwd(q, init, d_cum.contiguous(), ckpt,
                                            want_dq=want_dq, want_dinit=want_dinit)
        return d_q, d_init, None


def quat_cumprod(q: torch.Tensor, init: torch.Tensor, *, save_boundary_state: bool = True) -> torch.Tensor:
    """cum[t] = q_t (x) cum[t-1] with cum[-1] = init, differentiable in q and init.

    q: [b, s, h, j, 4], init: [b, h, j, 4], float32 or bfloat16, on the GPU.
    """
    if torch.is_grad_enabled() and (q.requires_grad or init.requires_grad):
        return QuatCumprodFunction.apply(q, init, save_boundary_state)
    return capi.quat_cumprod_fwd(q.contiguous(), init.contiguous())


def quat_cumprod_with_final(q: torch.Tensor, init: torch.Tensor, *, save_boundary_state: bool = True):
    """(cum, final_carry) with final_carry = cum[:, -1], a view whose gradient
    autograd folds into the last position of cum's gradient."""
    cum = quat_cumprod(q, init, save_boundary_state=save_boundary_state)
    return cum, cum[:, -1]
