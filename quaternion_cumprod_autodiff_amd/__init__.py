"""MI355X (gfx950) quaternion cumulative-product scan with a recompute-based VJP.

The computation runs in the HIP library ``libquatcumprod.so`` behind the C ABI
of ``include/quat_cumprod.h``; :mod:`.capi` is the ctypes binding and
:mod:`.autograd` wraps it as a ``torch.autograd.Function``.  Importing this
package does not load the library; the first call does.
"""

__version__ = "0.1.0"


def __getattr__(name):
    if name in ("quat_cumprod_fwd", "quat_cumprod_bwd", "new_ckpt", "workspace_bytes", "ckpt_bytes"):
        from . import capi
        return getattr(capi, name)
    if name in ("quat_cumprod", "quat_cumprod_with_final", "QuatCumprodFunction", "scan", "ScanFunction",
                "gated_deltanet2", "GatedDeltaNet2Function"):
        from . import autograd
        return getattr(autograd, name)
    raise AttributeError(name)
