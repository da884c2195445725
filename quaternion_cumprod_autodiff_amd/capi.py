"""ctypes binding of the C ABI in include/quat_cumprod.h.

Argument marshalling only: shapes, dtypes and device pointers of torch
tensors go in, every step of the scan runs in the HIP library
(libquatcumprod.so, built in-tree by build.py).  There is no fallback: if the
library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

from .build import LIB_PATH

QC_DTYPE_F32 = 0
QC_DTYPE_BF16 = 1
QC_PATH_AUTO = 0
QC_PATH_COLUMN = 1
QC_PATH_CHUNKED = 2
QC_PATH_RSCAN = 3
PATHS = {"auto": QC_PATH_AUTO, "column": QC_PATH_COLUMN, "chunked": QC_PATH_CHUNKED, "rscan": QC_PATH_RSCAN}
# Cross-tile carry scheme of the look-back path (QC_LOOKBACK_*).
LOOKBACKS = {"auto": 0, "fenwick": 1, "grouped": 2}
# How a backward without saved state gets its boundary products (QC_LEAVES_*).
LEAVES = {"auto": 0, "prepass": 1, "coresident": 2}
# What a ckpt buffer holds (QC_SAVED_*): the boundary prefix products, or only
# the final carry of every column.
SAVED = {"boundary": 0, "final": 1}

_DTYPES = {torch.float32: QC_DTYPE_F32, torch.bfloat16: QC_DTYPE_BF16}

# The exported symbols, as declared in include/quat_cumprod.h.
EXPORTS = (
    "quat_cumprod_workspace_bytes", "quat_cumprod_ckpt_bytes", "quat_cumprod_ckpt_bytes_ex",
    "quat_cumprod_workspace_init",
    "quat_cumprod_fwd", "quat_cumprod_bwd", "quat_cumprod_fwd_ex", "quat_cumprod_bwd_ex",
    "quat_cumprod_workspace_status", "quat_cumprod_strerror", "quat_cumprod_last_hip_error",
    "quat_cumprod_version", "quat_cumprod_bwd_noalloc",
    # include/qc_scan.h
    "qc_scan_width", "qc_scan_schedule_capacity", "qc_scan_schedule", "qc_scan_fwd",
    "qc_scan_bwd_trajectory", "qc_scan_bwd_checkpointed",
    # include/gdn2.h
    "gdn2_boundary_bytes", "gdn2_scratch_bytes", "gdn2_fwd", "gdn2_bwd",
    # include/qc_bench.h
    "qc_stream_copy",
)


class QcOptions(ctypes.Structure):
    _fields_ = [("path", ctypes.c_int32), ("lookback", ctypes.c_int32), ("leaves", ctypes.c_int32),
                ("saved", ctypes.c_int32), ("reserved", ctypes.c_int32 * 4)]


class QcScanPlan(ctypes.Structure):
    _fields_ = [("n_actions", ctypes.c_int64), ("bwd_start", ctypes.c_int64),
                ("forward_steps", ctypes.c_int64), ("prefix_steps", ctypes.c_int64)]


class QuatCumprodError(RuntimeError):
    def __init__(self, code: int, where: str):
        lib = load()
        msg = lib.quat_cumprod_strerror(code).decode()
        if code == -7:
            msg += ": " + lib.quat_cumprod_last_hip_error().decode()
        super().__init__(f"{where}: {msg} (code {code})")
        self.code = code


_lib = None
_lock = threading.Lock()


def load(path: str | None = None):
    """Load libquatcumprod.so (raises if it has not been built)."""
    global _lib
    with _lock:
        if _lib is not None and path is None:
            return _lib
        p = path or LIB_PATH
        if not os.path.exists(p):
            raise RuntimeError(f"HIP library not built: {p} is missing "
                               "(run __graft_entry__.build() or quaternion_cumprod_autodiff_amd/build.py)")
        lib = ctypes.CDLL(p)
        vp, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
        dims = [i64, i64, i64, i64, i32]
        lib.quat_cumprod_workspace_bytes.argtypes = dims
        lib.quat_cumprod_workspace_bytes.restype = sz
        lib.quat_cumprod_ckpt_bytes.argtypes = dims
        lib.quat_cumprod_ckpt_bytes.restype = sz
        lib.quat_cumprod_ckpt_bytes_ex.argtypes = dims + [ctypes.POINTER(QcOptions)]
        lib.quat_cumprod_ckpt_bytes_ex.restype = sz
        lib.quat_cumprod_workspace_init.argtypes = [vp, sz, vp]
        lib.quat_cumprod_workspace_init.restype = ctypes.c_int
        fwd = [vp, vp, vp, vp, sz] + dims + [vp, sz, vp]
        bwd = [vp, vp, vp, vp, sz, vp, vp] + dims + [vp, sz, vp]
        lib.quat_cumprod_fwd.argtypes = fwd
        lib.quat_cumprod_fwd.restype = ctypes.c_int
        lib.quat_cumprod_bwd.argtypes = bwd
        lib.quat_cumprod_bwd.restype = ctypes.c_int
        lib.quat_cumprod_fwd_ex.argtypes = fwd + [ctypes.POINTER(QcOptions)]
        lib.quat_cumprod_fwd_ex.restype = ctypes.c_int
        lib.quat_cumprod_bwd_ex.argtypes = bwd + [ctypes.POINTER(QcOptions)]
        lib.quat_cumprod_bwd_ex.restype = ctypes.c_int
        lib.quat_cumprod_bwd_noalloc.argtypes = [vp, vp, vp, vp, sz, vp, vp] + dims + [vp, vp]
        lib.quat_cumprod_bwd_noalloc.restype = ctypes.c_int
        lib.quat_cumprod_workspace_status.argtypes = [vp, sz, vp, i32, ctypes.POINTER(i32)]
        lib.quat_cumprod_workspace_status.restype = ctypes.c_int
        lib.quat_cumprod_strerror.argtypes = [i32]
        lib.quat_cumprod_strerror.restype = ctypes.c_char_p
        lib.quat_cumprod_last_hip_error.argtypes = []
        lib.quat_cumprod_last_hip_error.restype = ctypes.c_char_p
        lib.quat_cumprod_version.argtypes = []
        lib.quat_cumprod_version.restype = i32
        lib.qc_scan_width.argtypes = [i32]
        lib.qc_scan_width.restype = i32
        lib.qc_scan_schedule_capacity.argtypes = [i64]
        lib.qc_scan_schedule_capacity.restype = i64
        lib.qc_scan_schedule.argtypes = [i64, i32, vp, i64, ctypes.POINTER(QcScanPlan)]
        lib.qc_scan_schedule.restype = ctypes.c_int
        lib.qc_scan_fwd.argtypes = [i32, vp, vp, vp, i64, i64, i64, vp, i64, vp, i32, vp]
        lib.qc_scan_fwd.restype = ctypes.c_int
        lib.qc_scan_bwd_trajectory.argtypes = [i32, vp, vp, vp, vp, vp, vp, i64, i64, i64, vp]
        lib.qc_scan_bwd_trajectory.restype = ctypes.c_int
        lib.qc_scan_bwd_checkpointed.argtypes = [i32, vp, vp, vp, vp, vp, i64, i64, i64, vp, i64, i64,
                                                 vp, i32, vp, vp]
        lib.qc_scan_bwd_checkpointed.restype = ctypes.c_int
        lib.gdn2_boundary_bytes.argtypes = [i64] * 6
        lib.gdn2_boundary_bytes.restype = sz
        lib.gdn2_scratch_bytes.argtypes = [i64] * 6
        lib.gdn2_scratch_bytes.restype = sz
        lib.gdn2_fwd.argtypes = [vp] * 10 + [i64] * 6 + [vp]
        lib.gdn2_fwd.restype = ctypes.c_int
        lib.gdn2_bwd.argtypes = [vp] * 17 + [sz] + [i64] * 6 + [vp]
        lib.gdn2_bwd.restype = ctypes.c_int
        lib.qc_stream_copy.argtypes = [vp, vp, sz, i32, vp]
        lib.qc_stream_copy.restype = ctypes.c_int
        if path is None:
            _lib = lib
        return lib


def _check(rc: int, where: str):
    if rc != 0:
        raise QuatCumprodError(rc, where)


def _dims(q: torch.Tensor):
    if not q.is_cuda:
        raise ValueError("q must live on the GPU: the scan runs only in the HIP library, there is no CPU path")
    if q.dim() != 5 or q.shape[-1] != 4:
        raise ValueError(f"q must be [b, s, h, j, 4], got {tuple(q.shape)}")
    b, s, h, j, _ = q.shape
    return int(b), int(s), int(h), int(j)


def _check_like(name: str, t: torch.Tensor | None, shape, dtype, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")
    return _DTYPES[t.dtype]


def _ptr(t: torch.Tensor | None):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _options(path: str | None, lookback: str | None = None, leaves: str | None = None,
             saved: str = "boundary"):
    if path is None and lookback is None and leaves is None and saved == "boundary":
        return None
    o = QcOptions()
    o.path = PATHS[path or "auto"]
    o.lookback = LOOKBACKS[lookback or "auto"]
    o.leaves = LEAVES[leaves or "auto"]
    o.saved = SAVED[saved]
    return ctypes.byref(o)


def workspace_bytes(b, s, h, j, dtype=torch.float32) -> int:
    return int(load().quat_cumprod_workspace_bytes(b, s, h, j, _DTYPES[dtype]))


def ckpt_bytes(b, s, h, j, dtype=torch.float32, saved: str = "boundary") -> int:
    """Bytes of a ckpt buffer of the kind ``saved`` ("boundary" or "final")."""
    if saved not in SAVED:
        raise ValueError(f"saved must be one of {tuple(SAVED)}")
    return int(load().quat_cumprod_ckpt_bytes_ex(b, s, h, j, _DTYPES[dtype], _options(None, saved=saved)))


def _saved_kind(ckpt: torch.Tensor | None, saved: str | None) -> str:
    """The kind of a ckpt buffer: its tag from new_ckpt, else ``saved``, else
    "boundary"; a tag and an explicit ``saved`` must agree."""
    tag = getattr(ckpt, "qc_saved", None) if ckpt is not None else None
    if saved is not None and saved not in SAVED:
        raise ValueError(f"saved must be one of {tuple(SAVED)}")
    if tag is not None and saved is not None and tag != saved:
        raise ValueError(f"ckpt holds the {tag!r} state, not {saved!r}")
    return tag or saved or "boundary"


class QuatCumprodStatusError(RuntimeError):
    """A device-side condition reported through a workspace's status word:
    QC_STATUS_TIMEOUT (1, a cross-block wait hit its spin limit: results of
    the call are invalid) or QC_STATUS_ZERO (2, a backward met a prefix
    product that is exactly zero: its gradients are not finite)."""

    def __init__(self, bits: int, where: str):
        names = [n for b, n in ((1, "QC_STATUS_TIMEOUT"), (2, "QC_STATUS_ZERO")) if bits & b]
        super().__init__(f"{where}: device status {bits} ({', '.join(names) or 'unknown bits'})")
        self.bits = bits


# Byte offset of the sticky status word in a workspace (header word 2).
_STATUS_OFFSET = 8


class Workspace:
    """A zero-initialised device workspace that grows on demand.

    ``per_stream=False`` (an explicitly created workspace): one buffer per
    device; calls that share it must be ordered, as the C header requires.
    ``per_stream=True`` (the default workspace): one buffer per (device,
    stream), so calls on different streams never share carry slots or the
    leaves-only boundary scratch.  A buffer is allocated while its stream is
    current, so the caching allocator hands it (and, after growth, the old
    one) only to work ordered on that stream.

    Status: after a call, ``watch`` copies the buffer's status word into
    pinned host memory on the call's stream (no synchronisation); ``poll``
    raises QuatCumprodStatusError once such a copy has completed with a set
    bit (``wait=True`` waits for every pending copy first) and clears the
    word."""

    def __init__(self, per_stream: bool = False):
        self.per_stream = per_stream
        self._buf: dict = {}
        self._pending: list = []

    def _key(self, device: torch.device, stream):
        idx = device.index if device.index is not None else torch.cuda.current_device()
        if not self.per_stream:
            return idx
        st = stream if stream is not None else torch.cuda.current_stream(idx)
        return (idx, int(st.cuda_stream))

    def get(self, nbytes: int, device: torch.device, stream=None) -> torch.Tensor:
        key = self._key(device, stream)
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            nbytes = max(nbytes, 1 << 20)
            st = stream if stream is not None else torch.cuda.current_stream(device)
            with torch.cuda.stream(st):
                buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
            _check(load().quat_cumprod_workspace_init(_ptr(buf), buf.numel(), _stream(st)),
                   "quat_cumprod_workspace_init")
            self._buf[key] = buf
        return buf

    def status(self, device: torch.device, stream=None, clear: bool = True) -> int:
        """Sticky status bits of this workspace (for ``stream`` when per
        stream) since the last clear; synchronises the stream.  0 = normal;
        QC_STATUS_TIMEOUT = 1, QC_STATUS_ZERO = 2 (see the C header)."""
        buf = self._buf.get(self._key(device, stream))
        if buf is None:
            return 0
        out = ctypes.c_int32(0)
        _check(load().quat_cumprod_workspace_status(_ptr(buf), buf.numel(), _stream(stream), int(clear),
                                                    ctypes.byref(out)), "quat_cumprod_workspace_status")
        return int(out.value)

    def watch(self, device: torch.device, stream, where: str, word: torch.Tensor | None = None):
        """Queue an asynchronous copy of the status word after the work just
        enqueued on ``stream`` with this workspace.  ``word`` (one device
        int32) watches another status word instead, e.g. the generic scan's;
        a set word is cleared when it is reported."""
        st = stream if stream is not None else torch.cuda.current_stream(device)
        if word is None:
            buf = self._buf.get(self._key(device, st))
            if buf is None:
                return
            src = buf[_STATUS_OFFSET:_STATUS_OFFSET + 4].view(torch.int32)

            def clear():
                self.status(device, st, clear=True)
        else:
            src = word.view(torch.int32).reshape(1)

            def clear():
                with torch.cuda.stream(st):
                    src.zero_()
                st.synchronize()
        host = torch.empty(1, dtype=torch.int32, pin_memory=True)
        with torch.cuda.stream(st):
            host.copy_(src, non_blocking=True)
            ev = torch.cuda.Event()
            ev.record(st)
        self._pending.append((ev, host, clear, st, where))

    def poll(self, wait: bool = False):
        """Raise for a completed status copy that shows a set bit."""
        keep, bad = [], None
        for item in self._pending:
            ev, host, clear, st, where = item
            if wait:
                ev.synchronize()
            elif not ev.query():
                keep.append(item)
                continue
            bits = int(host.item())
            if bits and bad is None:
                bad = (bits, clear, st, where)
        self._pending = keep
        if bad is not None:
            bits, clear, st, where = bad
            clear()
            self._pending = [it for it in self._pending if it[3] != st]
            raise QuatCumprodStatusError(bits, where)


default_workspace = Workspace(per_stream=True)


def check_status(wait: bool = True):
    """Raise QuatCumprodStatusError if any watched call on the default
    workspace reported a device-side condition (``wait``: first wait for the
    pending status copies; a synchronisation point)."""
    default_workspace.poll(wait=wait)


def new_ckpt(q: torch.Tensor, saved: str = "boundary") -> torch.Tensor:
    """Allocate a buffer for the state a forward over q saves for its
    backward: "boundary" (the prefix products at a fixed stride of steps) or
    "final" (only the final carry of every column).  The buffer is tagged with
    its kind, which the forward and the backward then use."""
    b, s, h, j = _dims(q)
    ck = torch.empty(ckpt_bytes(b, s, h, j, q.dtype, saved), dtype=torch.uint8, device=q.device)
    ck.qc_saved = saved
    return ck


def quat_cumprod_fwd(q: torch.Tensor, init: torch.Tensor, cum: torch.Tensor | None = None,
                     ckpt: torch.Tensor | None = None, *, path: str | None = None, lookback: str | None = None,
                     saved: str | None = None, stream=None, workspace: Workspace | None = None) -> torch.Tensor:
    """cum[t] = q_t (x) cum[t-1], cum[-1] = init (device computation).

    If ``ckpt`` (from :func:`new_ckpt`) is given, the state for the backward
    is written into it as well (of the kind it was made for; ``saved`` names
    the kind of an untagged buffer).
    """
    b, s, h, j = _dims(q)
    dt = _dtype_code(q)
    if cum is None:
        cum = torch.empty_like(q)
    _check_like("init", init, (b, h, j, 4), q.dtype, q.device)
    _check_like("cum", cum, q.shape, q.dtype, q.device)
    if ckpt is not None and ckpt.device != q.device:
        raise ValueError("ckpt must be on q's device")
    kind = _saved_kind(ckpt, saved)
    ws = (workspace or default_workspace).get(workspace_bytes(b, s, h, j, q.dtype), q.device, stream)
    rc = load().quat_cumprod_fwd_ex(_ptr(q), _ptr(init), _ptr(cum), _ptr(ckpt),
                                    0 if ckpt is None else ckpt.numel() * ckpt.element_size(),
                                    b, s, h, j, dt, _ptr(ws), ws.numel(), _stream(stream),
                                    _options(path, lookback, saved=kind))
    _check(rc, "quat_cumprod_fwd")
    return cum


def quat_cumprod_bwd(q: torch.Tensor, init: torch.Tensor, d_cum: torch.Tensor,
                     ckpt: torch.Tensor | None = None, *, want_dq: bool = True, want_dinit: bool = True,
                     d_q: torch.Tensor | None = None, d_init: torch.Tensor | None = None,
                     path: str | None = None, lookback: str | None = None, leaves: str | None = None,
                     saved: str | None = None, stream=None, workspace: Workspace | None = None):
    """VJP of the scan: returns (d_q, d_init); an unwanted output is None.
    ``ckpt`` is the state the forward saved (its kind from its tag, else
    ``saved``).  Without ``ckpt``, ``leaves`` chooses how the boundary
    products are re-derived ("prepass", "coresident"; see QC_LEAVES_* in the C
    header)."""
    b, s, h, j = _dims(q)
    dt = _dtype_code(q)
    if want_dq and d_q is None:
        d_q = torch.empty_like(q)
    if want_dinit and d_init is None:
        d_init = torch.empty_like(init)
    if not want_dq:
        d_q = None
    if not want_dinit:
        d_init = None
    _check_like("init", init, (b, h, j, 4), q.dtype, q.device)
    _check_like("d_cum", d_cum, q.shape, q.dtype, q.device)
    _check_like("d_q", d_q, q.shape, q.dtype, q.device)
    _check_like("d_init", d_init, (b, h, j, 4), q.dtype, q.device)
    if ckpt is not None and ckpt.device != q.device:
        raise ValueError("ckpt must be on q's device")
    kind = _saved_kind(ckpt, saved)
    ws = (workspace or default_workspace).get(workspace_bytes(b, s, h, j, q.dtype), q.device, stream)
    rc = load().quat_cumprod_bwd_ex(_ptr(q), _ptr(init), _ptr(d_cum), _ptr(ckpt),
                                    0 if ckpt is None else ckpt.numel() * ckpt.element_size(),
                                    _ptr(d_q), _ptr(d_init), b, s, h, j, dt, _ptr(ws), ws.numel(),
                                    _stream(stream), _options(path, lookback, leaves, saved=kind))
    _check(rc, "quat_cumprod_bwd")
    return d_q, d_init


def stream_copy(src: torch.Tensor, dst: torch.Tensor, *, blocks_per_cu: int = 8, stream=None):
    """Plain streaming copy of src into dst (include/qc_bench.h): the
    practical bandwidth ceiling the scan kernels are measured against."""
    if src.numel() * src.element_size() != dst.numel() * dst.element_size():
        raise ValueError("src and dst must have the same size in bytes")
    _check(load().qc_stream_copy(_ptr(src), _ptr(dst), src.numel() * src.element_size(), int(blocks_per_cu),
                                 _stream(stream)), "qc_stream_copy")
    return dst


def quat_cumprod_bwd_noalloc(q: torch.Tensor, init: torch.Tensor, d_cum: torch.Tensor,
                             d_q: torch.Tensor | None, d_init: torch.Tensor | None,
                             ckpt: torch.Tensor | None = None, status: torch.Tensor | None = None, *, stream=None):
    """VJP of the scan into caller-provided outputs, with the library's fixed
    device array as workspace (quat_cumprod_bwd_noalloc): nothing is
    allocated.  ``status`` (optional) is one device int32 that receives the
    call's status bits.  ``ckpt`` must be a boundary state (this entry point
    takes no options)."""
    b, s, h, j = _dims(q)
    dt = _dtype_code(q)
    if _saved_kind(ckpt, None) != "boundary":
        raise ValueError("quat_cumprod_bwd_noalloc reads only a boundary-state ckpt")
    _check_like("init", init, (b, h, j, 4), q.dtype, q.device)
    _check_like("d_cum", d_cum, q.shape, q.dtype, q.device)
    _check_like("d_q", d_q, q.shape, q.dtype, q.device)
    _check_like("d_init", d_init, (b, h, j, 4), q.dtype, q.device)
    if status is not None and (status.dtype != torch.int32 or status.numel() != 1 or status.device != q.device):
        raise ValueError("status must be one int32 on q's device")
    rc = load().quat_cumprod_bwd_noalloc(_ptr(q), _ptr(init), _ptr(d_cum), _ptr(ckpt),
                                         0 if ckpt is None else ckpt.numel() * ckpt.element_size(),
                                         _ptr(d_q), _ptr(d_init), b, s, h, j, dt, _ptr(status), _stream(stream))
    _check(rc, "quat_cumprod_bwd_noalloc")
    return d_q, d_init


# ---------------------------------------------------------------- generic scan
# Binding of include/qc_scan.h: a scan with body "add" (c + x, width 1) or
# "quat" (x (x) c, width 4) over float32 [b, s, m, w] tensors, and its VJP from
# the whole trajectory or from k snapshots (binomial checkpointing).

SCAN_BODIES = {"add": 0, "quat": 1}


def _scan_dims(body: str, xs: torch.Tensor):
    if body not in SCAN_BODIES:
        raise ValueError(f"unknown scan body {body!r}")
    w = int(load().qc_scan_width(SCAN_BODIES[body]))
    if xs.dim() != 4 or xs.shape[-1] != w:
        raise ValueError(f"xs must be [b, s, m, {w}] for body {body!r}, got {tuple(xs.shape)}")
    if xs.dtype != torch.float32 or not xs.is_contiguous():
        raise ValueError("xs must be contiguous float32")
    if xs.device.type != "cuda":
        raise ValueError("the scan runs on the GPU only: xs must be a device tensor")
    b, s, m, _ = xs.shape
    return SCAN_BODIES[body], b, s, m, w


def _scan_like(name, t, shape, device):
    if t is None:
        return
    if tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or t.device != device or not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous float32 {tuple(shape)} on {device}")


class ScanSchedule:
    """Binomial-checkpointing schedule for ``s`` steps and ``k`` snapshot
    slots, built by the library on the host; ``device(dev)`` returns (and
    caches) its copy in device memory."""

    def __init__(self, s: int, k: int):
        lib = load()
        cap = int(lib.qc_scan_schedule_capacity(s))
        self.s, self.k = int(s), int(k)
        self.actions = torch.zeros((max(cap, 1), 4), dtype=torch.int32)
        plan = QcScanPlan()
        _check(lib.qc_scan_schedule(s, k, ctypes.c_void_p(self.actions.data_ptr()), cap, ctypes.byref(plan)),
               "qc_scan_schedule")
        self.n_actions = int(plan.n_actions)
        self.bwd_start = int(plan.bwd_start)
        self.forward_steps = int(plan.forward_steps)
        self.prefix_steps = int(plan.prefix_steps)
        self.actions = self.actions[: self.n_actions].clone()
        self._dev = {}

    def device(self, dev) -> torch.Tensor:
        dev = torch.device(dev)
        if dev not in self._dev:
            self._dev[dev] = self.actions.to(dev)
        return self._dev[dev]


def new_snapshots(body: str, xs: torch.Tensor, k: int) -> torch.Tensor:
    _, b, s, m, w = _scan_dims(body, xs)
    return torch.empty((k, b * m, w), dtype=torch.float64, device=xs.device)


def scan_fwd(body: str, xs: torch.Tensor, init: torch.Tensor, ys: torch.Tensor | None = None, *,
             schedule: ScanSchedule | None = None, snaps: torch.Tensor | None = None, want_ys: bool = True,
             stream=None):
    """ys[t] = f(ys[t-1], xs[t]) from init.  With ``schedule`` the forward
    sweep's part of it is carried out too, filling ``snaps``."""
    code, b, s, m, w = _scan_dims(body, xs)
    _scan_like("init", init, (b, m, w), xs.device)
    if want_ys and ys is None:
        ys = torch.empty_like(xs)
    if not want_ys:
        ys = None
    _scan_like("ys", ys, xs.shape, xs.device)
    sched = None
    k = 0
    start = 0
    if schedule is not None:
        if schedule.s != s:
            raise ValueError("schedule was built for another sequence length")
        if snaps is None or snaps.shape != (schedule.k, b * m, w) or snaps.dtype != torch.float64:
            raise ValueError("snaps must be float64 [k, b*m, w] (new_snapshots)")
        sched, k, start = schedule.device(xs.device), schedule.k, schedule.bwd_start
    rc = load().qc_scan_fwd(code, _ptr(xs), _ptr(init), _ptr(ys), b, s, m, _ptr(sched), start,
                            _ptr(snaps) if schedule is not None else None, k, _stream(stream))
    _check(rc, "qc_scan_fwd")
    return ys


def scan_bwd_trajectory(body: str, xs: torch.Tensor, init: torch.Tensor, ys: torch.Tensor,
                        upstream: torch.Tensor, *, d_xs: torch.Tensor | None = None,
                        d_init: torch.Tensor | None = None, stream=None):
    """VJP from the whole saved trajectory ys; returns (d_xs, d_init)."""
    code, b, s, m, w = _scan_dims(body, xs)
    d_xs = torch.empty_like(xs) if d_xs is None else d_xs
    d_init = torch.empty_like(init) if d_init is None else d_init
    for name, t, shp in (("init", init, (b, m, w)), ("ys", ys, xs.shape), ("upstream", upstream, xs.shape),
                         ("d_xs", d_xs, xs.shape), ("d_init", d_init, (b, m, w))):
        _scan_like(name, t, shp, xs.device)
    rc = load().qc_scan_bwd_trajectory(code, _ptr(xs), _ptr(init), _ptr(ys), _ptr(upstream), _ptr(d_xs),
                                       _ptr(d_init), b, s, m, _stream(stream))
    _check(rc, "qc_scan_bwd_trajectory")
    return d_xs, d_init


def scan_bwd_checkpointed(body: str, xs: torch.Tensor, init: torch.Tensor, upstream: torch.Tensor,
                          schedule: ScanSchedule, snaps: torch.Tensor, *, after_forward: bool = False,
                          status: torch.Tensor | None = None, d_xs: torch.Tensor | None = None,
                          d_init: torch.Tensor | None = None, stream=None):
    """VJP from k snapshots.  ``after_forward``: scan_fwd with this schedule
    already filled the snapshots, so the records start at bwd_start."""
    code, b, s, m, w = _scan_dims(body, xs)
    if schedule.s != s:
        raise ValueError("schedule was built for another sequence length")
    if snaps.shape != (schedule.k, b * m, w) or snaps.dtype != torch.float64 or snaps.device != xs.device:
        raise ValueError("snaps must be float64 [k, b*m, w] on xs's device (new_snapshots)")
    d_xs = torch.empty_like(xs) if d_xs is None else d_xs
    d_init = torch.empty_like(init) if d_init is None else d_init
    for name, t, shp in (("init", init, (b, m, w)), ("upstream", upstream, xs.shape),
                         ("d_xs", d_xs, xs.shape), ("d_init", d_init, (b, m, w))):
        _scan_like(name, t, shp, xs.device)
    if status is not None and (status.dtype != torch.int32 or status.numel() != 1 or status.device != xs.device):
        raise ValueError("status must be one int32 on xs's device")
    start = schedule.bwd_start if after_forward else 0
    rc = load().qc_scan_bwd_checkpointed(code, _ptr(xs), _ptr(init), _ptr(upstream), _ptr(d_xs), _ptr(d_init),
                                         b, s, m, _ptr(schedule.device(xs.device)), schedule.n_actions, start,
                                         _ptr(snaps), schedule.k, _ptr(status), _stream(stream))
    _check(rc, "qc_scan_bwd_checkpointed")
    return d_xs, d_init


# ---------------------------------------------------------------------------
# Gated DeltaNet-2 recurrence (include/gdn2.h).  query, key, erase, log_decay
# [B, H, T, L]; value, write [B, H, T, D]; initial_state [B, H, L, D]; all
# contiguous float32 on the GPU.

GDN2_INPUTS = ("query", "key", "value", "erase", "write", "log_decay", "initial_state")


def _gdn2_dims(query, value, chunk):
    if query.dim() != 4 or value.dim() != 4:
        raise ValueError("query must be [B, H, T, L] and value [B, H, T, D]")
    B, H, T, L = query.shape
    D = value.shape[3]
    if tuple(value.shape[:3]) != (B, H, T):
        raise ValueError("value must share query's [B, H, T]")
    if query.device.type != "cuda":
        raise ValueError("Gated DeltaNet-2 runs on the GPU only: inputs must be device tensors")
    if int(chunk) < 1:
        raise ValueError("chunk must be >= 1")
    return int(B), int(H), int(T), int(L), int(D), int(chunk)


def _gdn2_check(tensors: dict, B, H, T, L, D, device):
    shapes = {"query": (B, H, T, L), "key": (B, H, T, L), "erase": (B, H, T, L), "log_decay": (B, H, T, L),
              "value": (B, H, T, D), "write": (B, H, T, D), "initial_state": (B, H, L, D),
              "d_context": (B, H, T, D), "d_state": (B, H, L, D)}
    for name, t in tensors.items():
        if t is None:
            continue
        if (tuple(t.shape) != shapes[name] or t.dtype != torch.float32 or t.device != device
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be contiguous float32 {shapes[name]} on {device}")


def gdn2_fwd(query, key, value, erase, write, log_decay, initial_state, *, chunk: int = 32,
             want_boundary: bool = True, stream=None):
    """(context [B, H, T, D], final state [B, H, L, D], boundary states or None).

    Chunks of 16 and 32 run the chunk-WY form (the fastest; 32 is the
    default), every other chunk the step-by-step recurrence.  The returned
    saved state is tagged with its chunk (``gdn2_chunk``), and gdn2_bwd
    refuses it for another chunk."""
    B, H, T, L, D, chunk = _gdn2_dims(query, value, chunk)
    ins = dict(zip(GDN2_INPUTS, (query, key, value, erase, write, log_decay, initial_state)))
    _gdn2_check(ins, B, H, T, L, D, query.device)
    lib = load()
    nb = int(lib.gdn2_boundary_bytes(B, H, T, L, D, chunk))
    if nb == 0:
        raise QuatCumprodError(-2, "gdn2_fwd")
    ctx = torch.empty((B, H, T, D), dtype=torch.float32, device=query.device)
    state = torch.empty((B, H, L, D), dtype=torch.float32, device=query.device)
    bnd = torch.empty(nb // 4, dtype=torch.float32, device=query.device) if want_boundary else None
    rc = lib.gdn2_fwd(*[_ptr(ins[n]) for n in GDN2_INPUTS], _ptr(ctx), _ptr(state), _ptr(bnd),
                      B, H, T, L, D, chunk, _stream(stream))
    _check(rc, "gdn2_fwd")
    if bnd is not None:
        bnd.gdn2_chunk = chunk
    return ctx, state, bnd


def gdn2_bwd(query, key, value, erase, write, log_decay, boundary, d_context, d_state=None, *, chunk: int = 32,
             want=GDN2_INPUTS, stream=None, scratch=None):
    """Cotangents (query, key, value, erase, write, log_decay, initial_state);
    those not named in ``want`` are None.  ``boundary`` is gdn2_fwd's third
    output for the same inputs and chunk.  ``scratch`` (optional) is a float32
    device tensor of at least gdn2_scratch_bytes; by default one is allocated."""
    B, H, T, L, D, chunk = _gdn2_dims(query, value, chunk)
    ins = dict(zip(GDN2_INPUTS[:6], (query, key, value, erase, write, log_decay)))
    ins["d_context"], ins["d_state"] = d_context, d_state
    _gdn2_check(ins, B, H, T, L, D, query.device)
    lib = load()
    nb = int(lib.gdn2_boundary_bytes(B, H, T, L, D, chunk))
    if boundary is None or boundary.numel() * 4 != nb or boundary.dtype != torch.float32:
        raise ValueError("boundary must be gdn2_fwd's boundary states for the same sizes and chunk")
    made_with = getattr(boundary, "gdn2_chunk", None)
    if made_with is not None and made_with != chunk:
        raise ValueError(f"boundary was written by gdn2_fwd with chunk {made_with}, not {chunk}")
    nscr = int(lib.gdn2_scratch_bytes(B, H, T, L, D, chunk))
    if scratch is None:
        scratch = torch.empty(nscr // 4, dtype=torch.float32, device=query.device)
    elif (scratch.dtype != torch.float32 or scratch.device != query.device or not scratch.is_contiguous()
          or scratch.numel() * 4 < nscr):
        raise ValueError(f"scratch must be a contiguous float32 tensor of at least {nscr} bytes on {query.device}")
    outs = {}
    for name, src in zip(GDN2_INPUTS, (query, key, value, erase, write, log_decay, None)):
        shp = (B, H, L, D) if name == "initial_state" else tuple(src.shape)
        outs[name] = torch.empty(shp, dtype=torch.float32, device=query.device) if name in want else None
    rc = lib.gdn2_bwd(*[_ptr(ins[n]) for n in GDN2_INPUTS[:6]], _ptr(boundary), _ptr(d_context), _ptr(d_state),
                      *[_ptr(outs[n]) for n in GDN2_INPUTS], _ptr(scratch), nscr, B, H, T, L, D, chunk,
                      _stream(stream))
    _check(rc, "gdn2_bwd")
    return tuple(outs[n] for n in GDN2_INPUTS)
