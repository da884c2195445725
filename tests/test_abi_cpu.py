"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/quat_cumprod.h, include/qc_scan.h, include/gdn2.h and include/qc_bench.h declare, sizes its buffers as documented, and rejects
bad arguments with the documented codes before any HIP call (so fake device
pointers are safe here)."""
import ctypes
import os
import re
import subprocess

import pytest

from quaternion_cumprod_autodiff_amd import capi
from quaternion_cumprod_autodiff_amd.build import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("quat_cumprod.h", "qc_scan.h", "gdn2.h", "qc_bench.h")]

OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_ALIAS, E_WS, E_HIP, E_OPT = 0, -1, -2, -3, -4, -5, -6, -7, -8


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB_PATH):
        from quaternion_cumprod_autodiff_amd.build import build
        build()
    return capi.load()


def header_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b((?:quat_cumprod|qc_scan|gdn2|qc_stream)_\w+)\s*\(", text))
    return sorted(names)


def test_header_declares_what_the_binding_uses():
    assert header_functions() == sorted(capi.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT ((?:quat_cumprod|qc_scan|gdn2|qc_stream)_\w+)", out))
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, missing
    for f in header_functions():
        assert getattr(lib, f) is not None


def test_no_oracle_symbols_in_library():
    out = subprocess.run(["nm", "-D", LIB_PATH], capture_output=True, text=True, check=True).stdout
    assert "oracle" not in out


def test_version_and_strerror(lib):
    assert lib.quat_cumprod_version() == 100
    for code in (OK, E_NULL, E_SHAPE, E_ALIGN, E_DTYPE, E_ALIAS, E_WS, E_HIP, E_OPT):
        msg = lib.quat_cumprod_strerror(code).decode()
        assert msg and msg != "unknown error code"
    assert lib.quat_cumprod_strerror(-99).decode() == "unknown error code"
    assert lib.quat_cumprod_last_hip_error().decode() == ""


def test_buffer_sizes(lib):
    # ckpt: one internal-precision quaternion per column every 64 steps.
    for (b, s, h, j) in [(1, 1, 1, 1), (8, 4096, 32, 32), (1, 262144, 2, 8), (2, 65, 3, 5)]:
        n_ck = -(-s // 64)
        assert lib.quat_cumprod_ckpt_bytes(b, s, h, j, 0) == b * n_ck * h * j * 32
        assert lib.quat_cumprod_ckpt_bytes(b, s, h, j, 1) == b * n_ck * h * j * 16
        ws = lib.quat_cumprod_workspace_bytes(b, s, h, j, 0)
        assert ws >= lib.quat_cumprod_ckpt_bytes(b, s, h, j, 0) + 256 and ws % 256 == 0
    for bad in [(0, 1, 1, 1), (1, 0, 1, 1), (1, 1, 0, 1), (1, 1, 1, -3)]:
        assert lib.quat_cumprod_workspace_bytes(*bad, 0) == 0
        assert lib.quat_cumprod_ckpt_bytes(*bad, 0) == 0
    assert lib.quat_cumprod_workspace_bytes(1, 1, 1, 1, 7) == 0
    # sizes beyond the library's limits are rejected, not wrapped
    assert lib.quat_cumprod_workspace_bytes(1 << 20, 1 << 20, 1 << 10, 1 << 10, 0) == 0


# Fake, well-aligned, non-overlapping device addresses (never dereferenced).
def P(n):
    return ctypes.c_void_p(0x10_0000_0000 * n)


SHAPE = (2, 100, 3, 4)


def fwd(lib, q=1, init=2, cum=3, ckpt=None, ckb=0, shape=SHAPE, dt=0, ws=5, wsb=None, opts=None):
    ptr = lambda v: None if v is None else (v if isinstance(v, ctypes.c_void_p) else P(v))
    if wsb is None:
        wsb = lib.quat_cumprod_workspace_bytes(*shape, dt) if dt in (0, 1) else 1 << 20
    return lib.quat_cumprod_fwd_ex(ptr(q), ptr(init), ptr(cum), ptr(ckpt), ckb, *shape, dt, ptr(ws), wsb,
                                   None, opts)


def bwd(lib, q=1, init=2, dcum=3, ckpt=None, ckb=0, dq=6, di=7, shape=SHAPE, dt=0, ws=5, wsb=None, opts=None):
    ptr = lambda v: None if v is None else (v if isinstance(v, ctypes.c_void_p) else P(v))
    if wsb is None:
        wsb = lib.quat_cumprod_workspace_bytes(*shape, dt) if dt in (0, 1) else 1 << 20
    return lib.quat_cumprod_bwd_ex(ptr(q), ptr(init), ptr(dcum), ptr(ckpt), ckb, ptr(dq), ptr(di), *shape, dt,
                                   ptr(ws), wsb, None, opts)


def test_null_pointers(lib):
    assert fwd(lib, q=None) == E_NULL
    assert fwd(lib, init=None) == E_NULL
    assert fwd(lib, cum=None) == E_NULL
    assert bwd(lib, q=None) == E_NULL
    assert bwd(lib, init=None) == E_NULL
    assert bwd(lib, dcum=None) == E_NULL
    assert fwd(lib, ws=None) == E_WS
    assert bwd(lib, ws=None) == E_WS


def test_bwd_without_outputs_is_a_noop(lib):
    # Both gradients unwanted (untracked inputs): returns before any HIP call.
    assert bwd(lib, dq=None, di=None) == OK
    assert bwd(lib, dq=None, di=None, ws=None) == OK


def test_shapes_and_dtype(lib):
    for shape in [(0, 100, 3, 4), (2, 0, 3, 4), (2, 100, 0, 4), (2, 100, 3, -1)]:
        assert fwd(lib, shape=shape, wsb=1 << 30) == E_SHAPE
        assert bwd(lib, shape=shape, wsb=1 << 30) == E_SHAPE
    assert fwd(lib, dt=2) == E_DTYPE
    assert bwd(lib, dt=-1) == E_DTYPE


def test_alignment(lib):
    odd = ctypes.c_void_p(0x10_0000_0000 * 9 + 8)   # 8-byte aligned only
    assert fwd(lib, q=odd) == E_ALIGN
    assert fwd(lib, cum=odd) == E_ALIGN
    assert bwd(lib, dq=odd) == E_ALIGN
    assert bwd(lib, di=odd) == E_ALIGN
    # bfloat16 tensors need only 8-byte alignment; the workspace needs 16.
    wsb16 = lib.quat_cumprod_workspace_bytes(*SHAPE, 1)
    assert fwd(lib, q=odd, dt=1, wsb=wsb16, ws=ctypes.c_void_p(0x10_0000_0000 * 10 + 8)) == E_ALIGN
    assert fwd(lib, ckpt=odd, ckb=1 << 20) == E_ALIGN


def test_workspace_and_ckpt_sizes(lib):
    need = lib.quat_cumprod_workspace_bytes(*SHAPE, 0)
    assert fwd(lib, wsb=need - 1) == E_WS
    assert bwd(lib, wsb=need - 256) == E_WS
    ck = lib.quat_cumprod_ckpt_bytes(*SHAPE, 0)
    assert fwd(lib, ckpt=8, ckb=ck - 1) == E_WS
    assert bwd(lib, ckpt=8, ckb=ck - 1) == E_WS


def test_aliasing(lib):
    assert fwd(lib, cum=1) == E_ALIAS             # cum is q
    assert fwd(lib, ckpt=2, ckb=1 << 30) == E_ALIAS   # ckpt over init
    assert fwd(lib, ws=3) == E_ALIAS              # workspace over cum
    inside_q = ctypes.c_void_p(0x10_0000_0000 + 4096)
    assert fwd(lib, cum=inside_q) == E_ALIAS      # partial overlap
    assert bwd(lib, dq=3) == E_ALIAS              # d_q over d_cum
    assert bwd(lib, di=6) == E_ALIAS              # d_init over d_q
    assert bwd(lib, dq=8, ckpt=8, ckb=1 << 30) == E_ALIAS   # d_q over ckpt


def test_options(lib):
    o = capi.QcOptions()
    o.path = 4
    assert fwd(lib, opts=ctypes.byref(o)) == E_OPT
    o.path = 0
    o.lookback = 3
    assert bwd(lib, opts=ctypes.byref(o)) == E_OPT
    o.lookback = 0
    o.leaves = 3
    assert bwd(lib, opts=ctypes.byref(o)) == E_OPT
    o.leaves = 0
    o.saved = 2
    assert fwd(lib, opts=ctypes.byref(o)) == E_OPT
    assert bwd(lib, opts=ctypes.byref(o)) == E_OPT
    o.saved = 0
    o.reserved[2] = 1
    assert bwd(lib, opts=ctypes.byref(o)) == E_OPT


def test_final_carry_state(lib):
    """QC_SAVED_FINAL: the ckpt holds one internal-precision quaternion per
    column whatever s, is size-checked as such, and is refused by the
    reduce-then-scan backward (which has no pair carries)."""
    o = capi.QcOptions()
    o.saved = 1
    opt = ctypes.byref(o)
    for (b, s, h, j) in [(1, 1, 1, 1), (8, 4096, 32, 32), (1, 262144, 2, 8), (2, 65, 3, 5)]:
        assert lib.quat_cumprod_ckpt_bytes_ex(b, s, h, j, 0, opt) == b * h * j * 32
        assert lib.quat_cumprod_ckpt_bytes_ex(b, s, h, j, 1, opt) == b * h * j * 16
        assert lib.quat_cumprod_ckpt_bytes_ex(b, s, h, j, 0, None) == lib.quat_cumprod_ckpt_bytes(b, s, h, j, 0)
    assert lib.quat_cumprod_ckpt_bytes_ex(0, 1, 1, 1, 0, opt) == 0
    bad = capi.QcOptions()
    bad.saved = 5
    assert lib.quat_cumprod_ckpt_bytes_ex(1, 1, 1, 1, 0, ctypes.byref(bad)) == 0
    fin = lib.quat_cumprod_ckpt_bytes_ex(*SHAPE, 0, opt)
    assert fin < lib.quat_cumprod_ckpt_bytes(*SHAPE, 0)
    assert fwd(lib, ckpt=8, ckb=fin - 1, opts=opt) == E_WS
    assert bwd(lib, ckpt=8, ckb=fin - 1, opts=opt) == E_WS
    o.path = 3
    assert bwd(lib, ckpt=8, ckb=fin, opts=opt) == E_OPT


def test_binding_tags_ckpt_kind():
    """The binding sizes a ckpt by its kind and refuses a kind that
    disagrees with the buffer's tag (host-side checks only)."""
    import torch
    ck = torch.empty(0)
    ck.qc_saved = "final"
    assert capi._saved_kind(ck, None) == "final"
    assert capi._saved_kind(ck, "final") == "final"
    assert capi._saved_kind(None, None) == "boundary"
    assert capi._saved_kind(torch.empty(0), "final") == "final"
    with pytest.raises(ValueError, match="holds"):
        capi._saved_kind(ck, "boundary")
    with pytest.raises(ValueError):
        capi._saved_kind(None, "everything")


def test_workspace_helpers_validate(lib):
    assert lib.quat_cumprod_workspace_init(None, 1024, None) == E_NULL
    assert lib.quat_cumprod_workspace_init(ctypes.c_void_p(0x1008), 1024, None) == E_ALIGN
    assert lib.quat_cumprod_workspace_init(P(1), 16, None) == E_WS
    out = ctypes.c_int32(0)
    assert lib.quat_cumprod_workspace_status(None, 1024, None, 0, ctypes.byref(out)) == E_NULL
    assert lib.quat_cumprod_workspace_status(P(1), 1024, None, 0, None) == E_NULL


def test_binding_fails_loudly_without_library(tmp_path):
    with pytest.raises(RuntimeError, match="not built"):
        capi.load(str(tmp_path / "missing.so"))


def test_cpu_tensors_are_refused_not_computed():
    """There is no CPU path: host tensors raise before any library call."""
    import torch
    from quaternion_cumprod_autodiff_amd.autograd import quat_cumprod
    q = torch.zeros(1, 4, 1, 1, 4)
    init = torch.zeros(1, 1, 1, 4)
    with pytest.raises(ValueError, match="GPU"):
        quat_cumprod(q, init)
    with pytest.raises(ValueError, match="GPU"):
        capi.quat_cumprod_fwd(q, init)
    with pytest.raises(ValueError, match="GPU"):
        capi.quat_cumprod_bwd(q, init, q)


def test_scan_node_refuses_host_tensors():
    """The generic scan's autograd node has no CPU path: host tensors are
    refused before anything runs."""
    import torch
    from quaternion_cumprod_autodiff_amd.autograd import scan
    xs = torch.zeros((1, 4, 2, 4), requires_grad=True)
    init = torch.zeros((1, 2, 4))
    with pytest.raises(ValueError, match="GPU only"):
        scan("quat", xs, init)
    with pytest.raises(ValueError):
        scan("quat", xs, init, num_checkpoints=-1)


def test_gdn2_sizes_and_validation(lib):
    """Gated DeltaNet-2 entry points: documented buffer sizes, and bad
    arguments refused before any HIP call (fake device pointers)."""
    # heads x chunks x D x LP floats, LP = L = 3 rounded up to 16
    assert lib.gdn2_boundary_bytes(1, 2, 5, 3, 4, 2) == 2 * 3 * 4 * 16 * 4
    assert lib.gdn2_scratch_bytes(1, 2, 5, 3, 4, 2) == 2 * 2 * 4 * 16 * 4       # heads x chunk x D x LP
    assert lib.gdn2_scratch_bytes(1, 2, 5, 3, 4, 64) == 2 * 5 * 4 * 16 * 4      # a chunk longer than T
    assert lib.gdn2_boundary_bytes(1, 1, 4, 33, 2, 4) == 1 * 1 * 2 * 64 * 4     # L = 33 pads to 64
    assert lib.gdn2_boundary_bytes(1, 1, 1, 65, 4, 1) == 0                      # L > 64
    assert lib.gdn2_boundary_bytes(1, 1, 1, 4, 1025, 1) == 0                    # D > 1024
    # L = 3 (16 padded rows, 4 lanes per column): backward blocks of 8 waves x 16 columns.  D = 100
    # fits one block, and the scratch holds the states alone; D = 200 takes two blocks per head, and
    # the scratch also holds their shares of the four latent-vector cotangents, [heads, T, blocks, 4,
    # L], after the states (256-byte aligned).  L = 40 (64 padded rows, 8 lanes): 64-column blocks.
    assert lib.gdn2_scratch_bytes(1, 2, 5, 3, 100, 2) == 2 * 2 * 100 * 16 * 4
    states = 2 * 2 * 200 * 16 * 4
    assert lib.gdn2_scratch_bytes(1, 2, 5, 3, 200, 2) == (states + 255) // 256 * 256 + 2 * 5 * 2 * 4 * 3 * 4
    states = 1 * 3 * 100 * 64 * 4
    assert lib.gdn2_scratch_bytes(1, 1, 7, 40, 100, 3) == (states + 255) // 256 * 256 + 1 * 7 * 2 * 4 * 40 * 4
    assert lib.gdn2_boundary_bytes(1, 1, 1, 4, 4, 0) == 0
    G = 1 << 30
    A = 1 << 44
    ins = [A + i * G for i in range(7)]
    f = lib.gdn2_fwd
    assert f(*ins, A + 7 * G, None, None, 0, 1, 8, 4, 4, 2, None) == E_SHAPE
    assert f(*ins, A + 7 * G, None, None, 1, 1, 8, 65, 4, 2, None) == E_SHAPE
    assert f(*ins[:6], None, A + 7 * G, None, None, 1, 1, 8, 4, 4, 2, None) == E_NULL
    assert f(*ins, None, None, None, 1, 1, 8, 4, 4, 2, None) == E_NULL
    assert f(*ins, A + 7 * G + 2, None, None, 1, 1, 8, 4, 4, 2, None) == E_ALIGN
    assert f(*ins, A + 64, None, None, 1, 1, 8, 4, 4, 2, None) == E_ALIAS        # context over query
    b = lib.gdn2_bwd
    outs = [A + (10 + i) * G for i in range(7)]
    base = ins[:6] + [A + 8 * G, A + 9 * G, None] + outs
    assert b(*base, A + 20 * G, 0, 1, 1, 8, 4, 4, 2, None) == E_WS               # scratch too small
    assert b(*base, A + 20 * G + 4, 1 << 20, 1, 1, 8, 4, 4, 2, None) == E_ALIGN   # scratch not 16-byte aligned
    assert b(*base, None, 1 << 20, 1, 1, 8, 4, 4, 2, None) == E_WS
    assert b(*(ins[:6] + [None, A + 9 * G, None] + outs), A + 20 * G, 1 << 20, 1, 1, 8, 4, 4, 2, None) == E_NULL
    assert b(*(ins[:6] + [A + 8 * G, A + 9 * G, None] + [None] * 7), None, 0, 1, 1, 8, 4, 4, 2, None) == OK
    assert b(*(base[:9] + [A + 64] + outs[1:]), A + 20 * G, 1 << 20, 1, 1, 8, 4, 4, 2, None) == E_ALIAS


def test_gdn2_node_refuses_host_tensors():
    import torch
    from quaternion_cumprod_autodiff_amd.autograd import gated_deltanet2
    q = torch.zeros((1, 1, 3, 4), requires_grad=True)
    v = torch.zeros((1, 1, 3, 5))
    with pytest.raises(ValueError, match="GPU only"):
        gated_deltanet2(q, q, v, q, v, q, torch.zeros((1, 1, 4, 5)))


def test_stream_copy_validates_before_any_hip_call(lib):
    a, b = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 31)
    assert lib.qc_stream_copy(a, b, 0, 8, None) == OK                 # empty: no-op
    assert lib.qc_stream_copy(None, b, 64, 8, None) == E_NULL
    assert lib.qc_stream_copy(a, None, 64, 8, None) == E_NULL
    assert lib.qc_stream_copy(ctypes.c_void_p((1 << 30) + 4), b, 64, 8, None) == E_ALIGN
    assert lib.qc_stream_copy(a, b, 60, 8, None) == E_ALIGN
    assert lib.qc_stream_copy(a, ctypes.c_void_p((1 << 30) + 32), 64, 8, None) == E_ALIAS
    assert lib.qc_stream_copy(a, b, 64, 0, None) == E_OPT
    assert lib.qc_stream_copy(a, b, 64, 65, None) == E_OPT


def test_noalloc_validates_before_any_hip_call(lib):
    """Shapes beyond the fixed 64 MiB array, bad shapes, a misaligned or
    aliasing status word and a call with no output are all decided on the
    host (fake device pointers are never dereferenced)."""
    q, init, d = ctypes.c_void_p(1 << 30), ctypes.c_void_p(1 << 31), ctypes.c_void_p(1 << 32)
    dq, di = ctypes.c_void_p(1 << 33), ctypes.c_void_p(1 << 34)
    f = lib.quat_cumprod_bwd_noalloc
    assert f(q, init, d, None, 0, dq, di, 64, 4096, 32, 32, 0, None, None) == E_WS     # 288 MiB of workspace
    assert f(q, init, d, None, 0, dq, di, 0, 8, 1, 1, 0, None, None) == E_SHAPE
    assert f(q, init, d, None, 0, dq, di, 1, 8, 1, 1, 5, None, None) == E_DTYPE
    assert f(q, init, d, None, 0, None, None, 1, 8, 1, 1, 0, None, None) == OK          # nothing wanted
    assert f(q, init, d, None, 0, dq, di, 1, 8, 1, 1, 0, ctypes.c_void_p((1 << 35) + 2), None) == E_ALIGN
    assert f(q, init, d, None, 0, dq, di, 1, 8, 1, 1, 0, ctypes.c_void_p((1 << 33) + 16), None) == E_ALIAS
