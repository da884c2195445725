"""float64 CPU oracle for the quaternion cumulative-product scan (ctypes loader).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may use this package; the device library and
its Python binding never import it.

The arithmetic lives in ``quat_oracle.c`` (plain C, float64, sequential over
the sequence axis, OpenMP over independent columns).  Definitions follow the
burn-mamba source page "burn_mamba/mamba3/quat_scan/backward.rs", module
documentation, section "Gradient math".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "quat_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile quat_oracle.c with gcc into oracle/liboracle.so."""
    global _lib
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
        _lib = None
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        i64 = ctypes.c_int64
        lib.oracle_qmul.argtypes = [dp, dp, dp]
        lib.oracle_qmul.restype = None
        lib.oracle_threads.argtypes = [ctypes.c_int]
        lib.oracle_threads.restype = ctypes.c_int
        lib.oracle_fwd.argtypes = [dp, dp, dp, i64, i64, i64, ctypes.c_int]
        lib.oracle_fwd.restype = None
        lib.oracle_bwd.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64, ctypes.c_int]
        lib.oracle_bwd.restype = ctypes.c_int
        lib.oracle_bwd_closed_form.argtypes = [dp, dp, dp, dp, dp, i64, i64, i64,
                                               ctypes.c_int, ctypes.c_int]
        lib.oracle_bwd_closed_form.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dims(q: np.ndarray, init: np.ndarray):
    if q.ndim < 3 or q.shape[-1] != 4:
        raise ValueError("q must be [b, s, ..., 4]")
    b, s = q.shape[0], q.shape[1]
    m = int(np.prod(q.shape[2:-1], dtype=np.int64))
    if init.shape != (b,) + q.shape[2:]:
        raise ValueError(f"init must be {(b,) + q.shape[2:]}, got {init.shape}")
    return b, s, m


def threads(n: int = 0) -> int:
    """Threads an oracle call with ``nthreads=n`` uses (0 = OpenMP default)."""
    return _load().oracle_threads(n)


def qmul(a, b) -> np.ndarray:
    """Hamilton product of two single quaternions (w, x, y, z)."""
    a, b = _f64(a), _f64(b)
    out = np.empty(4)
    _load().oracle_qmul(_ptr(a), _ptr(b), _ptr(out))
    return out


def fwd(q, init, nthreads: int = 0) -> np.ndarray:
    """cum[t] = q_t (x) cum[t-1], cum[-1] = init, over axis 1 of q."""
    q, init = _f64(q), _f64(init)
    b, s, m = _dims(q, init)
    cum = np.empty_like(q)
    _load().oracle_fwd(_ptr(q), _ptr(init), _ptr(cum), b, s, m, nthreads)
    return cum


def bwd(q, init, d_cum, nthreads: int = 0, want_dq: bool = True, want_dinit: bool = True):
    """Exact VJP (reverse recurrence).  Returns (d_q, d_init); unwanted ones are None."""
    q, init, d_cum = _f64(q), _f64(init), _f64(d_cum)
    b, s, m = _dims(q, init)
    if d_cum.shape != q.shape:
        raise ValueError("d_cum must have q's shape")
    d_q = np.empty_like(q) if want_dq else None
    d_init = np.empty_like(init) if want_dinit else None
    rc = _load().oracle_bwd(_ptr(q), _ptr(init), _ptr(d_cum), _ptr(d_q), _ptr(d_init),
                            b, s, m, nthreads)
    if rc != 0:
        raise MemoryError("oracle_bwd could not allocate scratch")
    return d_q, d_init


def bwd_closed_form(q, init, d_cum, normalise: bool, nthreads: int = 0):
    """The page's closed-form VJP; ``normalise`` divides G[t] by |P_t|^2."""
    q, init, d_cum = _f64(q), _f64(init), _f64(d_cum)
    b, s, m = _dims(q, init)
    d_q = np.empty_like(q)
    d_init = np.empty_like(init)
    rc = _load().oracle_bwd_closed_form(_ptr(q), _ptr(init), _ptr(d_cum), _ptr(d_q),
                                        _ptr(d_init), b, s, m, int(normalise), nthreads)
    if rc != 0:
        raise MemoryError("oracle_bwd_closed_form could not allocate scratch")
    return d_q, d_init


# Generic scan (bodies "add" and "quat") and its VJP: plain numpy, float64.
from .generic_scan import BODIES as SCAN_BODIES, scan_bwd, scan_fwd  # noqa: E402

# Gated DeltaNet-2 recurrence and its VJP: plain numpy, float64.
from .gdn2 import gdn2_bwd, gdn2_fwd, gdn2_states  # noqa: E402,F401
