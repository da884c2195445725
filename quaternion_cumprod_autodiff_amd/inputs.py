"""Seeded synthetic inputs for the quaternion cumulative-product scan.

This module is shared by the tests, the benchmark and the smoke check.  It
draws inputs and rounds them to the storage dtype; it holds none of the scan's
arithmetic (no quaternion products, no scan, no gradient).

Layout (scalar-first quaternions, last axis = (w, x, y, z)):
    q, d_cum : [b, s, h, j, 4]      init : [b, h, j, 4]

Draw order from ``numpy.random.default_rng(seed)`` (PCG64) is always
q, then init, then d_cum.  Values are drawn in float64, normalised in float64
where the recipe says "unit", then rounded to the storage dtype with
round-to-nearest-even.  The float64 arrays returned alongside hold exactly the
rounded values, widened back, so a float64 checker sees the very inputs the
device sees.

Recipes
    unit    q = N(0,1)^4 / |N(0,1)^4|                  (random rotations)
    drift   theta ~ U(0, 0.05) rad, u = N(0,1)^3 / |.|,
            q = (cos(theta/2), sin(theta/2) u)           (near-identity steps)
    scaled  q = unit * U(0.5, 1.5)                       (non-unit steps)
    init    N(0,1)^4 / |.|  (unit) for every recipe
    d_cum   N(0,1) per component
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

# name -> (b, s, h, j, recipe, storage dtype)
CONFIGS = {
    "tiny": (1, 256, 4, 8, "unit", "f32"),
    "medium": (4, 2048, 16, 16, "unit", "f32"),
    "headline": (8, 4096, 32, 32, "unit", "f32"),
    "longseq": (1, 262144, 2, 8, "unit", "f32"),
    "drift_f32": (2, 65536, 16, 16, "drift", "f32"),
    "drift_bf16": (2, 65536, 16, 16, "drift", "bf16"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        rounded[nan] = 0x7FC0
    return rounded


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


_CHUNK = 1 << 18   # quaternions per generation chunk (small temporaries get reused)


def _rounded(x64: np.ndarray, dtype: str):
    """Round float64 values to the storage dtype: (storage values, widened float64)."""
    x32 = x64.astype(np.float32)  # nearest-even
    if dtype == "f32":
        return x32, x32
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bits, bf16_bits_to_f32(bits)
    raise ValueError(f"unknown storage dtype {dtype!r}")


class _Sink:
    """Storage array (+ optional float64 copy) filled chunk by chunk."""

    def __init__(self, n: int, dtype: str, want_f64: bool):
        if dtype not in ("f32", "bf16"):
            raise ValueError(f"unknown storage dtype {dtype!r}")
        self.dtype = dtype
        self.st = np.empty((n, 4), dtype=np.float32 if dtype == "f32" else np.uint16)
        self.f64 = np.empty((n, 4), dtype=np.float64) if want_f64 else None

    def put(self, lo: int, x64: np.ndarray):
        st, wide = _rounded(x64, self.dtype)
        hi = lo + x64.shape[0]
        self.st[lo:hi] = st
        if self.f64 is not None:
            self.f64[lo:hi] = wide


def _normalise(v: np.ndarray) -> np.ndarray:
    v /= np.sqrt(np.sum(v * v, axis=-1, keepdims=True))
    return v


@dataclass
class ScanInputs:
    b: int
    s: int
    h: int
    j: int
    dtype: str          # storage dtype: "f32" or "bf16"
    q: np.ndarray       # storage values (float32, or uint16 bf16 bits)
    init: np.ndarray
    d_cum: np.ndarray
    q64: np.ndarray | None      # float64 copies of the stored values
    init64: np.ndarray | None
    d_cum64: np.ndarray | None


def make_inputs(b: int, s: int, h: int, j: int, recipe: str = "unit",
                dtype: str = "f32", seed: int = 0, want_f64: bool = True) -> ScanInputs:
    """Draw q, init, d_cum for a [b, s, h, j] problem (see module docstring).

    Draws are made in chunks, which yields exactly the same stream as one
    draw of the whole array (numpy Generators are chunk-invariant)."""
    rng = np.random.default_rng(seed)
    n = b * s * h * j
    q = _Sink(n, dtype, want_f64)
    if recipe == "unit":
        for lo in range(0, n, _CHUNK):
            q.put(lo, _normalise(rng.standard_normal((min(n, lo + _CHUNK) - lo, 4))))
    elif recipe == "scaled":
        v = _normalise(rng.standard_normal((n, 4)))
        v *= rng.uniform(0.5, 1.5, size=n)[:, None]
        q.put(0, v)
        del v
    elif recipe == "drift":
        theta = rng.uniform(0.0, 0.05, size=n)
        for lo in range(0, n, _CHUNK):
            hi = min(n, lo + _CHUNK)
            u = _normalise(rng.standard_normal((hi - lo, 3)))
            half = 0.5 * theta[lo:hi]
            v = np.empty((hi - lo, 4))
            v[:, 0] = np.cos(half)
            v[:, 1:] = np.sin(half)[:, None] * u
            q.put(lo, v)
        del theta
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    init = _Sink(b * h * j, dtype, want_f64)
    init.put(0, _normalise(rng.standard_normal((b * h * j, 4))))
    d = _Sink(n, dtype, want_f64)
    for lo in range(0, n, _CHUNK):
        d.put(lo, rng.standard_normal((min(n, lo + _CHUNK) - lo, 4)))

    big, small = (b, s, h, j, 4), (b, h, j, 4)
    f64 = (lambda x, shp: x.f64.reshape(shp) if x.f64 is not None else None)
    return ScanInputs(b, s, h, j, dtype, q.st.reshape(big), init.st.reshape(small), d.st.reshape(big),
                      f64(q, big), f64(init, small), f64(d, big))


def make_config(name: str, seed: int = 0, want_f64: bool = True) -> ScanInputs:
    b, s, h, j, recipe, dtype = CONFIGS[name]
    return make_inputs(b, s, h, j, recipe, dtype, seed, want_f64)


# ---------------------------------------------------------------------------
# Generic scan (include/qc_scan.h): xs, upstream [b, s, m, w], init [b, m, w],
# float32.  Bodies: "add" (w = 1) draws N(0, 1) for xs and init; "quat"
# (w = 4) draws unit quaternions (N(0,1)^4 / |.|, normalised in float32 on the
# device).  upstream ~ N(0, 1).  Drawn on the device from a seeded
# torch.Generator in the order xs, init, upstream, so that launches with
# millions of columns do not wait on the host.

SCAN_WIDTH = {"add": 1, "quat": 4}


def make_generic_scan_inputs_device(body: str, b: int, s: int, m: int, seed: int, device):
    import torch
    w = SCAN_WIDTH[body]
    g = torch.Generator(device=device).manual_seed(seed)
    xs = torch.randn((b, s, m, w), device=device, generator=g)
    init = torch.randn((b, m, w), device=device, generator=g)
    if body == "quat":
        xs /= xs.norm(dim=-1, keepdim=True)
        init /= init.norm(dim=-1, keepdim=True)
    up = torch.randn((b, s, m, w), device=device, generator=g)
    return xs, init, up


# ---------------------------------------------------------------------------
# Gated DeltaNet-2 (include/gdn2.h): query, key, erase, log_decay [B, H, T, L];
# value, write [B, H, T, D]; initial_state [B, H, L, D]; float32.
#
# The burn_gdn page's tests fill every tensor deterministically, element idx
# (row-major) -> ((idx * stride) % modulus) / modulus + offset, with a
# (stride, modulus, offset) per tensor; "output_weight" weights the context
# in their loss.  The random recipe draws from one default_rng(seed) stream in
# the order below: query ~ N(0,1), key ~ N(0,1)/sqrt(L), value ~ N(0,1),
# erase ~ U(0,1), write ~ U(0,1), log_decay ~ U(-1.2, -0.2) (decays 0.30 ..
# 0.82, the span of the page's data), initial_state ~ N(0,1).

GDN2_PAGE_DATA = {
    "query": (3, 23, -0.35), "key": (5, 29, -0.25), "value": (7, 31, -0.2), "erase": (11, 37, 0.1),
    "write": (13, 41, 0.2), "log_decay": (17, 43, -1.2), "initial_state": (19, 47, -0.1),
    "output_weight": (23, 53, -0.3),
}


def _gdn2_shapes(B, H, T, L, D):
    return {"query": (B, H, T, L), "key": (B, H, T, L), "value": (B, H, T, D), "erase": (B, H, T, L),
            "write": (B, H, T, D), "log_decay": (B, H, T, L), "initial_state": (B, H, L, D),
            "output_weight": (B, H, T, D)}


def gdn2_page_tensor(shape, stride: int, modulus: int, offset: float) -> np.ndarray:
    idx = np.arange(int(np.prod(shape)), dtype=np.int64)
    return (((idx * stride) % modulus).astype(np.float32) / np.float32(modulus) + np.float32(offset)).reshape(shape)


def make_gdn2_page_inputs(B: int, H: int, T: int, L: int, D: int) -> dict:
    shapes = _gdn2_shapes(B, H, T, L, D)
    return {n: gdn2_page_tensor(shapes[n], *GDN2_PAGE_DATA[n]) for n in GDN2_PAGE_DATA}


def make_gdn2_random_inputs(B: int, H: int, T: int, L: int, D: int, seed: int = 0) -> dict:
    rng = np.random.default_rng(seed)
    s = _gdn2_shapes(B, H, T, L, D)
    out = {
        "query": rng.standard_normal(s["query"]),
        "key": rng.standard_normal(s["key"]) / np.sqrt(L),
        "value": rng.standard_normal(s["value"]),
        "erase": rng.uniform(0.0, 1.0, s["erase"]),
        "write": rng.uniform(0.0, 1.0, s["write"]),
        "log_decay": rng.uniform(-1.2, -0.2, s["log_decay"]),
        "initial_state": rng.standard_normal(s["initial_state"]),
    }
    return {n: v.astype(np.float32) for n, v in out.items()}
