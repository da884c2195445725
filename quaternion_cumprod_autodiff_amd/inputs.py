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


def _round_to_storage(x64: np.ndarray, dtype: str):
    """Return (storage array, float64 array of the stored values)."""
    x32 = x64.astype(np.float32)  # nearest-even
    if dtype == "f32":
        return x32, x32.astype(np.float64)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x32)
        return bits, bf16_bits_to_f32(bits).astype(np.float64)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def _unit4(rng: np.random.Generator, shape) -> np.ndarray:
    v = rng.standard_normal(tuple(shape) + (4,))
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
    """Draw q, init, d_cum for a [b, s, h, j] problem (see module docstring)."""
    rng = np.random.default_rng(seed)
    shp = (b, s, h, j)
    if recipe in ("unit", "scaled"):
        q = _unit4(rng, shp)
        if recipe == "scaled":
            q *= rng.uniform(0.5, 1.5, size=shp)[..., None]
    elif recipe == "drift":
        theta = rng.uniform(0.0, 0.05, size=shp)
        u = rng.standard_normal(shp + (3,))
        u /= np.sqrt(np.sum(u * u, axis=-1, keepdims=True))
        half = 0.5 * theta
        q = np.empty(shp + (4,), dtype=np.float64)
        q[..., 0] = np.cos(half)
        q[..., 1:] = np.sin(half)[..., None] * u
        del theta, u, half
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    init = _unit4(rng, (b, h, j))
    d_cum = rng.standard_normal(shp + (4,))

    q_st, q64 = _round_to_storage(q, dtype)
    del q
    init_st, init64 = _round_to_storage(init, dtype)
    d_st, d64 = _round_to_storage(d_cum, dtype)
    del d_cum
    if not want_f64:
        q64 = init64 = d64 = None
    return ScanInputs(b, s, h, j, dtype, q_st, init_st, d_st, q64, init64, d64)


def make_config(name: str, seed: int = 0, want_f64: bool = True) -> ScanInputs:
    b, s, h, j, recipe, dtype = CONFIGS[name]
    return make_inputs(b, s, h, j, recipe, dtype, seed, want_f64)
