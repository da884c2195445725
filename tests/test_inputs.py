"""The seeded input generator (CPU): chunked draws equal one-shot draws, the
recipes produce what they state, and the bf16 rounding is round-to-nearest-even
(checked against torch's own float32 -> bfloat16 conversion)."""
import numpy as np
import torch

from quaternion_cumprod_autodiff_amd.inputs import (CONFIGS, bf16_bits_to_f32, f32_to_bf16_bits, make_config,
                                                    make_inputs)

B, S, H, J = 1, 300, 30, 30          # 270,000 quaternions: more than one 2^18 generation chunk


def _unitise(v):
    return v / np.sqrt(np.sum(v * v, axis=-1, keepdims=True))


def _one_shot(recipe, seed):
    rng = np.random.default_rng(seed)
    n = B * S * H * J
    if recipe == "unit":
        q = _unitise(rng.standard_normal((n, 4)))
    else:
        theta = rng.uniform(0.0, 0.05, size=n)
        u = _unitise(rng.standard_normal((n, 3)))
        q = np.concatenate([np.cos(0.5 * theta)[:, None], np.sin(0.5 * theta)[:, None] * u], axis=1)
    init = _unitise(rng.standard_normal((B * H * J, 4)))
    d = rng.standard_normal((n, 4))
    return q, init, d


def test_chunked_draws_equal_one_shot_draws():
    for recipe in ("unit", "drift"):
        inp = make_inputs(B, S, H, J, recipe, "f32", seed=11)
        q, init, d = _one_shot(recipe, 11)
        np.testing.assert_array_equal(inp.q.reshape(-1, 4), q.astype(np.float32))
        np.testing.assert_array_equal(inp.init.reshape(-1, 4), init.astype(np.float32))
        np.testing.assert_array_equal(inp.d_cum.reshape(-1, 4), d.astype(np.float32))


def test_float64_copies_hold_exactly_the_stored_values():
    for dtype in ("f32", "bf16"):
        inp = make_inputs(2, 50, 3, 5, "unit", dtype, seed=3)
        for st, wide in ((inp.q, inp.q64), (inp.init, inp.init64), (inp.d_cum, inp.d_cum64)):
            widened = st.astype(np.float64) if dtype == "f32" else bf16_bits_to_f32(st).astype(np.float64)
            np.testing.assert_array_equal(widened, wide)


def test_recipes():
    unit = make_inputs(2, 400, 4, 4, "unit", "f32", seed=5)
    assert np.abs(np.linalg.norm(unit.q64, axis=-1) - 1).max() < 1e-6
    assert np.abs(np.linalg.norm(unit.init64, axis=-1) - 1).max() < 1e-6
    drift = make_inputs(2, 400, 4, 4, "drift", "f32", seed=5)
    half_angle = np.arccos(np.clip(drift.q64[..., 0], -1, 1))
    assert half_angle.max() <= 0.025 + 1e-6 and drift.q64[..., 0].min() > 0.999
    scaled = make_inputs(2, 400, 4, 4, "scaled", "f32", seed=5)
    norms = np.linalg.norm(scaled.q64, axis=-1)
    assert 0.5 - 1e-6 <= norms.min() and norms.max() <= 1.5 + 1e-6 and norms.std() > 0.2
    d = unit.d_cum64
    assert abs(d.mean()) < 0.05 and abs(d.std() - 1) < 0.05


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(9)
    x = np.concatenate([
        rng.standard_normal(10000).astype(np.float32) * np.float32(10.0) ** rng.integers(-20, 20, 10000),
        np.float32([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 3.0e38, -0.0, 0.0, 1e-40]),
    ]).astype(np.float32)
    ours = f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(ours, ref)
    assert f32_to_bf16_bits(np.float32([np.nan]))[0] & 0x7FC0 == 0x7FC0


def test_named_workloads():
    assert set(CONFIGS) == {"tiny", "medium", "headline", "longseq", "drift_f32", "drift_bf16"}
    assert CONFIGS["headline"] == (8, 4096, 32, 32, "unit", "f32")
    tiny = make_config("tiny")
    assert tiny.q.shape == (1, 256, 4, 8, 4) and tiny.init.shape == (1, 4, 8, 4)
