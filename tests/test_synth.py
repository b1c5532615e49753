"""Host-side checks of the seeded input generator (CPU)."""
import numpy as np

import synth
from synth import recipes


def test_deterministic_and_counter_addressed():
    a = synth.normal_bf16(7, "w", (64, 96))
    b = synth.normal_bf16(7, "w", (64, 96))
    np.testing.assert_array_equal(a, b)
    # element i of a tensor only depends on (seed, name, i): a window with an offset
    # reproduces the same values
    c = synth.normal_bf16(7, "w", (10, 96), offset=5 * 96)
    np.testing.assert_array_equal(c, a[5:15])
    assert not np.array_equal(a, synth.normal_bf16(8, "w", (64, 96)))
    assert not np.array_equal(a, synth.normal_bf16(7, "w2", (64, 96)))


def test_strided_writes_place_logical_values():
    lg = synth.normal_bf16(3, "kv.0.v", (2, 5, 8))
    out = np.zeros((2, 8, 16), np.uint16)  # transposed, padded [b][col][row]
    synth.normal_bf16_strided_host(3, "kv.0.v", out, (2, 5, 8), (8 * 16, 1, 16))
    np.testing.assert_array_equal(out[:, :, :5], lg.transpose(0, 2, 1))
    assert np.all(out[:, :, 5:] == 0)


def test_normal_moments_and_support():
    x = synth.bf16_to_f32(synth.normal_bf16(1, "x", (1 << 20,))).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    assert np.abs(x).max() <= 6.0
    w = synth.bf16_to_f32(synth.normal_bf16(1, "n", (1 << 16,), 1.0, 0.05)).astype(np.float64)
    assert abs(w.mean() - 1.0) < 2e-3 and abs(w.std() - 0.05) < 2e-3


def test_uniform_ids_range():
    ids = synth.uniform_i32(2, "input.ids", (4, 2048), 0, 151936)
    assert ids.min() >= 0 and ids.max() < 151936
    counts = np.bincount(ids.ravel() * 16 // 151936, minlength=16)
    assert counts.min() > 0.8 * counts.mean()


def test_bf16_round_trip():
    x = np.array([1.0, -2.5, 3.14159, 1e-3, 65504.0], np.float32)
    b = synth.f32_to_bf16(x)
    y = synth.bf16_to_f32(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)
    np.testing.assert_array_equal(synth.f32_to_bf16(y), b)


def test_layer_recipe_shapes():
    cfg = recipes.QWEN3_0P6B
    specs = recipes.layer_specs(cfg, 3)
    shapes = {f: s for f, _, s, _, _ in specs}
    assert shapes["q"] == (2048, 1024) and shapes["k"] == (1024, 1024)
    assert shapes["o"] == (1024, 2048) and shapes["down"] == (1024, 3072)
    assert recipes.param_count(cfg) == 596049920
