"""Pins of the RMSNorm + rotary oracle (oracle/rope_oracle.py), on the CPU.

Each pin checks the oracle against something other than itself: torch's
rms_norm, invariants of rotations, a hand closed form, a permutation
identity between the two pairings, and the pages' published rounding
figures.  Planted mistakes at the bottom must each fail some pin.
"""
import math

import numpy as np
import pytest
import torch

import oracle.rope_oracle as ro
from dsa_synth import make_rope_inputs, rope_tables


def _rel_rmse(a, b):
    return float(np.sqrt(np.sum((a - b) ** 2) / np.sum(b ** 2)))


def test_identity_rotation_is_torch_rms_norm():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 128)) * 3.0
    g = rng.uniform(0.5, 1.5, 128)
    D = 128
    cos, sin = np.ones((1, D // 2)), np.zeros((1, D // 2))
    got = ro.rmsnorm_rope(x[None, None], g, cos, sin, [1], 1e-6)[0, 0]
    ref = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(g), eps=1e-6)
    assert np.allclose(got, ref.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("interleaved", [False, True])
def test_rotation_preserves_every_pair_norm(interleaved):
    x = make_rope_inputs(1, 4, 3, 64, 5000, "f32", [4000], seed=2)
    y = ro.rms_norm(x["x"].double().numpy(), x["gamma"].numpy(), 1e-6)
    out = ro.rmsnorm_rope(x["x"], x["gamma"], x["cos"], x["sin"], [4000], 1e-6, interleaved)
    a, b = ro.pair_index(64, interleaved)
    c, s = x["cos"].double().numpy(), x["sin"].double().numpy()
    # cos^2 + sin^2 is 1 only to FP32 table precision
    for t in range(4):
        p = 4000 - 4 + t
        scale = c[p] ** 2 + s[p] ** 2
        n_in = (y[0, t][..., a] ** 2 + y[0, t][..., b] ** 2) * scale
        n_out = out[0, t][..., a] ** 2 + out[0, t][..., b] ** 2
        assert np.allclose(n_out, n_in, rtol=1e-12)


def test_dot_product_depends_only_on_relative_position():
    D = 64
    cos, sin = rope_tables(4096, D, base=1.0e4)
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(D), rng.standard_normal(D)
    g = np.ones(D)
    def at(v, p):
        return ro.rotate(ro.rms_norm(v, g, 0.0), cos[p], sin[p])
    d1 = at(q, 300) @ at(k, 100)
    d2 = at(q, 1300) @ at(k, 1100)
    d3 = at(q, 300) @ at(k, 200)
    assert abs(d1 - d2) < 1e-4 * abs(d1) + 1e-5        # tables are FP32
    assert abs(d1 - d3) > 1e-3


def test_two_dimensional_closed_form():
    a, b, p, th = 0.75, -2.0, 7, 0.3
    eps = 0.01
    cos = np.array([[math.cos(i * th)] for i in range(10)])
    sin = np.array([[math.sin(i * th)] for i in range(10)])
    r = 1.0 / math.sqrt((a * a + b * b) / 2 + eps)
    y0, y1 = 1.5 * a * r, 0.5 * b * r                   # gamma = (1.5, 0.5)
    want = [y0 * math.cos(p * th) - y1 * math.sin(p * th),
            y1 * math.cos(p * th) + y0 * math.sin(p * th)]
    got = ro.rmsnorm_rope(np.array([[[[a, b]]]]), [1.5, 0.5], cos, sin, [p + 1], eps)[0, 0, 0]
    assert np.allclose(got, want, rtol=1e-14)


def test_interleaved_equals_rotate_half_under_a_permutation():
    D = 32
    rng = np.random.default_rng(4)
    x = rng.standard_normal(D)
    g = rng.uniform(0.5, 1.5, D)
    cos, sin = rope_tables(100, D)
    perm = np.concatenate([np.arange(0, D, 2), np.arange(1, D, 2)])   # (2i, 2i+1) -> (i, i+D/2)
    inter = ro.rotate(ro.rms_norm(x, g, 1e-6), cos[37], sin[37], interleaved=True)
    half = ro.rotate(ro.rms_norm(x[perm], g[perm], 1e-6), cos[37], sin[37], interleaved=False)
    assert np.allclose(inter[perm], half, rtol=1e-14, atol=1e-15)


def test_norm_is_scale_invariant_without_eps():
    rng = np.random.default_rng(5)
    x = rng.standard_normal(64)
    g = rng.uniform(0.5, 1.5, 64)
    assert np.allclose(ro.rms_norm(1000.0 * x, g, 0.0), ro.rms_norm(x, g, 0.0), rtol=1e-13)
    y = ro.rms_norm(x, np.ones(64), 0.0)
    assert abs(np.mean(y * y) - 1.0) < 1e-13


def test_rows_outside_the_tables_are_not_produced():
    x = make_rope_inputs(2, 3, 1, 64, 16, "f32", [16, 18], seed=6)
    out = ro.rmsnorm_rope(x["x"], x["gamma"], x["cos"], x["sin"], [16, 18], 1e-6)
    assert np.all(np.isfinite(out[0]))
    assert np.all(np.isfinite(out[1, 0])) and np.all(np.isnan(out[1, 1:]))   # positions 16, 17


def test_single_fp16_rounding_matches_the_pages_relative_rmse():
    # The pages: exact-FP32 RMSNorm + RoPE with FP16 output has Q/K relative
    # RMSE 0.0207%; rounding once to FP16 gives that figure.
    x = make_rope_inputs(2, 16, 8, 128, 40000, "bf16", [32768, 40000], seed=7)
    ref = ro.rmsnorm_rope(x["x"], x["gamma"], x["cos"], x["sin"], [32768, 40000], 1e-6)
    f16 = torch.from_numpy(ref).half().double().numpy()
    assert 0.9 * 2.07e-4 <= _rel_rmse(f16, ref) <= 1.1 * 2.07e-4


# --------------------------------------------------------------- mutants
PINS = [test_identity_rotation_is_torch_rms_norm,
        lambda: test_rotation_preserves_every_pair_norm(False),
        lambda: test_rotation_preserves_every_pair_norm(True),
        test_dot_product_depends_only_on_relative_position,
        test_two_dimensional_closed_form,
        test_interleaved_equals_rotate_half_under_a_permutation,
        test_norm_is_scale_invariant_without_eps,
        test_single_fp16_rounding_matches_the_pages_relative_rmse]

_rms, _rot, _pairs = ro.rms_norm, ro.rotate, ro.pair_index


def _rms_eps_outside(x, gamma, eps):
    x = ro._f64(x)
    return ro._f64(gamma) * x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + float(eps))


def _rms_sum_not_mean(x, gamma, eps):
    x = ro._f64(x)
    return ro._f64(gamma) * x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + float(eps))


def _rot_sign_flipped(y, cos_row, sin_row, interleaved=False):
    return _rot(y, cos_row, -ro._f64(sin_row), interleaved)


def _pairs_adjacent_always(D, interleaved):
    return _pairs(D, True)


def _rot_wrong_pairing(y, cos_row, sin_row, interleaved=False):
    return _rot(y, cos_row, sin_row, not interleaved)


MUTANTS = [("rms_norm", _rms_eps_outside), ("rms_norm", _rms_sum_not_mean),
           ("rotate", _rot_sign_flipped), ("pair_index", _pairs_adjacent_always),
           ("rotate", _rot_wrong_pairing)]


def _caught():
    for pin in PINS:
        try:
            pin()
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name,mutant", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_every_planted_mistake_is_caught(monkeypatch, name, mutant):
    monkeypatch.setattr(ro, name, mutant)
    assert _caught(), f"planted mistake {mutant.__name__} passed every pin"
