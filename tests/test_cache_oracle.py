"""Pins of the KV-cache append oracle (oracle/cache_oracle.py), on the CPU.

The quantiser is checked against an exact-rational brute force whose FP32
steps are rounded by a routine written here from the IEEE definition, and
against properties the quantisation must have whatever its implementation;
planted mistakes at the bottom must each fail some pin.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle.cache_oracle as co


# ------------------------------------------------------------ brute force
def _f32_round(q):
    """Correctly rounded (nearest, ties to even) FP32 value of a rational q."""
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    c = np.float32(float(q))              # within one FP32 ulp of q
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - q)
        if best is None or d < best[0] or (
                d == best[0] and (np.float32(cand).view(np.uint32) & 1) == 0):
            best = (d, cand)
    return np.float32(best[1])


def _rint_half_even(q):
    q = Fraction(q)
    f = q.numerator // q.denominator
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def _brute_quantize(x):
    xs = [Fraction(float(v)) for v in np.asarray(x, dtype=np.float32)]
    amax = max(abs(v) for v in xs)
    if amax == 0:
        return np.zeros(len(xs), np.int8), np.float32(0.0)
    scale = _f32_round(amax / 127)
    codes = []
    for v in xs:
        q = _f32_round(v / Fraction(float(scale)))
        codes.append(max(-127, min(127, _rint_half_even(Fraction(float(q))))))
    return np.array(codes, np.int8), scale


def test_quantizer_matches_exact_rational_brute_force():
    rng = np.random.default_rng(11)
    rows = [rng.standard_normal(16).astype(np.float32) for _ in range(40)]
    rows += [(rng.standard_normal(8) * 1e-30).astype(np.float32),
             (rng.standard_normal(8) * 1e30).astype(np.float32),
             np.array([127, 2.5, 3.5, -2.5, -0.5, 0.5, 1.5, 126.5], np.float32),  # halves
             np.array([0.0, -0.0, 3.0, 0.0], np.float32)]
    # values whose quotient by the scale lies within an FP32 ulp of k + 1/2:
    # there the FP32 quotient decides the code
    s0 = np.float32(0.0137)
    rows.append(np.array([np.float32(127 * float(s0))] +
                         [np.float32((k + 0.5) * float(s0)) for k in range(-126, 126)], np.float32))
    for x in rows:
        c, s = co.quantize_row_int8(x)
        bc, bs = _brute_quantize(x)
        assert s == bs and s.dtype == np.float32, (x, s, bs)
        assert np.array_equal(c, bc), (x, c, bc)


def test_halfway_codes_round_to_even():
    # amax = 127 gives scale exactly 1, so x / scale = x
    c, s = co.quantize_row_int8(np.array([127, 2.5, 3.5, -2.5, -3.5, 0.5], np.float32))
    assert s == 1.0
    assert c.tolist() == [127, 2, 4, -2, -4, 0]


def test_generator_int8_rows_requantize_to_their_codes():
    rng = np.random.default_rng(12)
    for _ in range(200):
        codes = rng.integers(-127, 128, 128).astype(np.int8)
        codes[rng.integers(0, 128)] = 127 * (1 if rng.random() < 0.5 else -1)
        scale = np.float32(rng.uniform(0.005, 0.05))
        x = (codes.astype(np.float64) * float(scale)).astype(np.float32)
        c, s = co.quantize_row_int8(x)
        assert np.array_equal(c, codes)
        ulp = np.spacing(scale)
        assert abs(float(s) - float(scale)) <= 2 * ulp


def test_quantization_error_is_at_most_half_a_step():
    rng = np.random.default_rng(13)
    for _ in range(100):
        x = (rng.standard_normal(128) * rng.uniform(0.01, 100)).astype(np.float32)
        c, s = co.quantize_row_int8(x)
        assert np.abs(c).max() == 127
        err = np.abs(c.astype(np.float64) * float(s) - x.astype(np.float64))
        assert err.max() <= 0.5 * float(s) * (1 + 1e-5)
        assert c.min() >= -127


def test_sign_symmetry_and_power_of_two_scaling():
    rng = np.random.default_rng(14)
    for _ in range(50):
        x = rng.standard_normal(64).astype(np.float32)
        c, s = co.quantize_row_int8(x)
        cn, sn = co.quantize_row_int8(-x)
        assert sn == s and np.array_equal(cn, -c)
        c4, s4 = co.quantize_row_int8(x * np.float32(4.0))
        assert s4 == s * np.float32(4.0) and np.array_equal(c4, c)


def test_all_zero_row_gives_zero_codes_and_zero_scale():
    c, s = co.quantize_row_int8(np.zeros(128, np.float32))
    assert s == 0.0 and not c.any()


def test_rows_quantize_independently_per_token_and_head():
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 2, 16)).astype(np.float32)
    x[1, 0] *= 1000.0
    codes, scales = co.quantize_rows_int8(x)
    for i in range(3):
        for h in range(2):
            c, s = co.quantize_row_int8(x[i, h])
            assert scales[i, h] == s and np.array_equal(codes[i, h], c)


def _append_case(kv_dtype):
    rng = np.random.default_rng(16)
    B, L, H, D, S, Di = 2, 8, 2, 16, 3, 8
    kv_len = [5, 9]                      # second sequence: its last token falls off the cache
    if kv_dtype == "i8":
        kc = rng.integers(-127, 128, (B, L, H, D)).astype(np.int8)
        vc = rng.integers(-127, 128, (B, L, H, D)).astype(np.int8)
        ksc = rng.uniform(0.005, 0.05, (B, L, H)).astype(np.float32)
        vsc = rng.uniform(0.005, 0.05, (B, L, H)).astype(np.float32)
    else:
        kc = rng.standard_normal((B, L, H, D))
        vc = rng.standard_normal((B, L, H, D))
        ksc = vsc = None
    ks = rng.integers(-8, 9, (B, L, Di)).astype(np.float64)
    kn = rng.standard_normal((B, S, H, D)).astype(np.float32)
    vn = rng.standard_normal((B, S, H, D)).astype(np.float32)
    ksn = rng.integers(-8, 9, (B, S, Di)).astype(np.float64)
    return kc, vc, ksc, vsc, ks, kn, vn, ksn, kv_len, S, L


@pytest.mark.parametrize("kv_dtype", ["f16", "bf16", "i8"])
def test_append_writes_exactly_the_new_positions(kv_dtype):
    kc, vc, ksc, vsc, ks, kn, vn, ksn, kv_len, S, L = _append_case(kv_dtype)
    k2, v2, ks2, vs2, st2 = co.cache_append(kc, vc, kn, vn, kv_len, kv_dtype, ksc, vsc, ks, ksn)
    written = {(0, 2), (0, 3), (0, 4), (1, 6), (1, 7)}
    assert set((b, p) for b, _, p in co.append_positions(kv_len, S, L)) == written
    for b in range(2):
        for p in range(L):
            if (b, p) in written:
                s = p - (kv_len[b] - S)
                assert np.array_equal(st2[b, p], ksn[b, s])
                if kv_dtype == "i8":
                    c, sc = co.quantize_rows_int8(kn[b, s])
                    assert np.array_equal(k2[b, p], c) and np.array_equal(ks2[b, p], sc)
                    # dequantised value within half a step of the input
                    err = np.abs(k2[b, p] * ks2[b, p][:, None] - kn[b, s])
                    assert np.all(err <= 0.5 * ks2[b, p][:, None] * (1 + 1e-5))
                else:
                    import torch
                    td = {"f16": torch.float16, "bf16": torch.bfloat16}[kv_dtype]
                    ref = torch.from_numpy(vn[b, s]).to(td).double().numpy()
                    assert np.array_equal(v2[b, p], ref)
                    assert np.all(np.abs(k2[b, p] - kn[b, s]) <= 2.0 ** -8 * np.abs(kn[b, s]))
            else:
                assert np.array_equal(k2[b, p], kc[b, p]) and np.array_equal(v2[b, p], vc[b, p])
                assert np.array_equal(st2[b, p], ks[b, p])
                if kv_dtype == "i8":
                    assert ks2[b, p].tolist() == ksc[b, p].tolist()


# --------------------------------------------------------------- mutants
QUANT_PINS = [test_quantizer_matches_exact_rational_brute_force,
              test_halfway_codes_round_to_even,
              test_generator_int8_rows_requantize_to_their_codes,
              test_quantization_error_is_at_most_half_a_step,
              test_sign_symmetry_and_power_of_two_scaling,
              test_all_zero_row_gives_zero_codes_and_zero_scale]
APPEND_PINS = [lambda: test_append_writes_exactly_the_new_positions("i8"),
               lambda: test_append_writes_exactly_the_new_positions("f16")]

_true_quantize = co.quantize_row_int8
_true_positions = co.append_positions


def _q_scale_128(x):
    x = np.asarray(x, np.float32)
    amax = np.float32(np.abs(x).max())
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    s = np.float32(amax / np.float32(128.0))
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8), s


def _q_truncates(x):
    x = np.asarray(x, np.float32)
    amax = np.float32(np.abs(x).max())
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    s = np.float32(amax / np.float32(127.0))
    return np.clip(np.trunc(x / s), -127, 127).astype(np.int8), s


def _q_half_away(x):
    x = np.asarray(x, np.float32)
    amax = np.float32(np.abs(x).max())
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    s = np.float32(amax / np.float32(127.0))
    q = x / s
    return np.clip(np.sign(q) * np.floor(np.abs(q) + 0.5), -127, 127).astype(np.int8), s


def _q_fp64_division(x):
    x = np.asarray(x, np.float32)
    amax = np.abs(x.astype(np.float64)).max()
    if amax == 0:
        return np.zeros(x.shape, np.int8), np.float32(0)
    s = amax / 127.0
    return np.clip(np.rint(x / s), -127, 127).astype(np.int8), np.float32(s)


def _positions_off_by_one(kv_len, S, L_cap):
    return [(b, s, p + 1) for b, s, p in _true_positions(kv_len, S, L_cap) if p + 1 < L_cap]


MUTANTS = [("quantize_row_int8", _q_scale_128, QUANT_PINS),
           ("quantize_row_int8", _q_truncates, QUANT_PINS),
           ("quantize_row_int8", _q_half_away, QUANT_PINS),
           ("quantize_row_int8", _q_fp64_division, QUANT_PINS),
           ("append_positions", _positions_off_by_one, APPEND_PINS)]


def _caught(pin_list):
    for pin in pin_list:
        try:
            pin()
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name,mutant,pin_list", MUTANTS, ids=[m[1].__name__ for m in MUTANTS])
def test_every_planted_mistake_is_caught(monkeypatch, name, mutant, pin_list):
    monkeypatch.setattr(co, name, mutant)
    assert _caught(pin_list), f"planted mistake {mutant.__name__} passed every pin"
