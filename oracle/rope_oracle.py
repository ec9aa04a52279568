"""CPU oracle of RMSNorm + rotary position embedding -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module.  The HIP library never calls it and shares no code with it.

The op (ORT PR #33997 "Support FP16 KV cache and FP16 query/key in
DynamicSparseAttention<BFloat16> and FP32 rotary cache / FP16 output in
RMSNormRotary", Description item 1) normalises each query/key head vector
and rotates it by its token position, in exact arithmetic with no
intermediate 16-bit rounding, then rounds once to the FP16 (or BF16) output;
the rotary cos/sin tables are kept in FP32.  The pages quote the effect of
that single rounding: Q/K relative RMSE 0.0207% (vs 0.1954% with BF16
intermediates).

Readings where the pages are silent:
  * RMSNorm over the D values of one head vector x with a per-dim weight g:
        y_d = g_d * x_d / sqrt(mean_d(x_d^2) + eps);
  * rotary pairs (d, d + D/2) ("rotate half") by default, (2i, 2i + 1) when
    `interleaved`; for pair i with angle table entries c = cos[p, i] and
    s = sin[p, i] (tables [max_pos, D/2], FP32, supplied by the caller):
        out_a = y_a * c - y_b * s,   out_b = y_b * c + y_a * s;
  * the rotation covers all D dims; the position of token s of sequence b is
    p = kv_len[b] - S + s, as for the attention queries.
Computed in FP64 from the exact input values; the result is returned
unrounded (callers round once to the output dtype).

Pins (tests/test_rope_oracle.py): torch's rms_norm on the identity rotation,
pair-norm preservation, the relative-position property of the dot product,
a two-dimensional closed form, interleaved/rotate-half equivalence under a
permutation, scale invariance, and the pages' 0.0207% / 0.1954% rounding
figures reproduced in kind.
"""
import numpy as np


def _f64(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.dtype.is_floating_point:
            x = x.double()
        return x.numpy().astype(np.float64, copy=False)
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, gamma, eps):
    """y = gamma * x / sqrt(mean(x^2) + eps) over the last axis (FP64)."""
    x = _f64(x)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return _f64(gamma) * x / np.sqrt(ms + float(eps))


def pair_index(D, interleaved):
    """(a, b) index arrays of the rotated pairs, pair i uses table column i."""
    i = np.arange(D // 2)
    if interleaved:
        return 2 * i, 2 * i + 1
    return i, i + D // 2


def rotate(y, cos_row, sin_row, interleaved=False):
    """Rotate every pair of y (last axis D) by the angles of one position."""
    y = _f64(y)
    D = y.shape[-1]
    a, b = pair_index(D, interleaved)
    c, s = _f64(cos_row), _f64(sin_row)
    out = np.empty_like(y)
    out[..., a] = y[..., a] * c - y[..., b] * s
    out[..., b] = y[..., b] * c + y[..., a] * s
    return out


def rmsnorm_rope(x, gamma, cos_cache, sin_cache, kv_len, eps, interleaved=False):
    """x [B, S, H, D] -> unrounded FP64 [B, S, H, D]; rows whose position lies
    outside the tables are NaN (the kernel leaves them unwritten)."""
    x = _f64(x)
    B, S, H, D = x.shape
    cos_cache, sin_cache = _f64(cos_cache), _f64(sin_cache)
    out = np.full(x.shape, np.nan)
    for b in range(B):
        for s in range(S):
            p = int(kv_len[b]) - S + s
            if 0 <= p < cos_cache.shape[0]:
                out[b, s] = rotate(rms_norm(x[b, s], gamma, eps), cos_cache[p], sin_cache[p],
                                   interleaved)
    return out
