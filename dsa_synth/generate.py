"""Seeded synthetic inputs for the sparse GQA attention hot path.

One PCG64 stream per workload, drawn in a fixed order:
q_idx, key_state, w, Q, K, V, k_scale, v_scale.

* indexer query/key values: integers uniform in [-8, 8], stored in the indexer
  dtype (BF16 by default; every such integer is exact there);
* indexer head weights w_h: integers uniform in [1, 4], one per head, FP32,
  broadcast over batch and query tokens;
* Q, K, V: N(0, 1) drawn in FP32 and rounded to nearest-even into the storage
  dtype;
* INT8 KV: codes uniform in [-127, 127] and one FP32 scale per token per KV
  head for K and one for V, uniform in [0.005, 0.05).

With integer indexer inputs every partial sum of a score is an integer below
2**24 in magnitude, so scores are exact in FP32 whatever the summation order.
This module returns host tensors only; it does no arithmetic of the method.
"""
import numpy as np
import torch

from .workloads import Workload

_TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16,
          "i8": torch.int8}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH[name]


def _normal(rng, shape, dtype_name):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return torch.from_numpy(x).to(_TORCH[dtype_name])


def _int_uniform(rng, lo, hi, shape, dtype_name):
    x = rng.integers(lo, hi + 1, size=shape, dtype=np.int16).astype(np.float32)
    return torch.from_numpy(x).to(_TORCH[dtype_name])


def make_inputs(w: Workload, seed=None, kv_len=None):
    """Host tensors for one layer of workload `w`.

    Returns a dict with keys q_idx, w_idx, key_state (absent without an
    indexer), q, k_cache, v_cache, k_scale, v_scale (None unless INT8 KV),
    kv_len (int32 [B]) and, for dense-selection workloads, indices.
    `kv_len` overrides the per-sequence live length (default: every sequence
    full, kv_len = L).
    """
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    B, S, L = w.B, w.S, w.L
    out = {}
    if w.has_indexer:
        out["q_idx"] = _int_uniform(rng, -8, 8, (B, S, w.H_idx, w.D_idx), w.idx_dtype)
        out["key_state"] = _int_uniform(rng, -8, 8, (B, L, w.D_idx), w.idx_dtype)
        heads = rng.integers(1, 5, size=(w.H_idx,)).astype(np.float32)
        out["w_idx"] = torch.from_numpy(np.tile(heads, (B, S, 1)))
    out["q"] = _normal(rng, (B, S, w.H_q, w.D), w.q_dtype)
    if w.kv_dtype == "i8":
        kv_shape = (B, L, w.H_kv, w.D)
        out["k_cache"] = torch.from_numpy(
            rng.integers(-127, 128, size=kv_shape, dtype=np.int8))
        out["v_cache"] = torch.from_numpy(
            rng.integers(-127, 128, size=kv_shape, dtype=np.int8))
        out["k_scale"] = torch.from_numpy(
            rng.uniform(0.005, 0.05, size=(B, L, w.H_kv)).astype(np.float32))
        out["v_scale"] = torch.from_numpy(
            rng.uniform(0.005, 0.05, size=(B, L, w.H_kv)).astype(np.float32))
    else:
        out["k_cache"] = _normal(rng, (B, L, w.H_kv, w.D), w.kv_dtype)
        out["v_cache"] = _normal(rng, (B, L, w.H_kv, w.D), w.kv_dtype)
        out["k_scale"] = None
        out["v_scale"] = None
    if kv_len is None:
        kv_len = w.live_lengths
    out["kv_len"] = torch.tensor(kv_len, dtype=torch.int32)
    if not w.has_indexer:
        # Dense selection: every cached key of the row, in ascending order.
        out["indices"] = torch.arange(w.k, dtype=torch.int32).repeat(B, S, 1).contiguous()
    return out


def integer_scores(rng, shape, lo, hi):
    """FP32 array of integers uniform in [lo, hi] (a tie-heavy score source)."""
    return torch.from_numpy(rng.integers(lo, hi + 1, size=shape).astype(np.float32))


def indexer_like_scores(rng, shape, sigma=2100.0):
    """FP32 integers drawn from N(0, sigma^2), rounded to nearest.

    The spread of a 16-head x 64-dim indexer score with integer inputs in
    [-8, 8] and weights in [1, 4]; a stand-in score matrix for top-k tests
    at full size without running the indexer.
    """
    x = np.rint(rng.standard_normal(size=shape, dtype=np.float32) * np.float32(sigma))
    return torch.from_numpy(x.astype(np.float32))


def make_append_inputs(B, S, H_kv, D, L_cap, new_dtype, kv_dtype, kv_len, D_idx=64,
                       idx_dtype="bf16", seed=0, scale=1.0):
    """Inputs of one KV-cache append: pre-filled caches plus the new tokens.

    Draw order: k_cache, v_cache, (k_scale, v_scale), key_state, k_new, v_new,
    key_state_new.  Caches hold generator values (N(0,1) or INT8 codes with
    scales in [0.005, 0.05)); new K/V are N(0,1)*scale in new_dtype; indexer
    keys are integers in [-8, 8].  kv_len is the post-append length list.
    """
    rng = np.random.default_rng(seed)
    out = {}
    if kv_dtype == "i8":
        out["k_cache"] = torch.from_numpy(rng.integers(-127, 128, (B, L_cap, H_kv, D), dtype=np.int8))
        out["v_cache"] = torch.from_numpy(rng.integers(-127, 128, (B, L_cap, H_kv, D), dtype=np.int8))
        out["k_scale"] = torch.from_numpy(rng.uniform(0.005, 0.05, (B, L_cap, H_kv)).astype(np.float32))
        out["v_scale"] = torch.from_numpy(rng.uniform(0.005, 0.05, (B, L_cap, H_kv)).astype(np.float32))
    else:
        out["k_cache"] = _normal(rng, (B, L_cap, H_kv, D), kv_dtype)
        out["v_cache"] = _normal(rng, (B, L_cap, H_kv, D), kv_dtype)
        out["k_scale"] = out["v_scale"] = None
    out["key_state"] = _int_uniform(rng, -8, 8, (B, L_cap, D_idx), idx_dtype)
    kn = rng.standard_normal(size=(B, S, H_kv, D), dtype=np.float32) * np.float32(scale)
    vn = rng.standard_normal(size=(B, S, H_kv, D), dtype=np.float32) * np.float32(scale)
    out["k_new"] = torch.from_numpy(kn).to(_TORCH[new_dtype])
    out["v_new"] = torch.from_numpy(vn).to(_TORCH[new_dtype])
    out["key_state_new"] = _int_uniform(rng, -8, 8, (B, S, D_idx), idx_dtype)
    out["kv_len"] = torch.tensor(list(kv_len), dtype=torch.int32)
    return out


def make_new_tokens(B, S, H_kv, D, new_dtype, D_idx=64, idx_dtype="bf16", seed=0):
    """New K/V rows [B, S, H_kv, D] (N(0,1) in new_dtype) and indexer keys
    [B, S, D_idx] (integers in [-8, 8]) for one append step."""
    rng = np.random.default_rng(seed)
    return {"k_new": _normal(rng, (B, S, H_kv, D), new_dtype),
            "v_new": _normal(rng, (B, S, H_kv, D), new_dtype),
            "key_state_new": _int_uniform(rng, -8, 8, (B, S, D_idx), idx_dtype)}


def rope_tables(max_pos, D, base=1.0e6):
    """Caller-side FP32 rotary tables [max_pos, D/2]: cos and sin of
    p * base**(-2i/D), evaluated in FP64 and rounded to FP32."""
    inv = base ** (-np.arange(0, D, 2, dtype=np.float64) / D)
    ang = np.arange(max_pos, dtype=np.float64)[:, None] * inv[None, :]
    return (torch.from_numpy(np.cos(ang).astype(np.float32)),
            torch.from_numpy(np.sin(ang).astype(np.float32)))


def make_rope_inputs(B, S, H, D, max_pos, x_dtype, kv_len, seed=0, base=1.0e6):
    """Inputs of one RMSNorm + rotary call: head vectors x [B, S, H, D]
    (N(0,1) times a per-head spread in [0.5, 8], rounded to x_dtype), the
    FP32 norm weight [D] in [0.5, 1.5), the FP32 rotary tables and kv_len."""
    rng = np.random.default_rng(seed)
    spread = rng.uniform(0.5, 8.0, size=(1, 1, H, 1)).astype(np.float32)
    x = rng.standard_normal(size=(B, S, H, D), dtype=np.float32) * spread
    gamma = rng.uniform(0.5, 1.5, size=(D,)).astype(np.float32)
    cos, sin = rope_tables(max_pos, D, base)
    return {"x": torch.from_numpy(x).to(_TORCH[x_dtype]), "gamma": torch.from_numpy(gamma),
            "cos": cos, "sin": sin, "kv_len": torch.tensor(list(kv_len), dtype=torch.int32)}


def make_aux_inputs(B, S_aux, H_kv, D, aux_dtype, seed=0, value_scale=1.0):
    """Auxiliary (not yet cached) K/V [B, S_aux, H_kv, D]: N(0,1) in aux_dtype,
    V optionally multiplied by value_scale (large values exercise dtypes
    whose range the cache dtype lacks)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal(size=(B, S_aux, H_kv, D), dtype=np.float32)
    v = rng.standard_normal(size=(B, S_aux, H_kv, D), dtype=np.float32) * np.float32(value_scale)
    return {"aux_k": torch.from_numpy(k).to(_TORCH[aux_dtype]),
            "aux_v": torch.from_numpy(v).to(_TORCH[aux_dtype])}
