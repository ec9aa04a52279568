"""CPU oracle for the KV-cache append step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module.  The HIP library never calls it and shares no code with it.

The step (ORT PR #33997, file table: "Updates preparation, cache writes,
attention kernels, and dispatch"; ORT PR #33802 Summary item 1: an INT8 KV
cache with one FP32 scale per token per KV head; the 128K-prefill and 256K
configurations append new tokens after the cached ones) writes the S new
tokens of every sequence into the caches before attention reads them:

* token s of sequence b lands at position kv_len[b] - S + s, where kv_len is
  the length after the append (the same kv_len the indexer, the top-k and
  the attention use for that step); positions outside [0, L_cap) are
  skipped;
* FP32 / FP16 / BF16 caches store the new K and V values rounded once,
  round-to-nearest-even, to the cache dtype;
* an INT8 cache stores, for every (token, KV head) row of D values x, the
  symmetric absmax quantisation computed in FP32:
      amax  = max_d |x_d|
      scale = fp32(amax / 127)
      code  = clip(rint(fp32(x_d / scale)), -127, 127)   (ties to even)
  and scale = 0 with all codes 0 for an all-zero row;
* the indexer key-state cache receives the new tokens' indexer keys as they
  are (same dtype).

The pages give no quantisation formula; symmetric absmax with 127 levels per
sign is the plainest reading of "codes uniform in [-127, 127] with an FP32
scale per token per KV head", and the quantised code is an integer decided by
floating point, so the oracle takes that decision in FP32, as the kernel does.

Pins (tests/test_cache_oracle.py): exact-rational brute force with correctly
rounded FP32 steps, requantisation of generator INT8 rows recovering their
codes, the error bound |code*scale - x| <= scale/2, sign symmetry, power-of-two
scaling, the all-zero row, and position bookkeeping of the append.
"""
import numpy as np


def quantize_row_int8(x):
    """Symmetric absmax INT8 quantisation of one row, in FP32 arithmetic.

    x: 1-D array of FP32-representable values.  Returns (codes int8 array,
    scale np.float32).
    """
    x = np.asarray(x, dtype=np.float32)
    amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0.0)
    if amax == 0.0:
        return np.zeros(x.shape, dtype=np.int8), np.float32(0.0)
    scale = np.float32(amax / np.float32(127.0))
    q = np.rint(x / scale)                      # FP32 division, then ties-to-even
    codes = np.clip(q, -127.0, 127.0).astype(np.int8)
    return codes, scale


def quantize_rows_int8(x):
    """quantize_row_int8 over the last axis of x ([..., D]) -> (codes, scales)."""
    x = np.asarray(x, dtype=np.float32)
    flat = x.reshape(-1, x.shape[-1])
    codes = np.empty(flat.shape, dtype=np.int8)
    scales = np.empty(flat.shape[0], dtype=np.float32)
    for r in range(flat.shape[0]):
        codes[r], scales[r] = quantize_row_int8(flat[r])
    return codes.reshape(x.shape), scales.reshape(x.shape[:-1])


def round_to_dtype(x, dtype):
    """Round FP32-representable values once, RNE, to 'f32' | 'f16' | 'bf16'.

    Returned as FP64 values (exact) for comparison.
    """
    import torch
    t = torch.as_tensor(np.asarray(x, dtype=np.float64))
    td = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[dtype]
    return t.to(td).double().numpy()


def append_positions(kv_len, S, L_cap):
    """[(b, s, pos)] for every new token whose position lies inside the cache."""
    out = []
    for b, n in enumerate(kv_len):
        for s in range(S):
            pos = int(n) - S + s
            if 0 <= pos < L_cap:
                out.append((b, s, pos))
    return out


def cache_append(k_cache, v_cache, k_new, v_new, kv_len, kv_dtype,
                 k_scale=None, v_scale=None, key_state=None, key_state_new=None):
    """Returns copies of the caches after appending the new tokens.

    k_cache, v_cache: [B, L_cap, H_kv, D] (numpy; int8 codes for kv_dtype 'i8')
    k_new, v_new:     [B, S, H_kv, D] FP32-representable values
    k_scale, v_scale: [B, L_cap, H_kv] FP32 (kv_dtype 'i8' only)
    key_state:        [B, L_cap, D_idx] or None; key_state_new [B, S, D_idx]
    """
    k_cache = np.array(k_cache, copy=True)
    v_cache = np.array(v_cache, copy=True)
    k_scale = None if k_scale is None else np.array(k_scale, copy=True)
    v_scale = None if v_scale is None else np.array(v_scale, copy=True)
    key_state = None if key_state is None else np.array(key_state, copy=True)
    S = k_new.shape[1]
    L_cap = k_cache.shape[1]
    for b, s, pos in append_positions(kv_len, S, L_cap):
        if kv_dtype == "i8":
            k_cache[b, pos], k_scale[b, pos] = quantize_rows_int8(k_new[b, s])
            v_cache[b, pos], v_scale[b, pos] = quantize_rows_int8(v_new[b, s])
        else:
            k_cache[b, pos] = round_to_dtype(k_new[b, s], kv_dtype)
            v_cache[b, pos] = round_to_dtype(v_new[b, s], kv_dtype)
        if key_state is not None:
            key_state[b, pos] = key_state_new[b, s]
    return k_cache, v_cache, k_scale, v_scale, key_state
