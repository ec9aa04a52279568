"""Helpers shared by the GPU parity tests (argument plumbing only)."""
import sys

import numpy as np
import pytest
import torch

DEV = torch.device("cuda:0")


def load_dsa():
    """The HIP library binding; fails (never skips) when it cannot run here."""
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    import sparse_gqa_attention_amd as dsa    # raises if libdsa.so is missing
    return dsa


@pytest.fixture(scope="module")
def dsa():
    return load_dsa()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def upload(x):
    return {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}


def run_indexer(dsa, g, L, max_kv_len=None):
    q = g["q_idx"]
    B, S = q.shape[0], q.shape[1]
    scores = torch.full((B, S, L), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_score(q, g["w_idx"], g["key_state"], g["kv_len"], scores,
                          max_kv_len=max_kv_len)
    return scores


def run_topk(dsa, scores, kv_len, k, max_kv_len=None):
    B, S, _ = scores.shape
    idx = torch.full((B, S, k), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(scores, kv_len, k, idx, max_kv_len=max_kv_len)
    return idx


def run_attention(dsa, g, indices, out_dtype, decode=True, scale=0.0, max_kv_len=None):
    q = g["q"]
    out = torch.full(q.shape, float("nan"), dtype=out_dtype, device=DEV)
    fn = dsa.dsa_attention_decode if decode else dsa.dsa_attention_prefill
    fn(q, g["k_cache"], g["v_cache"], indices, g["kv_len"], out,
       k_scale=g.get("k_scale"), v_scale=g.get("v_scale"), softmax_scale=scale,
       max_kv_len=max_kv_len)
    return out


def first_mismatch(a, b):
    bad = np.argwhere(a != b)
    if bad.size == 0:
        return "none"
    i = tuple(bad[0])
    return f"{len(bad)} mismatches, first at {i}: got {a[i]} want {b[i]}"
