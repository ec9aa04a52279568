"""Sparse attention with auxiliary (not yet cached) K/V on the GPU vs the
FP64 oracle (oracle/aux_oracle.py), through dsa_attention_decode/_prefill.

Same gate as the plain attention tests: relative RMSE <= 1e-3 and, per
element, |error| <= max(4e-3, one ulp) against the oracle rounded once.
"""
import numpy as np
import pytest
import torch

import oracle.aux_oracle as ao
from dsa_synth import SPEC_DECODE_32K, make_aux_inputs, make_inputs, scaled, torch_dtype
from gpu_util import DEV, dsa, say, upload  # noqa: F401
from parity import assert_output_close
from test_gpu_attention import random_selection

pytestmark = pytest.mark.gpu

# (q, kv, out, aux, D, H_q, H_kv)
COMBOS = [
    ("bf16", "f16", "bf16", "bf16", 128, 24, 2),   # BF16 aux next to an FP16 cache
    ("bf16", "f16", "bf16", "f16", 128, 24, 2),
    ("f16", "bf16", "f16", "bf16", 128, 12, 2),     # FP16 query, BF16 aux: FP32 products
    ("bf16", "i8", "bf16", "bf16", 128, 48, 8),
    ("f32", "f32", "f32", "f32", 64, 4, 1),
    ("f16", "f16", "f32", "f32", 64, 12, 2),        # FP32 aux
]


def _run(dsa, combo, B, S, S_aux, L, k, kv_len, decode, seed, value_scale=1.0):
    qd, kd, od, ad, D, H_q, H_kv = combo
    say(f"aux {combo} B={B} S={S} S_aux={S_aux} L={L} k={k} kv_len={kv_len} decode={decode} "
        f"value_scale={value_scale}")
    w = scaled(SPEC_DECODE_32K, B=B, S=S, L=L, H_q=H_q, H_kv=H_kv, D=D, q_dtype=qd,
               kv_dtype=kd, out_dtype=od, k=k, H_idx=None, D_idx=None, seed=seed, kv_len=None)
    x = make_inputs(w, kv_len=kv_len)
    x.update(make_aux_inputs(B, S_aux, H_kv, D, ad, seed=seed + 1, value_scale=value_scale))
    idx = random_selection(np.random.default_rng(seed), kv_len, S, k, L)
    g = upload(x)
    out = torch.full((B, S, H_q, D), float("nan"), dtype=torch_dtype(od), device=DEV)
    fn = dsa.dsa_attention_decode if decode else dsa.dsa_attention_prefill
    fn(g["q"], g["k_cache"], g["v_cache"], idx.to(DEV), g["kv_len"], out,
       k_scale=g["k_scale"], v_scale=g["v_scale"], aux_k=g["aux_k"], aux_v=g["aux_v"])
    torch.cuda.synchronize()
    ref = ao.sparse_attention_with_aux(x["q"], x["k_cache"], x["v_cache"], idx, kv_len,
                                       x["aux_k"], x["aux_v"], k_scale=x["k_scale"],
                                       v_scale=x["v_scale"])
    if value_scale != 1.0:
        # values far from 1: the error bound scales with the values' magnitude
        got = out.cpu().double().numpy()
        assert np.all(np.isfinite(got)), "non-finite output"
        ref = torch.from_numpy(ref).to(torch_dtype(od)).double().numpy()   # rounded once
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        mx = float(np.max(np.abs(got - ref)))
        assert rel <= 1e-3 and mx <= 4e-3 * value_scale, (rel, mx)
    else:
        rel, mx = assert_output_close(out, ref, od, what=f"aux {combo} decode={decode}")
    if od == "f32":
        assert rel <= 1e-5
    say(f"  rel={rel:.2e} max={mx:.2e}")


@pytest.mark.parametrize("decode", [True, False], ids=["decode", "prefill"])
@pytest.mark.parametrize("combo", COMBOS, ids=lambda c: "-".join(map(str, c)))
def test_aux_dtype_combos(dsa, combo, decode):
    # second sequence holds only the fresh tokens (kv_len == S_aux): aux-only rows
    _run(dsa, combo, B=2, S=8, S_aux=8, L=900, k=200, kv_len=[900, 8], decode=decode, seed=41)


def test_aux_bf16_values_beyond_fp16_range_next_to_fp16_cache(dsa):
    # the aux V reaches ~4e5, which an FP16 conversion would turn into inf
    _run(dsa, COMBOS[0], B=2, S=8, S_aux=8, L=700, k=128, kv_len=[700, 300], decode=True,
         seed=42, value_scale=1.0e5)


@pytest.mark.parametrize("decode", [True, False], ids=["decode", "prefill"])
def test_aux_longer_than_the_query_run(dsa, decode):
    # 12 fresh tokens, the last 4 of which are queries
    _run(dsa, COMBOS[1], B=2, S=4, S_aux=12, L=500, k=100, kv_len=[500, 12], decode=decode, seed=43)


def test_aux_prefill_chunk(dsa):
    _run(dsa, COMBOS[1], B=1, S=96, S_aux=96, L=1200, k=256, kv_len=[1200], decode=False, seed=44)


def test_aux_with_the_maximum_number_of_splits(dsa):
    # a long selection reaches the split cap; the aux keys take the last merge slot
    _run(dsa, ("f16", "f16", "f16", "f16", 64, 4, 1), B=1, S=1, S_aux=1, L=20000, k=9000,
         kv_len=[20000], decode=True, seed=45)


@pytest.mark.parametrize("combo", [COMBOS[0], COMBOS[3], COMBOS[4]],
                         ids=lambda c: "-".join(map(str, c)))
def test_aux_prefill_whole_row_waves(dsa, combo):
    # >= 2048 (row, KV head) pairs: the main launch runs whole-row waves, each
    # writing its row's partial next to the auxiliary split's (32 fresh tokens;
    # the second sequence holds 40 tokens, so its early rows see few cache keys)
    H_kv = combo[6]
    S = -(-1024 // H_kv) + 1
    _run(dsa, combo, B=2, S=S, S_aux=32, L=S + 300, k=100, kv_len=[S + 300, S], decode=False,
         seed=44)
