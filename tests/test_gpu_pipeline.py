"""The whole hot path (indexer -> top-k -> attention) at the five workloads'
full sizes, in the launch configuration the bench times, vs the oracle
pipeline on sampled rows: scores and indices bit-exact, outputs in tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_synth import ALL, RAGGED, make_inputs, torch_dtype
from gpu_util import (DEV, dsa, first_mismatch, run_attention, run_indexer,  # noqa: F401
                      run_topk, say, upload)
from parity import assert_output_close

pytestmark = pytest.mark.gpu

SAMPLE_ROWS = {
    "tiny_decode_1k": None,
    "spec_decode_32k": None,
    "prefill_128k": [(0, 0), (0, 1), (0, 777), (0, 1024), (0, 2047)],
    "int8_batched_decode_64k": [(0, 0), (5, 0)],
    "decode_256k": None,
    # ragged batches: rows of every sequence, including the first token of a
    # fresh sequence (one candidate key) and sequences far below capacity
    "ragged_decode_256k": [(0, 0), (0, 7), (1, 3), (2, 0), (2, 7), (3, 5)],
    "ragged_prefill_64k": [(0, 0), (0, 511), (1, 100), (1, 511), (2, 0), (2, 1), (2, 511)],
}


@pytest.mark.parametrize("wl", ALL + RAGGED, ids=lambda w: w.name)
def test_pipeline_full_size(dsa, wl):
    say(f"pipeline {wl.name} kv_len={wl.live_lengths} max_kv_len={wl.max_kv_len}")
    x = make_inputs(wl)
    g = upload(x)
    B, S, L = wl.B, wl.S, wl.L
    decode = wl.decode_form
    mx = wl.max_kv_len
    if wl.has_indexer:
        scores = run_indexer(dsa, g, L, max_kv_len=mx)
        idx = run_topk(dsa, scores, g["kv_len"], wl.k, max_kv_len=mx)
    else:
        scores, idx = None, g["indices"]
    out = run_attention(dsa, g, idx, torch_dtype(wl.out_dtype), decode=decode, max_kv_len=mx)
    torch.cuda.synchronize()

    rows = SAMPLE_ROWS[wl.name] or [(b, s) for b in range(B) for s in range(S)]
    kv_len = x["kv_len"].tolist()
    ref_idx = np.asarray(x["indices"]) if not wl.has_indexer else np.full((B, S, wl.k), -1)
    for b, s in rows:
        if not wl.has_indexer:
            continue
        pos = kv_len[b] - S + s
        ref_sc = oracle.indexer_scores_row(x["q_idx"][b, s], x["w_idx"][b, s], x["key_state"][b], pos)
        got_sc = scores[b, s, :pos + 1].cpu().double().numpy()
        assert np.array_equal(got_sc, ref_sc[:pos + 1]), f"scores ({b},{s}): {first_mismatch(got_sc, ref_sc[:pos + 1])}"
        ref_idx[b, s] = oracle.topk_row(ref_sc, pos, wl.k)
        got_i = idx[b, s].cpu().numpy()
        assert np.array_equal(got_i, ref_idx[b, s]), f"indices ({b},{s}): {first_mismatch(got_i, ref_idx[b, s])}"
    ref = oracle.sparse_attention(x["q"], x["k_cache"], x["v_cache"], ref_idx, kv_len,
                                  k_scale=x["k_scale"], v_scale=x["v_scale"], rows=rows)
    got = out.cpu()
    sel_got = torch.stack([got[b, s] for b, s in rows])
    sel_ref = np.stack([ref[b, s] for b, s in rows])
    rel, mx = assert_output_close(sel_got, sel_ref, wl.out_dtype, what=wl.name, strict=True)
    if wl.out_dtype == "f32":
        assert rel <= 1e-5
    say(f"pipeline {wl.name}: rows={len(rows)} rel={rel:.2e} max={mx:.2e}")
