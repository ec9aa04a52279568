"""The whole hot path (indexer -> top-k -> attention) at the five workloads'
full sizes, in the launch configuration the bench times (the plans it logs
are asserted), vs the oracle pipeline: scores and indices bit-exact on every
row (the 2048-row prefill included), outputs in tolerance on every row of the
decode workloads and on 128 prefill rows covering every indexer token block.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import oracle
from dsa_synth import ALL, RAGGED, make_inputs, torch_dtype
from gpu_util import (DEV, dsa, first_mismatch, run_attention, run_indexer,  # noqa: F401
                      run_topk, say, upload)
from parity import assert_output_close

pytestmark = pytest.mark.gpu

# Attention rows compared with the oracle (None: every row).  The 128K
# prefill's indexer deals its 2048 tokens to 64 workgroups of 32 tokens (8
# waves x 2 token pairs); two rows per block, in both halves of the block,
# at offsets that walk every wave and both token pairs.
PREFILL_ROWS = [(0, 32 * i + o) for i in range(64) for o in ((i * 5) % 16, 16 + (i * 7) % 16)]
SAMPLE_ROWS = {
    "tiny_decode_1k": None,
    "spec_decode_32k": None,
    "prefill_128k": PREFILL_ROWS,
    "int8_batched_decode_64k": None,
    "decode_256k": None,
    # ragged batches: rows of every sequence, including the first token of a
    # fresh sequence (one candidate key) and sequences far below capacity
    "ragged_decode_256k": [(0, 0), (0, 7), (1, 3), (2, 0), (2, 7), (3, 5)],
    "ragged_prefill_64k": [(0, 0), (0, 511), (1, 100), (1, 511), (2, 0), (2, 1), (2, 511)],
}


# The launches each workload makes (indexer kernel, top-k plan, attention
# form), as dsa_describe_plan reports them -- the same descriptions the bench
# logs next to its timings.
EXPECTED_PLANS = {
    "tiny_decode_1k": ("indexer_score_kernel", "small", "attention_decode/split"),
    "spec_decode_32k": ("indexer_score_kernel", "resident", "attention_decode/split"),
    "prefill_128k": ("indexer_fold_kernel", "stream", "attention_prefill/wave_rows"),
    "int8_batched_decode_64k": (None, None, "attention_decode/split"),
    "decode_256k": ("indexer_stream_kernel", "split", "attention_decode/split"),
    "ragged_decode_256k": ("indexer_stream_kernel", "split", "attention_decode/split"),
    "ragged_prefill_64k": ("indexer_fold_kernel", "stream", "attention_prefill/wave_rows"),
}


def _plans(dsa, wl, g, idx, out):
    mx = wl.max_kv_len
    got = [None, None]
    if wl.has_indexer:
        got[0] = dsa.plan_fields(dsa.dsa_describe_plan(dsa.DSA_PLAN_INDEXER, wl.B, wl.S, wl.L, mx,
                                                       D_idx=wl.D_idx))["kernel"]
        got[1] = dsa.plan_fields(dsa.dsa_describe_plan(dsa.DSA_PLAN_TOPK, wl.B, wl.S, wl.L, mx,
                                                       k=wl.k))["plan"]
    a = dsa.attention_args(g["q"], g["k_cache"], g["v_cache"], idx, g["kv_len"], out,
                           g["k_scale"], g["v_scale"], max_kv_len=mx)
    op = dsa.DSA_PLAN_ATTENTION_DECODE if wl.decode_form else dsa.DSA_PLAN_ATTENTION_PREFILL
    f = dsa.plan_fields(dsa.dsa_describe_plan(op, attention=a))
    got.append(f"{f['op']}/{f['schedule']}")
    return tuple(got)


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
    assert _plans(dsa, wl, g, idx, out) == EXPECTED_PLANS[wl.name]

    rows = SAMPLE_ROWS[wl.name] or [(b, s) for b in range(B) for s in range(S)]
    kv_len = x["kv_len"].tolist()
    ref_idx = np.asarray(x["indices"]) if not wl.has_indexer else np.full((B, S, wl.k), -1)
    if wl.has_indexer:
        # scores and indices bit-exact on every row of the layer (oracle rows
        # computed in threads: NumPy's matmul and sort release the GIL)
        got_sc_all = scores.cpu().numpy()
        got_idx_all = idx.cpu().numpy()
        qi, wi, ks = (np.asarray(x[n]) if x[n].dtype == torch.float32 else x[n].float().numpy()
                      for n in ("q_idx", "w_idx", "key_state"))

        def check_row(bs):
            b, s = bs
            pos = kv_len[b] - S + s
            ref_sc = oracle.indexer_scores_row(qi[b, s], wi[b, s], ks[b], pos)
            got_sc = got_sc_all[b, s, :pos + 1].astype(np.float64)
            if not np.array_equal(got_sc, ref_sc[:pos + 1]):
                return f"scores ({b},{s}): {first_mismatch(got_sc, ref_sc[:pos + 1])}"
            ref_idx[b, s] = oracle.topk_row(ref_sc, pos, wl.k)
            if not np.array_equal(got_idx_all[b, s], ref_idx[b, s]):
                return f"indices ({b},{s}): {first_mismatch(got_idx_all[b, s], ref_idx[b, s])}"
            return None
        all_rows = [(b, s) for b in range(B) for s in range(S)]
        with ThreadPoolExecutor(16) as ex:
            bad = [m for m in ex.map(check_row, all_rows) if m]
        assert not bad, f"{len(bad)} row(s) differ; first: {bad[0]}"
        say(f"pipeline {wl.name}: scores and indices bit-exact on all {len(all_rows)} rows")
    ref = oracle.sparse_attention(x["q"], x["k_cache"], x["v_cache"], ref_idx, kv_len,
                                  k_scale=x["k_scale"], v_scale=x["v_scale"], rows=rows)
    got = out.cpu()
    sel_got = torch.stack([got[b, s] for b, s in rows])
    sel_ref = np.stack([ref[b, s] for b, s in rows])
    rel, mx = assert_output_close(sel_got, sel_ref, wl.out_dtype, what=wl.name, strict=True)
    if wl.out_dtype == "f32":
        assert rel <= 1e-5
    say(f"pipeline {wl.name}: rows={len(rows)} rel={rel:.2e} max={mx:.2e}")
