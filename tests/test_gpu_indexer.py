"""Indexer scores on the GPU vs the FP64 oracle: bit-exact (integer inputs)."""
import numpy as np
import pytest
import torch

import oracle
from dsa_synth import (SPEC_DECODE_32K, TINY_DECODE, DECODE_256K, PREFILL_128K,
                       make_inputs, scaled)
from gpu_util import DEV, dsa, first_mismatch, run_indexer, say, upload  # noqa: F401

pytestmark = pytest.mark.gpu

# (B, S, H_idx, D_idx, L, kv_len, idx dtype)
SMALL = [
    (1, 1, 4, 32, 1024, None, "bf16"),
    (1, 8, 16, 64, 3000, None, "bf16"),            # ragged key tail
    (2, 20, 16, 64, 2500, [2500, 1800], "bf16"),   # two token pairs per wave, ragged kv_len
    (2, 3, 7, 128, 777, [777, 500], "f16"),
    (1, 9, 16, 32, 1500, None, "f16"),
    (3, 8, 16, 64, 5000, [5000, 8, 4000], "bf16"),  # kv_len == S
    (1, 40, 12, 64, 700, None, "bf16"),
    (1, 40, 16, 128, 900, None, "bf16"),          # prefill form, one token pair per wave
    (2, 33, 5, 32, 1300, [1300, 1000], "f16"),    # prefill form, D_idx 32, ragged kv_len
]


def _check(g_scores, x, S, what):
    kv_len = x["kv_len"].tolist()
    ref = oracle.indexer_scores(x["q_idx"], x["w_idx"], x["key_state"], kv_len, S)
    got = g_scores.cpu().double().numpy()
    B, _, L = got.shape
    for b in range(B):
        for s in range(S):
            pos = kv_len[b] - S + s
            a, r = got[b, s, :pos + 1], ref[b, s, :pos + 1]
            assert np.array_equal(a, r), f"{what} b={b} s={s}: {first_mismatch(a, r)}"
        assert np.all(np.isnan(got[b, :, kv_len[b]:])), f"{what}: wrote past kv_len"


@pytest.mark.parametrize("case", SMALL, ids=lambda c: f"B{c[0]}S{c[1]}H{c[2]}D{c[3]}L{c[4]}{c[6]}")
def test_indexer_small_exact(dsa, case):
    B, S, H, Di, L, kv, dt = case
    say(f"indexer small {case}")
    w = scaled(SPEC_DECODE_32K, B=B, S=S, H_idx=H, D_idx=Di, L=L, H_q=2, H_kv=1, D=64,
               idx_dtype=dt, seed=1000 + L)
    x = make_inputs(w, kv_len=kv)
    g = upload(x)
    scores = run_indexer(dsa, g, L)
    torch.cuda.synchronize()
    _check(scores, x, S, str(case))


# Decode shapes with more key runs than two per CU, which stream up to four
# runs per workgroup: every D_idx, partial token blocks (S < 8), ragged
# kv_len (one sequence of a single token) and ragged last runs.
LONG_DECODE = [
    (2, 3, 16, 64, 100000, [100000, 37001], "bf16"),
    (1, 8, 4, 32, 300000, None, "bf16"),
    (3, 1, 7, 128, 30000, [30000, 1, 17777], "f16"),
]


@pytest.mark.parametrize("case", LONG_DECODE, ids=lambda c: f"B{c[0]}S{c[1]}H{c[2]}D{c[3]}L{c[4]}{c[6]}")
def test_indexer_long_decode_streams_exact(dsa, case):
    B, S, H, Di, L, kv, dt = case
    say(f"indexer long decode {case}")
    w = scaled(SPEC_DECODE_32K, B=B, S=S, H_idx=H, D_idx=Di, L=L, H_q=2, H_kv=1, D=64,
               idx_dtype=dt, seed=2000 + L)
    x = make_inputs(w, kv_len=kv)
    scores = run_indexer(dsa, upload(x), L)
    torch.cuda.synchronize()
    _check(scores, x, S, str(case))


@pytest.mark.parametrize("wl", [TINY_DECODE, SPEC_DECODE_32K, DECODE_256K], ids=lambda w: w.name)
def test_indexer_full_size_all_rows(dsa, wl):
    say(f"indexer full {wl.name}")
    x = make_inputs(wl)
    scores = run_indexer(dsa, upload(x), wl.L)
    torch.cuda.synchronize()
    _check(scores, x, wl.S, wl.name)


def test_indexer_prefill_128k_sampled_rows(dsa):
    wl = PREFILL_128K
    say("indexer full prefill_128k (sampled rows)")
    x = make_inputs(wl)
    scores = run_indexer(dsa, upload(x), wl.L)
    torch.cuda.synchronize()
    rows = [0, 1, 15, 16, 511, 1024, 2046, 2047]
    got = scores[0, rows].cpu().double().numpy()
    for i, s in enumerate(rows):
        pos = wl.L - wl.S + s
        ref = oracle.indexer_scores_row(x["q_idx"][0, s], x["w_idx"][0, s], x["key_state"][0], pos)
        a, r = got[i, :pos + 1], ref[:pos + 1]
        assert np.array_equal(a, r), f"row {s}: {first_mismatch(a, r)}"


# Prefill shapes long enough that each workgroup streams several key runs
# through its two LDS buffers (odd and even run counts, a ragged last run,
# partial token blocks, one short sequence), checked on sampled rows.
# (B, S, H_idx, D_idx, L, kv_len, idx dtype, sampled token rows)
STREAMED = [
    (2, 70, 16, 64, 300000, [300000, 123457], "bf16", [0, 1, 2, 3, 31, 32, 63, 64, 65, 68, 69]),
    (1, 40, 16, 32, 600000, None, "f16", [0, 7, 8, 33, 39]),
    (1, 33, 8, 128, 400000, [399999], "bf16", [0, 15, 16, 31, 32]),
]


@pytest.mark.parametrize("case", STREAMED, ids=lambda c: f"B{c[0]}S{c[1]}D{c[3]}L{c[4]}")
def test_indexer_prefill_streamed_sampled_rows(dsa, case):
    B, S, H, Di, L, kv, dt, rows = case
    say(f"indexer streamed prefill {case[:7]}")
    w = scaled(SPEC_DECODE_32K, B=B, S=S, H_idx=H, D_idx=Di, L=L, H_q=2, H_kv=1, D=64,
               idx_dtype=dt, seed=2000 + Di)
    x = make_inputs(w, kv_len=kv)
    scores = run_indexer(dsa, upload(x), L)
    torch.cuda.synchronize()
    kv_len = x["kv_len"].tolist()
    for b in range(B):
        got = scores[b, rows].cpu().double().numpy()
        for i, s in enumerate(rows):
            pos = kv_len[b] - S + s
            ref = oracle.indexer_scores_row(x["q_idx"][b, s], x["w_idx"][b, s], x["key_state"][b],
                                            pos)
            a, r = got[i, :pos + 1], ref[:pos + 1]
            assert np.array_equal(a, r), f"b={b} row {s}: {first_mismatch(a, r)}"
            assert np.all(np.isnan(got[i, kv_len[b]:])), f"b={b} row {s}: wrote past kv_len"


def test_indexer_decode_beyond_grid_limit_streams(dsa):
    # A decode step (S <= 8) over more keys than one-run workgroups can cover
    # within the grid's y limit (60000 runs of 128 keys at D_idx 128) takes
    # the streaming kernel.  Small integer inputs keep every score exact;
    # sampled keys (first and last runs, random ones) are checked against the
    # oracle applied to those key rows alone.
    B, S, H, Di, L = 1, 2, 2, 128, 8_000_000
    say(f"indexer decode beyond grid limit L={L}")
    g = torch.Generator(device=DEV).manual_seed(21)
    ks = torch.randint(-4, 5, (B, L, Di), generator=g, device=DEV).to(torch.bfloat16)
    q = torch.randint(-4, 5, (B, S, H, Di), generator=g, device=DEV).to(torch.bfloat16)
    w = torch.randint(1, 5, (B, S, H), generator=g, device=DEV).to(torch.float32)
    kv = torch.tensor([L], dtype=torch.int32, device=DEV)
    scores = torch.full((B, S, L), float("nan"), dtype=torch.float32, device=DEV)
    dsa.dsa_indexer_score(q, w, ks, kv, scores)
    torch.cuda.synchronize()
    r = np.random.default_rng(22)
    keys = np.unique(np.concatenate([np.arange(0, 300), np.arange(L - 300, L),
                                     r.integers(0, L, size=4000)]))
    sub = ks[0, torch.from_numpy(keys).to(DEV)].float().cpu().numpy()
    for s in range(S):
        pos = L - S + s
        ok = keys[keys <= pos]
        ref = oracle.indexer_scores_row(q[0, s].float().cpu().numpy(), w[0, s].cpu().numpy(),
                                        sub[:len(ok)], len(ok) - 1)
        got = scores[0, s, torch.from_numpy(ok).to(DEV)].double().cpu().numpy()
        assert np.array_equal(got, ref), f"s={s}: {first_mismatch(got, ref)}"
