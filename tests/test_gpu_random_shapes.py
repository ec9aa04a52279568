"""Seeded random shapes across the indexer plans, the top-k plans and the
attention schedules.

Each case draws its sizes, live lengths, runtime bound and score or input
distribution from a fixed seed, so a failure names a reproducible case.
The plans and schedules a case lands on are whatever the planner picks for
those sizes: the sweep covers plan boundaries (4096 and 32768 keys, 128
rows, the split counts of the decode attention) that hand-picked tests may
straddle.  Indexer scores (integer inputs) and top-k indices are
bit-exact against the oracle; attention outputs pass the same gate as the
other attention tests.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_synth import SPEC_DECODE_32K, indexer_like_scores, make_inputs, scaled, torch_dtype
from gpu_util import (DEV, dsa, first_mismatch, run_attention, run_indexer, run_topk,  # noqa: F401
                      say, upload)
from parity import assert_output_close
from test_gpu_attention import COMBOS, random_selection

pytestmark = pytest.mark.gpu


def _topk_case(seed):
    r = np.random.default_rng(1000 + seed)
    L = int(r.choice([64, 700, 1024, 4096, 4100, 9001, 32768, 40000, 100000]))
    S = int(r.choice([1, 3, 8, 130, 130]))
    B = int(r.integers(1, 3))
    if B * S * L > 6_000_000:                   # keep the oracle's sorts to seconds
        S = max(1, 6_000_000 // (B * L))
    if seed % 6 == 5:                           # many rows of more than 4096 keys: streaming
        B, S, L = 1, 130, int(r.choice([9001, 20000, 40000]))
    k = int(r.choice([1, 7, 128, 512, 2048, max(1, L // 2), L + 5]))
    mx = int(r.integers(max(S, min(L, 64)), L + 1))    # the runtime bound
    if seed % 6 == 5:
        mx = int(r.integers(5000, L + 1))
    kv = [int(r.integers(S, mx + 1)) for _ in range(B)]
    kind = int(r.integers(0, 4))
    if kind == 0:
        sc = r.standard_normal((B, S, L)).astype(np.float32)
    elif kind == 1:
        sc = r.integers(-30, 31, size=(B, S, L)).astype(np.float32)
    elif kind == 2:
        sc = indexer_like_scores(r, (B, S, L)).numpy()
    else:                                       # signed zeros, -inf, denormals, ties
        vals = np.array([0.0, -0.0, -np.inf, 2.0 ** -149, -(2.0 ** -149), 1.0, 1.0], dtype=np.float32)
        sc = vals[r.integers(0, vals.shape[0], size=(B, S, L))]
    return B, S, L, k, mx, kv, kind, sc


@pytest.mark.parametrize("seed", range(24))
def test_topk_random_shapes(dsa, seed):
    B, S, L, k, mx, kv, kind, sc = _topk_case(seed)
    plan = dsa.plan_fields(dsa.dsa_describe_plan(dsa.DSA_PLAN_TOPK, B, S, L, mx, k=k))["plan"]
    say(f"topk seed={seed} B={B} S={S} L={L} k={k} max_kv_len={mx} kv_len={kv} kind={kind} plan={plan}")
    g_kv = torch.tensor(kv, dtype=torch.int32, device=DEV)
    idx = run_topk(dsa, torch.from_numpy(sc).to(DEV), g_kv, k, max_kv_len=mx)
    got = idx.cpu().numpy()
    for b in range(B):
        for s in range(S):
            want = oracle.topk_row(sc[b, s], kv[b] - S + s, k)
            assert np.array_equal(got[b, s], want), \
                f"seed {seed} ({plan}) row ({b},{s}): {first_mismatch(got[b, s], want)}"


def _attention_case(seed):
    r = np.random.default_rng(2000 + seed)
    combo = COMBOS[int(r.integers(0, len(COMBOS)))]
    B = int(r.integers(1, 3))
    S = int(r.choice([1, 2, 5, 8, 16]))
    L = int(r.choice([300, 2100, 9000, 20000]))
    k = int(r.choice([1, 33, 200, 1000, 2048, 3000]))
    mx = int(r.integers(max(S, 64), L + 1))
    kv = [int(r.integers(S, mx + 1)) for _ in range(B)]
    decode = bool(r.integers(0, 2))
    return combo, B, S, L, k, mx, kv, decode


@pytest.mark.parametrize("seed", range(16))
def test_attention_random_shapes(dsa, seed):
    combo, B, S, L, k, mx, kv, decode = _attention_case(seed)
    qd, kd, od, D, H_q, H_kv = combo
    w = scaled(SPEC_DECODE_32K, B=B, S=S, L=L, H_q=H_q, H_kv=H_kv, D=D, q_dtype=qd,
               kv_dtype=kd, out_dtype=od, k=k, H_idx=None, D_idx=None, seed=3000 + seed)
    x = make_inputs(w, kv_len=kv)
    idx = random_selection(np.random.default_rng(seed), kv, S, k, L)
    g = upload(x)
    out = run_attention(dsa, g, idx.to(DEV), torch_dtype(od), decode=decode, max_kv_len=mx)
    torch.cuda.synchronize()
    ref = oracle.sparse_attention(x["q"], x["k_cache"], x["v_cache"], idx, kv,
                                  k_scale=x["k_scale"], v_scale=x["v_scale"])
    rel, mx_err = assert_output_close(out, ref, od, what=f"seed {seed} {combo} decode={decode}")
    if od == "f32":
        assert rel <= 1e-5, f"seed {seed} {combo}: FP32 output rel RMSE {rel:.2e}"
    say(f"attention seed={seed} {combo} B={B} S={S} L={L} k={k} max_kv_len={mx} kv_len={kv} "
        f"decode={decode}: rel={rel:.2e} max={mx_err:.2e}")


def _indexer_case(seed):
    r = np.random.default_rng(4000 + seed)
    B = int(r.integers(1, 4))
    S = int(r.choice([1, 2, 5, 8, 9, 33, 70]))
    H = int(r.integers(1, 17))
    Di = int(r.choice([32, 64, 128]))
    L = int(r.choice([S + 3, 500, 2049, 9000, 40000, 90000]))
    dt = "bf16" if r.integers(0, 2) == 0 else "f16"
    mx = int(r.integers(S, L + 1))
    kv = [int(r.integers(S, mx + 1)) for _ in range(B)]
    kv[int(r.integers(0, B))] = mx              # the bound is reached
    return B, S, H, Di, L, dt, mx, kv


@pytest.mark.parametrize("seed", range(16))
def test_indexer_random_shapes(dsa, seed):
    B, S, H, Di, L, dt, mx, kv = _indexer_case(seed)
    plan = dsa.plan_fields(dsa.dsa_describe_plan(dsa.DSA_PLAN_INDEXER, B, S, L, mx, D_idx=Di))["kernel"]
    say(f"indexer seed={seed} B={B} S={S} H={H} D={Di} L={L} {dt} max_kv_len={mx} kv_len={kv} {plan}")
    w = scaled(SPEC_DECODE_32K, B=B, S=S, H_idx=H, D_idx=Di, L=L, H_q=2, H_kv=1, D=64,
               idx_dtype=dt, seed=5000 + seed)
    x = make_inputs(w, kv_len=kv)
    g = upload(x)
    scores = run_indexer(dsa, g, L, max_kv_len=mx)
    torch.cuda.synchronize()
    ref = oracle.indexer_scores(x["q_idx"], x["w_idx"], x["key_state"], kv, S)
    got = scores.cpu().double().numpy()
    for b in range(B):
        for s in range(S):
            pos = kv[b] - S + s
            a, want = got[b, s, :pos + 1], ref[b, s, :pos + 1]
            assert np.array_equal(a, want), f"seed {seed} ({plan}) b={b} s={s}: {first_mismatch(a, want)}"
        assert np.all(np.isnan(got[b, :, kv[b]:])), f"seed {seed} ({plan}): wrote past kv_len"
