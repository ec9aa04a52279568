"""Pins of the FP64 oracle against what the pages and the mathematics fix.

None of these re-types the oracle's own formula: each checks it against a
brute force, a closed form, an independent library routine (torch's
scaled_dot_product_attention) or an invariant chosen so that a dropped term,
a wrong sign or index, or a transposed operand fails at least one of them.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from dsa_synth import make_inputs, scaled, TINY_DECODE, INT8_DECODE_64K

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- scores
def test_scores_match_python_integer_brute_force():
    rng = np.random.default_rng(11)
    B, S, H, Di, L = 2, 3, 3, 5, 9
    q = rng.integers(-8, 9, size=(B, S, H, Di))
    ks = rng.integers(-8, 9, size=(B, L, Di))
    w = rng.integers(1, 5, size=(B, S, H)).astype(np.float64)
    kv_len = [L, L - 2]
    got = oracle.indexer_scores(q, w, ks, kv_len, S)
    for b in range(B):
        for s in range(S):
            pos = kv_len[b] - S + s
            for j in range(L):
                if j > pos:
                    assert math.isnan(got[b, s, j])
                    continue
                want = 0
                for h in range(H):
                    dot = 0
                    for d in range(Di):
                        dot += int(q[b, s, h, d]) * int(ks[b, j, d])
                    want += int(w[b, s, h]) * dot
                assert got[b, s, j] == want


def test_scores_one_hot_keys_pick_weighted_query_column():
    rng = np.random.default_rng(12)
    H, Di, L = 4, 6, 12
    q = rng.integers(-8, 9, size=(H, Di)).astype(np.float64)
    w = np.array([1.0, 2.0, 3.0, 4.0])
    ks = np.zeros((L, Di))
    for j in range(L):
        ks[j, j % Di] = 1.0
    got = oracle.indexer_scores_row(q, w, ks, pos=L - 1)
    for j in range(L):
        assert got[j] == sum(w[h] * q[h, j % Di] for h in range(H))


def test_scores_scale_with_weights_and_flip_with_keys():
    rng = np.random.default_rng(13)
    q = rng.integers(-8, 9, size=(16, 64)).astype(np.float64)
    ks = rng.integers(-8, 9, size=(40, 64)).astype(np.float64)
    w = rng.integers(1, 5, size=16).astype(np.float64)
    base = oracle.indexer_scores_row(q, w, ks, pos=39)
    assert np.array_equal(oracle.indexer_scores_row(q, 2 * w, ks, pos=39), 2 * base)
    assert np.array_equal(oracle.indexer_scores_row(q, w, -ks, pos=39), -base)
    # Only head 3 weighted: the score is that head's plain dot product.
    w3 = np.zeros(16)
    w3[3] = 1.0
    assert np.array_equal(oracle.indexer_scores_row(q, w3, ks, pos=39), ks @ q[3])


# ----------------------------------------------------------------- top-k
def _brute_force_topk(scores, pos, k):
    n = pos + 1
    chosen = []
    for j in range(n):
        rank = sum(1 for i in range(n) if scores[i] > scores[j])
        rank += sum(1 for i in range(j) if scores[i] == scores[j])
        if rank < k:
            chosen.append(j)
    return chosen + [-1] * (k - len(chosen))


@pytest.mark.parametrize("seed", range(6))
def test_topk_matches_brute_force_rank_definition(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(5, 60))
    pos = int(rng.integers(0, L))
    k = int(rng.integers(1, 40))
    sc = rng.integers(-3, 4, size=L).astype(np.float64)   # many ties
    assert list(oracle.topk_row(sc, pos, k)) == _brute_force_topk(sc, pos, k)


def test_topk_tie_storm_takes_lowest_indices():
    assert list(oracle.topk_row(np.full(100, 7.0), 99, 10)) == list(range(10))


def test_topk_short_row_pads_with_minus_one():
    got = oracle.topk_row(np.arange(50.0), 4, 8)
    assert list(got) == [0, 1, 2, 3, 4, -1, -1, -1]
    assert list(oracle.topk_row(np.arange(5.0), -1, 3)) == [-1, -1, -1]


def test_topk_is_nested_in_k():
    rng = np.random.default_rng(5)
    sc = rng.integers(-20, 21, size=300).astype(np.float64)
    prev = set()
    for k in range(1, 60):
        cur = set(oracle.topk_row(sc, 299, k).tolist())
        assert prev <= cur and len(cur) == k
        prev = cur


def test_topk_ignores_scores_beyond_position():
    rng = np.random.default_rng(6)
    sc = rng.normal(size=500)
    base = oracle.topk_row(sc, 300, 32)
    poisoned = sc.copy()
    poisoned[301:] = 1e30
    assert np.array_equal(oracle.topk_row(poisoned, 300, 32), base)


def test_topk_signed_zeros_tie_and_minus_inf_ranks_last():
    sc = np.array([-0.0, 0.0, -0.0, -np.inf, 0.0, -1.0])
    assert list(oracle.topk_row(sc, 5, 3)) == [0, 1, 2]
    assert list(oracle.topk_row(sc, 5, 6)) == [0, 1, 2, 3, 4, 5]
    assert list(oracle.topk_row(sc, 5, 5)) == [0, 1, 2, 4, 5]


def test_topk_picks_highest_not_lowest():
    sc = np.array([1.0, 5.0, 3.0, 9.0, -2.0])
    assert list(oracle.topk_row(sc, 4, 2)) == [1, 3]


# ----------------------------------------------------------------- attention
def _causal_gqa_sdpa(q, k, v, kv_len, scale):
    """Ordinary causal GQA attention from torch's SDPA in FP64 on the CPU."""
    B, S, H_q, D = q.shape
    L, H_kv = k.shape[1], k.shape[2]
    ratio = H_q // H_kv
    out = np.zeros((B, S, H_q, D))
    for b in range(B):
        qt = torch.from_numpy(q[b]).permute(1, 0, 2)                 # [H_q, S, D]
        kt = torch.from_numpy(k[b]).permute(1, 0, 2).repeat_interleave(ratio, 0)
        vt = torch.from_numpy(v[b]).permute(1, 0, 2).repeat_interleave(ratio, 0)
        pos = torch.arange(S) + (kv_len[b] - S)
        mask = torch.arange(L)[None, :] <= pos[:, None]              # [S, L]
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt.contiguous(), vt.contiguous(), attn_mask=mask, scale=scale)
        out[b] = o.permute(1, 0, 2).numpy()
    return out


@pytest.mark.parametrize("H_q,H_kv", [(6, 2), (4, 4), (12, 1)])
def test_full_selection_equals_causal_gqa_attention(H_q, H_kv):
    rng = np.random.default_rng(21)
    B, S, L, D = 2, 3, 20, 8
    q = rng.normal(size=(B, S, H_q, D))
    k = rng.normal(size=(B, L, H_kv, D))
    v = rng.normal(size=(B, L, H_kv, D))
    kv_len = [L, L - 5]
    idx = np.broadcast_to(np.arange(L), (B, S, L))       # k = L >= pos + 1
    scale = 0.37
    got = oracle.sparse_attention(q, k, v, idx, kv_len, scale=scale)
    want = _causal_gqa_sdpa(q, k, v, kv_len, scale)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(22)
    q = rng.normal(size=(6, 16))
    k = rng.normal(size=(50, 2, 16))
    v = np.empty((50, 2, 16))
    v[:, 0, :] = 3.25
    v[:, 1, :] = -1.5
    idx = rng.choice(50, size=9, replace=False)
    out = oracle.attention_row(q, k, v, idx, 49, 50, 0.25)
    assert np.allclose(out[:3], 3.25, rtol=0, atol=1e-13)
    assert np.allclose(out[3:], -1.5, rtol=0, atol=1e-13)


def test_weights_sum_to_one_and_vanish_off_selection():
    rng = np.random.default_rng(23)
    q = rng.normal(size=(4, 8))
    k = rng.normal(size=(30, 1, 8))
    v = rng.normal(size=(30, 1, 8))
    idx = np.array([3, 7, 11, 25, 29, -1])
    _, wts = oracle.attention_row(q, k, v, idx, 26, 30, 0.5, return_weights=True)
    np.testing.assert_allclose(wts.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    off = np.ones(30, dtype=bool)
    off[[3, 7, 11, 25]] = False           # 29 > pos and -1 are not valid keys
    assert np.all(wts[:, off] == 0)
    assert np.all(wts[:, ~off] > 0)


def test_single_key_returns_its_value_row():
    rng = np.random.default_rng(24)
    q = rng.normal(size=(4, 8))
    k = rng.normal(size=(30, 2, 8))
    v = rng.normal(size=(30, 2, 8))
    out = oracle.attention_row(q, k, v, np.array([17]), 29, 30, 0.5)
    assert np.array_equal(out[:2], np.broadcast_to(v[17, 0], (2, 8)))
    assert np.array_equal(out[2:], np.broadcast_to(v[17, 1], (2, 8)))


def test_two_keys_follow_the_logistic_closed_form():
    rng = np.random.default_rng(25)
    D = 8
    q = rng.normal(size=(1, D))
    k = rng.normal(size=(10, 1, D))
    v = rng.normal(size=(10, 1, D))
    scale = 0.7
    l0 = scale * q[0] @ k[2, 0]
    l1 = scale * q[0] @ k[6, 0]
    sig = 1.0 / (1.0 + math.exp(-(l0 - l1)))
    want = sig * v[2, 0] + (1 - sig) * v[6, 0]
    out = oracle.attention_row(q, k, v, np.array([6, 2]), 9, 10, scale)
    np.testing.assert_allclose(out[0], want, rtol=1e-13, atol=1e-14)


def test_index_order_and_invalid_entries_do_not_matter():
    rng = np.random.default_rng(26)
    q = rng.normal(size=(6, 8))
    k = rng.normal(size=(40, 3, 8))
    v = rng.normal(size=(40, 3, 8))
    idx = np.array([1, 5, 9, 20, 33])
    base = oracle.attention_row(q, k, v, idx, 35, 40, 0.3)
    perm = oracle.attention_row(q, k, v, idx[::-1].copy(), 35, 40, 0.3)
    noisy = oracle.attention_row(q, k, v, np.array([-1, 33, 38, 1, 5, 39, 9, -1, 20]),
                                 35, 40, 0.3)
    np.testing.assert_allclose(perm, base, rtol=1e-14, atol=1e-14)
    np.testing.assert_allclose(noisy, base, rtol=1e-14, atol=1e-14)


def test_row_without_valid_keys_is_zero():
    q = np.ones((2, 4))
    k = np.ones((5, 1, 4))
    v = np.ones((5, 1, 4))
    assert np.all(oracle.attention_row(q, k, v, np.array([-1, 4]), 3, 5, 1.0) == 0)


def test_large_logit_gap_keeps_the_small_weight():
    # exp(-100) is far below FP32's range but exact enough in FP64.
    q = np.array([[1.0, 0.0]])
    k = np.array([[[0.0, 0.0]], [[100.0, 0.0]]])
    v = np.array([[[1.0, 1.0]], [[0.0, 0.0]]])
    out = oracle.attention_row(q, k, v, np.array([0, 1]), 1, 2, 1.0)
    np.testing.assert_allclose(out[0], math.exp(-100) / (1 + math.exp(-100)), rtol=1e-12)


# ----------------------------------------------------------------- INT8 cache
def test_int8_generator_values_round_trip():
    w = scaled(INT8_DECODE_64K, B=2, L=256, H_q=12, H_kv=2, k=256)
    x = make_inputs(w)
    for codes, sc in ((x["k_cache"], x["k_scale"]), (x["v_cache"], x["v_scale"])):
        deq = oracle.dequantize(codes, sc)
        back = np.rint(deq / sc.double().numpy()[..., None])
        assert np.array_equal(back, codes.numpy().astype(np.float64))
        assert codes.abs().max() <= 127
        assert float(sc.min()) >= 0.005 and float(sc.max()) < 0.05


def test_int8_path_equals_float_path_on_dequantised_cache():
    w = scaled(INT8_DECODE_64K, B=2, L=96, H_q=12, H_kv=2, k=96)
    x = make_inputs(w)
    rows = [(0, 0), (1, 0)]
    got = oracle.sparse_attention(x["q"], x["k_cache"], x["v_cache"], x["indices"],
                                  x["kv_len"].tolist(), k_scale=x["k_scale"],
                                  v_scale=x["v_scale"], rows=rows)
    kf = x["k_cache"].double() * x["k_scale"].double()[..., None]
    vf = x["v_cache"].double() * x["v_scale"].double()[..., None]
    want = oracle.sparse_attention(x["q"], kf, vf, x["indices"], x["kv_len"].tolist(),
                                   rows=rows)
    assert np.array_equal(got, want)


def test_worked_example_from_the_pages():
    g = json.load(open(os.path.join(GOLDEN, "int8_rising_max.json")))
    D = 16
    q = np.zeros((1, 1, 1, D))
    q[0, 0, 0, 0] = 1.0
    codes_k = np.zeros((1, 2, 1, D), dtype=np.int8)
    codes_k[0, 1, 0, 0] = int(g["logits"][1])            # logit = 1 * 88 * 1
    codes_v = np.zeros((1, 2, 1, D), dtype=np.int8)
    codes_v[0, 0, 0, :] = g["value_codes"][0]
    codes_v[0, 1, 0, :] = g["value_codes"][1]
    k_scale = np.ones((1, 2, 1))
    v_scale = np.full((1, 2, 1), 2.0 ** g["value_scale_log2"])
    out = oracle.sparse_attention(q, codes_k, codes_v, np.array([[[0, 1]]]), [2],
                                  scale=1.0, k_scale=k_scale, v_scale=v_scale)
    closed = 2.0 ** 120 * math.exp(-88) / (1 + math.exp(-88))
    np.testing.assert_allclose(out[0, 0, 0], closed, rtol=1e-12)
    assert abs(out[0, 0, 0, 0] - g["printed_expected"]) < g["printed_abs_precision"]
    assert out[0, 0, 0, 0] != g["faulty_kernel_output"]


# ----------------------------------------------------------------- generator
def test_generator_is_seeded_and_integer_valued():
    a = make_inputs(TINY_DECODE)
    b = make_inputs(TINY_DECODE)
    for key in ("q_idx", "key_state", "w_idx", "q", "k_cache", "v_cache"):
        assert torch.equal(a[key], b[key])
    qi = a["q_idx"].double()
    assert torch.equal(qi, qi.round()) and qi.abs().max() <= 8
    w = a["w_idx"]
    assert torch.equal(w, w.round()) and w.min() >= 1 and w.max() <= 4
    assert not torch.equal(a["q"], make_inputs(TINY_DECODE, seed=99)["q"])


def test_integer_scores_are_exact_in_fp32():
    x = make_inputs(scaled(TINY_DECODE, L=200))
    sc = oracle.indexer_scores(x["q_idx"], x["w_idx"], x["key_state"],
                               x["kv_len"].tolist(), 1)
    assert np.all(np.abs(sc) < 2 ** 24)
    assert np.array_equal(sc.astype(np.float32).astype(np.float64), sc)
