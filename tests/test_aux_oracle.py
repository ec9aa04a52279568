"""Pins of the auxiliary-K/V attention oracle (oracle/aux_oracle.py), on the CPU."""
import numpy as np
import pytest
import torch

import oracle
import oracle.aux_oracle as ao


def _case(seed, B=2, S=4, L=40, H_q=6, H_kv=2, D=16, k=12, S_aux=4):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, S, H_q, D))
    kc = rng.standard_normal((B, L, H_kv, D))
    vc = rng.standard_normal((B, L, H_kv, D))
    ak = rng.standard_normal((B, S_aux, H_kv, D))
    av = rng.standard_normal((B, S_aux, H_kv, D))
    kv_len = [L, L - 9]
    idx = np.full((B, S, k), -1)
    for b in range(B):
        for s in range(S):
            pos = kv_len[b] - S + s
            idx[b, s] = np.sort(rng.choice(pos + 1, size=k, replace=False))
    return q, kc, vc, ak, av, kv_len, idx


def test_aux_equal_to_cache_rows_reproduces_plain_attention():
    q, kc, vc, ak, av, kv_len, idx = _case(1)
    S_aux = ak.shape[1]
    for b in range(2):
        lo = kv_len[b] - S_aux
        ak[b], av[b] = kc[b, lo:kv_len[b]], vc[b, lo:kv_len[b]]
        # every aux position selected in the plain run, so both see the same keys
        for s in range(q.shape[1]):
            pos = kv_len[b] - q.shape[1] + s
            extra = [p for p in range(lo, pos + 1)]
            keep = [j for j in idx[b, s] if 0 <= j < lo][: idx.shape[2] - len(extra)]
            row = np.full(idx.shape[2], -1)
            sel = sorted(keep + extra)
            row[:len(sel)] = sel
            idx[b, s] = row
    want = oracle.sparse_attention(q, kc, vc, idx, kv_len)
    got = ao.sparse_attention_with_aux(q, kc, vc, idx, kv_len, ak, av)
    assert np.allclose(got, want, rtol=1e-12, atol=1e-13)


def test_aux_alone_is_causal_attention():
    q, kc, vc, ak, av, kv_len, idx = _case(2)
    idx[:] = -1                                   # no cache key selected
    got = ao.sparse_attention_with_aux(q, kc, vc, idx, kv_len, ak, av)
    B, S, H_q, D = q.shape
    ratio = H_q // ak.shape[2]
    for b in range(B):
        qq = torch.from_numpy(q[b]).permute(1, 0, 2)                      # [H_q, S, D]
        kk = torch.from_numpy(ak[b]).permute(1, 0, 2).repeat_interleave(ratio, 0)
        vv = torch.from_numpy(av[b]).permute(1, 0, 2).repeat_interleave(ratio, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True)
        assert np.allclose(got[b], ref.permute(1, 0, 2).numpy(), rtol=1e-12, atol=1e-13)


def test_cache_rows_in_the_aux_range_are_ignored():
    q, kc, vc, ak, av, kv_len, idx = _case(3)
    a = ao.sparse_attention_with_aux(q, kc, vc, idx, kv_len, ak, av)
    kc2, vc2 = kc.copy(), vc.copy()
    for b in range(2):
        kc2[b, kv_len[b] - ak.shape[1]:kv_len[b]] *= 50.0
        vc2[b, kv_len[b] - ak.shape[1]:kv_len[b]] += 9.0
    b_ = ao.sparse_attention_with_aux(q, kc2, vc2, idx, kv_len, ak, av)
    assert np.array_equal(a, b_)


def test_constant_values_give_constant_output_and_weights_sum_to_one():
    q, kc, vc, ak, av, kv_len, idx = _case(4)
    vc[:] = 0.75
    av[:] = 0.75
    got = ao.sparse_attention_with_aux(q, kc, vc, idx, kv_len, ak, av)
    assert np.allclose(got, 0.75, rtol=1e-14)
    _, w = ao.attention_row_with_aux(q[0, 1], kc[0], vc[0], idx[0, 1], kv_len[0] - 4 + 1,
                                     kv_len[0], 0.25, ak[0], av[0], return_weights=True)
    assert np.allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    L = kc.shape[1]
    # aux tokens after the query's position carry no weight
    assert np.all(w[:, L + 2:] == 0.0)


# --------------------------------------------------------------- mutants
PINS = [test_aux_equal_to_cache_rows_reproduces_plain_attention, test_aux_alone_is_causal_attention,
        test_cache_rows_in_the_aux_range_are_ignored,
        test_constant_values_give_constant_output_and_weights_sum_to_one]
_true = ao.attention_row_with_aux


def _aux_not_causal(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, aux_k_b, aux_v_b,
                    return_weights=False):
    return _true(q_bs, k_b, v_b, idx_row, pos + 10 ** 6, kv_len_b, scale, aux_k_b, aux_v_b,
                 return_weights)


def _cache_range_kept(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, aux_k_b, aux_v_b,
                      return_weights=False):
    # cache keys in the aux range stay attendable (double counting)
    n = np.asarray(aux_k_b).shape[0]
    return _true(q_bs, k_b, v_b, idx_row, pos, kv_len_b + n, scale,
                 np.zeros((0,) + np.asarray(aux_k_b).shape[1:]),
                 np.zeros((0,) + np.asarray(aux_v_b).shape[1:]), return_weights)


def _aux_shifted(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, aux_k_b, aux_v_b,
                 return_weights=False):
    return _true(q_bs, k_b, v_b, idx_row, pos - 1, kv_len_b, scale, aux_k_b, aux_v_b,
                 return_weights)


MUTANTS = [_aux_not_causal, _cache_range_kept, _aux_shifted]


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m.__name__ for m in MUTANTS])
def test_every_planted_mistake_is_caught(monkeypatch, mutant):
    monkeypatch.setattr(ao, "attention_row_with_aux", mutant)
    caught = False
    for pin in PINS:
        try:
            pin()
        except Exception:
            caught = True
            break
    assert caught, f"planted mistake {mutant.__name__} passed every pin"
