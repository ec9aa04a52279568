"""Plant plausible mistakes in the oracle and check that some pin fails.

Each mutant replaces one oracle function by a subtly wrong variant (a dropped
term, a wrong index or sign, a reversed tie-break, an exclusive bound); the
pins in test_oracle.py must reject every one of them.  The mistakes are
planted in the oracle only, on the CPU.
"""
import numpy as np
import pytest

import oracle
import oracle.dsa_oracle as od
import test_oracle as pins


def _scores_unweighted(q_idx_bs, w_bs, key_state_b, pos):
    return od.indexer_scores_row.__wrapped__(q_idx_bs, np.ones_like(od._f64(w_bs)),
                                             key_state_b, pos)


def _scores_exclusive_bound(q_idx_bs, w_bs, key_state_b, pos):
    return od.indexer_scores_row.__wrapped__(q_idx_bs, w_bs, key_state_b, pos - 1)


def _scores_key_transposed(q_idx_bs, w_bs, key_state_b, pos):
    ks = od._f64(key_state_b)
    ks = ks[:, ::-1].copy()          # dims paired in the wrong order
    return od.indexer_scores_row.__wrapped__(q_idx_bs, w_bs, ks, pos)


def _topk_high_index_ties(scores_row, pos, k):
    sc = od._f64(scores_row)
    n = min(max(pos + 1, 0), sc.shape[0])
    cand = np.arange(n)
    order = np.lexsort((-cand, -sc[:n]))
    out = np.full(k, -1)
    ch = np.sort(cand[order[:k]])
    out[:len(ch)] = ch
    return out


def _topk_lowest(scores_row, pos, k):
    return od.topk_row.__wrapped__(-od._f64(scores_row), pos, k)


def _topk_exclusive(scores_row, pos, k):
    return od.topk_row.__wrapped__(scores_row, pos - 1, k)


def _topk_unsorted(scores_row, pos, k):
    out = od.topk_row.__wrapped__(scores_row, pos, k)
    valid = out[out >= 0][::-1]
    res = out.copy()
    res[:len(valid)] = valid
    return res


def _attn_wrong_group(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, return_weights=False):
    # query head h reads KV head h % H_kv instead of h // ratio
    K, V = od._f64(k_b), od._f64(v_b)
    H_q, H_kv = od._f64(q_bs).shape[0], K.shape[1]
    ratio = H_q // H_kv
    perm = [(h % H_kv) for h in range(H_q)]
    Kx = np.stack([K[:, perm[g * ratio], :] for g in range(H_kv)], axis=1)
    Vx = np.stack([V[:, perm[g * ratio], :] for g in range(H_kv)], axis=1)
    return od.attention_row.__wrapped__(q_bs, Kx, Vx, idx_row, pos, kv_len_b, scale,
                                        return_weights)


def _attn_no_max_shift(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, return_weights=False):
    q, K, V = od._f64(q_bs), od._f64(k_b), od._f64(v_b)
    H_q, D = q.shape
    H_kv = K.shape[1]
    ratio = H_q // H_kv
    idx = np.asarray(idx_row)
    live = min(int(kv_len_b), K.shape[0], pos + 1)
    allowed = np.zeros(K.shape[0], bool)
    allowed[idx[(idx >= 0) & (idx < live)]] = True
    out = np.zeros((H_q, D))
    wts = np.zeros((H_q, K.shape[0]))
    if not allowed.any():
        return (out, wts) if return_weights else out
    for g in range(H_kv):
        hs = slice(g * ratio, (g + 1) * ratio)
        lg = scale * (q[hs] @ K[:, g, :].T)
        p = np.where(allowed, np.exp(np.minimum(lg, 700)), 0.0).astype(np.float32).astype(np.float64)
        out[hs] = (p @ V[:, g, :]) / p.sum(axis=1, keepdims=True)
        wts[hs] = p / p.sum(axis=1, keepdims=True)
    return (out, wts) if return_weights else out


def _attn_unscaled(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, return_weights=False):
    return od.attention_row.__wrapped__(q_bs, k_b, v_b, idx_row, pos, kv_len_b, 1.0,
                                        return_weights)


def _attn_exclusive(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, return_weights=False):
    return od.attention_row.__wrapped__(q_bs, k_b, v_b, idx_row, pos - 1, kv_len_b, scale,
                                        return_weights)


def _dequant_neighbour_head(codes, scale):
    return od._f64(codes) * np.roll(od._f64(scale), 1, axis=-1)[..., None]


def _dequant_divides(codes, scale):
    return od._f64(codes) / od._f64(scale)[..., None]


SCORE_PINS = [pins.test_scores_match_python_integer_brute_force,
              pins.test_scores_one_hot_keys_pick_weighted_query_column,
              pins.test_scores_scale_with_weights_and_flip_with_keys]
TOPK_PINS = [lambda: pins.test_topk_matches_brute_force_rank_definition(s) for s in range(6)] + [
    pins.test_topk_tie_storm_takes_lowest_indices, pins.test_topk_short_row_pads_with_minus_one,
    pins.test_topk_picks_highest_not_lowest, pins.test_topk_signed_zeros_tie_and_minus_inf_ranks_last]
ATTN_PINS = [lambda: pins.test_full_selection_equals_causal_gqa_attention(6, 2),
             lambda: pins.test_full_selection_equals_causal_gqa_attention(12, 1),
             pins.test_single_key_returns_its_value_row,
             pins.test_two_keys_follow_the_logistic_closed_form,
             pins.test_weights_sum_to_one_and_vanish_off_selection,
             pins.test_large_logit_gap_keeps_the_small_weight,
             pins.test_worked_example_from_the_pages]
DEQ_PINS = [pins.test_int8_generator_values_round_trip,
            pins.test_int8_path_equals_float_path_on_dequantised_cache]

MUTANTS = [
    ("indexer_scores_row", _scores_unweighted, SCORE_PINS),
    ("indexer_scores_row", _scores_exclusive_bound, SCORE_PINS),
    ("indexer_scores_row", _scores_key_transposed, SCORE_PINS),
    ("topk_row", _topk_high_index_ties, TOPK_PINS),
    ("topk_row", _topk_lowest, TOPK_PINS),
    ("topk_row", _topk_exclusive, TOPK_PINS),
    ("topk_row", _topk_unsorted, TOPK_PINS),
    ("attention_row", _attn_wrong_group, ATTN_PINS),
    ("attention_row", _attn_no_max_shift, ATTN_PINS),
    ("attention_row", _attn_unscaled, ATTN_PINS),
    ("attention_row", _attn_exclusive, ATTN_PINS),
    ("dequantize", _dequant_neighbour_head, DEQ_PINS),
    ("dequantize", _dequant_divides, DEQ_PINS),
]


def _caught(pin_list):
    for pin in pin_list:
        try:
            pin()
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name,mutant,pin_list", MUTANTS,
                         ids=[m[1].__name__ for m in MUTANTS])
def test_every_planted_mistake_is_caught(monkeypatch, name, mutant, pin_list):
    original = getattr(od, name)
    if not hasattr(original, "__wrapped__"):
        # keep a handle on the true function for mutants built on top of it
        def passthrough(*a, **kw):
            return original(*a, **kw)
        passthrough.__wrapped__ = original
        original = passthrough
    getattr(od, name).__wrapped__ = getattr(original, "__wrapped__", original)
    monkeypatch.setattr(od, name, mutant)
    monkeypatch.setattr(oracle, name, mutant)
    assert _caught(pin_list), f"planted mistake {mutant.__name__} passed every pin"
