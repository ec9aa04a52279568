"""CPU oracle of sparse attention with auxiliary K/V -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module.  The HIP library never calls it and shares no code with it.

Auxiliary K/V (ORT PR #33997, review and follow-up commit: auxiliary K/V are
kept in their own floating type next to an FP16 main cache, converting BF16
auxiliary values to FP16 can overflow, and "auxiliary-range" regressions
cover them) are the step's fresh keys and values, not yet written to the
cache, that take part in the same softmax as the selected cache keys.

Readings where the pages are silent:
  * aux_k, aux_v [B, S_aux, H_kv, D] hold the tokens at positions
    kv_len[b] - S_aux + t (kv_len counts them), in their own dtype, used
    as is;
  * query token s (position pos = kv_len[b] - S + s) attends to aux token t
    iff its position is <= pos (causal) and >= 0;
  * cache entries at positions >= kv_len[b] - S_aux are not attended (those
    tokens are not in the cache yet; the aux copy is the one that counts),
    so selected indices in that range are ignored;
  * one softmax over the allowed cache keys and the allowed aux keys, in
    FP64, dense masked form as in dsa_oracle.attention_row.

Pins (tests/test_aux_oracle.py): aux equal to the cache rows reproduces
plain sparse attention, aux alone is causal attention from torch's SDPA,
cache rows in the aux range have no effect, constant V, weight sums.
"""
import numpy as np

from .dsa_oracle import _f64, dequantize, query_position


def attention_row_with_aux(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale, aux_k_b, aux_v_b,
                           return_weights=False):
    """One query token: q_bs [H_q, D]; k_b, v_b [L, H_kv, D] (dequantised);
    idx_row [k]; aux_k_b, aux_v_b [S_aux, H_kv, D]."""
    q, K, V = _f64(q_bs), _f64(k_b), _f64(v_b)
    AK, AV = _f64(aux_k_b), _f64(aux_v_b)
    H_q, D = q.shape
    L, H_kv = K.shape[0], K.shape[1]
    n_aux = AK.shape[0]
    ratio = H_q // H_kv
    idx = np.asarray(idx_row, dtype=np.int64)
    cache_live = min(int(kv_len_b) - n_aux, L, pos + 1)
    allowed = np.zeros(L + n_aux, dtype=bool)
    ok = idx[(idx >= 0) & (idx < cache_live)]
    allowed[ok] = True
    aux_pos = int(kv_len_b) - n_aux + np.arange(n_aux)
    allowed[L:] = (aux_pos >= 0) & (aux_pos <= pos)
    Kx = np.concatenate([K, AK], axis=0)
    Vx = np.concatenate([V, AV], axis=0)
    out = np.zeros((H_q, D))
    weights = np.zeros((H_q, L + n_aux))
    if not allowed.any():
        return (out, weights) if return_weights else out
    for g in range(H_kv):
        heads = slice(g * ratio, (g + 1) * ratio)
        logits = scale * (q[heads] @ Kx[:, g, :].T)
        logits[:, ~allowed] = -np.inf
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        denom = p.sum(axis=1, keepdims=True)
        out[heads] = (p @ Vx[:, g, :]) / denom
        weights[heads] = p / denom
    return (out, weights) if return_weights else out


def sparse_attention_with_aux(q, k_cache, v_cache, indices, kv_len, aux_k, aux_v, scale=None,
                              k_scale=None, v_scale=None, rows=None):
    """Output float64 [B, S, H_q, D] (or only `rows`) of sparse attention
    over the selected cache keys plus the auxiliary keys."""
    qf = _f64(q)
    B, S, H_q, D = qf.shape
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    idx = np.asarray(indices.cpu() if hasattr(indices, "cpu") else indices)
    out = np.zeros((B, S, H_q, D))
    rows = [(b, s) for b in range(B) for s in range(S)] if rows is None else rows
    by_b = {}
    for b, s in rows:
        by_b.setdefault(b, []).append(s)
    for b, ss in by_b.items():
        if k_scale is not None:
            Kb = dequantize(k_cache[b], k_scale[b])
            Vb = dequantize(v_cache[b], v_scale[b])
        else:
            Kb, Vb = _f64(k_cache[b]), _f64(v_cache[b])
        for s in ss:
            pos = query_position(kv_len[b], S, s)
            out[b, s] = attention_row_with_aux(qf[b, s], Kb, Vb, idx[b, s], pos, kv_len[b],
                                               scale, aux_k[b], aux_v[b])
    return out
