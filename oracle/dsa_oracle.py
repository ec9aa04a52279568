"""CPU oracle for dynamic sparse GQA attention -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the bench's CPU-baseline leg may import
this module.  The HIP library never calls it, and it shares no code with the
HIP library: it computes every quantity from its plain definition, in FP64,
with NumPy primitives (matmul, exp, lexsort) as the only building blocks.

The method (ORT PR #33997 "Support FP16 KV cache and FP16 query/key in
DynamicSparseAttention<BFloat16> ...", Description item 2 and its test names
"SelectedOnly..."; ORT PR #33802 "Optimize Qwen3.8-Flash-Next DSA, Indexer,
HC, and QMoE kernels for SM12x and 256K context", Summary items 1-2) has three
stages:

1. indexer score of cached token j for query token (b, s): the per-head dot
   products of the indexer query heads with the token's indexer key, reduced
   over the heads with per-head weights,
       score[b,s,j] = sum_h w[b,s,h] * (q_idx[b,s,h,:] . key_state[b,j,:]),
   defined for j <= pos(b,s) = kv_len[b] - S + s (causal, own token included);
2. per-query top-k: the k highest-scoring keys among 0..pos, equal scores
   broken toward the lower index, listed in ascending index order and padded
   with -1 when fewer than k keys exist;
3. softmax attention of every query head over only the selected keys, with
   query head h reading KV head h // (H_q / H_kv); an INT8 cache holds codes
   and one FP32 scale per token per KV head for K and for V.

Readings where the pages are silent (all listed in the design notes): no
per-head nonlinearity and no scale in the score; one key-state vector per
token shared by all indexer heads; ascending output order; -1 padding;
softmax scale 1/sqrt(D) unless given; a row with no valid selected key yields
zeros.

Pins (tests/test_oracle.py): Python-integer brute force of the scores,
one-hot key special case, brute-force rank definition of the top-k, tie
storms, nesting, equality with ordinary causal GQA attention from torch's
scaled_dot_product_attention when every key is selected, constant V, weight
sums, single-key and two-key closed forms, permutation invariance, INT8
round trip and the pages' large-value-scale worked example.
"""
import numpy as np


def _f64(x):
    """Exact FP64 copy of a host tensor or array (every storage dtype embeds)."""
    if hasattr(x, "detach"):
        x = x.detach().cpu()
        if x.dtype.is_floating_point:
            x = x.double()
        return x.numpy().astype(np.float64, copy=False)
    return np.asarray(x, dtype=np.float64)


def query_position(kv_len_b, S, s):
    """Absolute position of query token s of a sequence holding kv_len_b tokens."""
    return int(kv_len_b) - S + s


# ---------------------------------------------------------------- 1. scores
def indexer_scores_row(q_idx_bs, w_bs, key_state_b, pos):
    """Scores of one query token against every cached token.

    q_idx_bs [H_idx, D_idx], w_bs [H_idx], key_state_b [L, D_idx].
    Returns float64 [L]; entries j > pos are NaN (not defined by the method).
    Per-head contraction first, then the weighted reduction over heads
    (ORT PR #33802, Summary item 2: per-head scoring reduced over 16 heads).
    """
    q = _f64(q_idx_bs)
    w = _f64(w_bs)
    ks = _f64(key_state_b)
    per_head = q @ ks.T                  # [H_idx, L]: q_idx_h . key_state_j
    score = w @ per_head                 # sum_h w_h * (q_idx_h . key_state_j)
    score[max(pos + 1, 0):] = np.nan
    return score


def indexer_scores(q_idx, w, key_state, kv_len, S):
    """All scores, float64 [B, S, L]; NaN where j > pos(b, s)."""
    q, wf, ks = _f64(q_idx), _f64(w), _f64(key_state)
    B, L = ks.shape[0], ks.shape[1]
    out = np.full((B, S, L), np.nan)
    for b in range(B):
        for s in range(S):
            out[b, s] = indexer_scores_row(q[b, s], wf[b, s], ks[b],
                                           query_position(kv_len[b], S, s))
    return out


# ---------------------------------------------------------------- 2. top-k
def topk_row(scores_row, pos, k):
    """Top-k of one row by a full stable sort.

    Candidates are keys 0..pos (clamped to the row).  Keys are ordered by
    score, highest first, equal scores by lower index first; the first k are
    kept and listed in ascending index order; missing slots hold -1.
    (Per-2048-key chunking and radix merging on ORT PR #33802, Summary item 2,
    change the cost, never the selected set.)
    """
    sc = _f64(scores_row)
    n = min(max(pos + 1, 0), sc.shape[0])
    cand = np.arange(n)
    order = np.lexsort((cand, -sc[:n]))   # primary: score desc; secondary: index asc
    chosen = np.sort(cand[order[:k]])
    out = np.full(k, -1, dtype=np.int64)
    out[:chosen.shape[0]] = chosen
    return out


def topk(scores, kv_len, S, k):
    """int64 [B, S, k] selected indices for every row of `scores` [B, S, L]."""
    sc = _f64(scores)
    B = sc.shape[0]
    out = np.empty((B, S, k), dtype=np.int64)
    for b in range(B):
        for s in range(S):
            out[b, s] = topk_row(sc[b, s], query_position(kv_len[b], S, s), k)
    return out


# ---------------------------------------------------------------- INT8 cache
def dequantize(codes, scale):
    """codes [..., D] (integers) times one scale per row scale [...], in FP64.

    An 8-bit code times an FP32 scale is exact in FP64.
    """
    return _f64(codes) * _f64(scale)[..., None]


# ---------------------------------------------------------------- 3. attention
def attention_row(q_bs, k_b, v_b, idx_row, pos, kv_len_b, scale,
                  return_weights=False):
    """Sparse GQA attention of one query token.

    q_bs [H_q, D]; k_b, v_b [L, H_kv, D] (already dequantised); idx_row [k].
    Dense form of the definition: the logits of every head against every
    cached key are formed, every key outside the selected set (or beyond
    pos, or beyond the live length) is masked to -inf, and
        out_h = sum_j p_j v_j / sum_j p_j,  p_j = exp(logit_j - max_j logit_j).
    A row with no valid selected key gives zeros.
    """
    q, K, V = _f64(q_bs), _f64(k_b), _f64(v_b)
    H_q, D = q.shape
    L, H_kv = K.shape[0], K.shape[1]
    ratio = H_q // H_kv
    idx = np.asarray(idx_row, dtype=np.int64)
    live = min(int(kv_len_b), L, pos + 1)
    ok = idx[(idx >= 0) & (idx < live)]
    allowed = np.zeros(L, dtype=bool)
    allowed[ok] = True
    out = np.zeros((H_q, D))
    weights = np.zeros((H_q, L))
    if not allowed.any():
        return (out, weights) if return_weights else out
    for g in range(H_kv):
        heads = slice(g * ratio, (g + 1) * ratio)
        logits = scale * (q[heads] @ K[:, g, :].T)        # [ratio, L], dense
        logits[:, ~allowed] = -np.inf
        m = logits.max(axis=1, keepdims=True)
        p = np.exp(logits - m)
        denom = p.sum(axis=1, keepdims=True)
        out[heads] = (p @ V[:, g, :]) / denom
        weights[heads] = p / denom
    return (out, weights) if return_weights else out


def sparse_attention(q, k_cache, v_cache, indices, kv_len, scale=None,
                     k_scale=None, v_scale=None, rows=None):
    """Attention output float64 [B, S, H_q, D] (or only `rows`).

    q [B, S, H_q, D]; caches [B, L, H_kv, D]; indices [B, S, k];
    k_scale / v_scale [B, L, H_kv] for an INT8 cache, else None.
    scale defaults to 1/sqrt(D).  `rows` is an optional list of (b, s): only
    those rows are computed, the rest stay zero.
    """
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
            out[b, s] = attention_row(qf[b, s], Kb, Vb, idx[b, s], pos,
                                      kv_len[b], scale)
    return out
