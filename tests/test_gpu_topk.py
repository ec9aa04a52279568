"""Top-k on the GPU vs the oracle's full stable sort: indices bit-exact.

Score matrices are generated on the CPU and uploaded, so the GPU kernel and
the oracle read the same FP32 values.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_synth import indexer_like_scores, integer_scores
from gpu_util import DEV, dsa, first_mismatch, run_topk, say  # noqa: F401

pytestmark = pytest.mark.gpu


def _check(dsa, scores_cpu, kv_len, k, rows=None, what=""):
    B, S, L = scores_cpu.shape
    say(f"topk {what} B={B} S={S} L={L} k={k} ws={dsa.dsa_topk_workspace_bytes(B, S, L, k)}")
    g_scores = scores_cpu.to(DEV)
    g_kv = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    idx = run_topk(dsa, g_scores, g_kv, k)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    rows = [(b, s) for b in range(B) for s in range(S)] if rows is None else rows
    for b, s in rows:
        pos = kv_len[b] - S + s
        want = oracle.topk_row(scores_cpu[b, s], pos, k)
        assert np.array_equal(got[b, s], want), f"{what} row ({b},{s}): {first_mismatch(got[b, s], want)}"
    return got


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("B,S,L,k", [(1, 8, 32768, 2048), (1, 300, 5000, 512), (2, 4, 20000, 100),
                                     (1, 1, 1024, 128), (1, 8, 262144, 2048)])
def test_topk_normal_floats(dsa, B, S, L, k):
    sc = torch.from_numpy(rng(L + k).standard_normal(size=(B, S, L)).astype(np.float32))
    _check(dsa, sc, [L] * B, k, what="normal")


@pytest.mark.parametrize("B,S,L,k", [(1, 8, 32768, 2048), (1, 200, 3000, 256), (1, 8, 70000, 1000)])
def test_topk_heavy_ties(dsa, B, S, L, k):
    _check(dsa, integer_scores(rng(7), (B, S, L), -20, 20), [L] * B, k, what="ints[-20,20]")
    _check(dsa, integer_scores(rng(8), (B, S, L), -1, 1), [L] * B, k, what="ints[-1,1]")


@pytest.mark.parametrize("B,S,L,k", [(1, 8, 32768, 2048), (1, 200, 3000, 256), (1, 3, 50000, 4096)])
def test_topk_tie_storm_takes_lowest_indices(dsa, B, S, L, k):
    got = _check(dsa, torch.full((B, S, L), 3.0), [L] * B, k, what="tie storm")
    assert np.array_equal(got[0, 0], np.arange(k))


def test_topk_narrow_bin_forces_deep_descent(dsa):
    # All keys share their top 11 bits: the first bin holds every key, so
    # both plans must descend through all three radix levels.
    r = rng(9)
    for (B, S, L, k) in [(1, 8, 40000, 2048), (1, 150, 9000, 700)]:
        base = r.integers(0, 1 << 16, size=(B, S, L))
        sc = torch.from_numpy((1.0 + base.astype(np.float64) * 2.0 ** -23).astype(np.float32))
        _check(dsa, sc, [L] * B, k, what="narrow")


def test_topk_short_rows_and_ragged_lengths(dsa):
    r = rng(10)
    _check(dsa, torch.from_numpy(r.standard_normal((1, 4, 100)).astype(np.float32)), [100], 128,
           what="k > n")
    sc = torch.from_numpy(r.standard_normal((3, 8, 40000)).astype(np.float32))
    got = _check(dsa, sc, [40000, 20000, 5], 1000, what="ragged multi")
    assert np.all(got[2, :3] == -1)        # pos < 0: nothing to select
    sc = torch.from_numpy(r.standard_normal((3, 50, 4000)).astype(np.float32))
    _check(dsa, sc, [4000, 2500, 60], 300, what="ragged row")


def test_topk_ignores_poison_beyond_position(dsa):
    r = rng(11)
    B, S, L, k = 1, 8, 30000, 2048
    sc = torch.from_numpy(r.standard_normal((B, S, L)).astype(np.float32))
    kv = 20000
    for s in range(S):                          # +inf beyond each row's position
        sc[0, s, kv - S + s + 1:] = float("inf")
    _check(dsa, sc, [kv], k, what="poison")


def test_topk_signed_zero_and_minus_inf(dsa):
    r = rng(12)
    for (B, S, L, k) in [(1, 8, 20000, 3000), (1, 130, 2000, 600)]:
        choice = r.integers(0, 4, size=(B, S, L))
        vals = np.array([0.0, -0.0, -np.inf, 1.0], dtype=np.float32)
        sc = torch.from_numpy(vals[choice])
        _check(dsa, sc, [L] * B, k, what="zeros/-inf")


def test_topk_denormal_and_signed_zero_thresholds(dsa):
    # Thresholds among denormals of either sign and signed zeros: the plans
    # that test hits on floats must agree with the key order there (no
    # flushing to zero, -0.0 equal to +0.0).
    r = rng(17)
    tiny = np.float32(2.0 ** -149)
    for (B, S, L, k) in [(1, 8, 32768, 2048), (1, 130, 3000, 256), (1, 8, 40000, 2048)]:
        for lo, hi in ((-40, 41), (-40, 1)):
            codes = r.integers(lo, hi, size=(B, S, L))
            sc = codes.astype(np.float32) * tiny
            sc[(codes == 0) & (r.random(size=codes.shape) < 0.5)] = np.float32(-0.0)
            _check(dsa, torch.from_numpy(sc), [L] * B, k, what=f"denormals[{lo},{hi})")


def test_topk_prefill_128k_shape(dsa):
    sc = indexer_like_scores(rng(13), (1, 2048, 131072))
    _check(dsa, sc, [131072], 2048, rows=[(0, s) for s in (0, 1, 500, 1023, 1024, 2047)],
           what="prefill_128k-shaped")


def test_topk_k_beyond_list_capacity_uses_exact_fallback(dsa):
    r = rng(14)
    # streaming plan (many rows) and split plan (few long rows), k above the list capacity
    _check(dsa, integer_scores(r, (1, 130, 12000), -50, 50), [12000], 5000, what="row k>cap")
    _check(dsa, torch.from_numpy(r.standard_normal((1, 4, 40000)).astype(np.float32)), [40000],
           9000, what="multi k>cap")


def _sample_positions(n, sample=8192, block=256):
    nb = sample // block
    return np.concatenate([np.arange(b * (n - block) // (nb - 1), b * (n - block) // (nb - 1) + block)
                           for b in range(nb)])


@pytest.mark.parametrize("B,S,L,k,sample,over", [
    (1, 8, 30000, 2048, 2048, "row"),        # LDS-resident rows: sample over each row
    (1, 8, 40000, 2048, 2048, "bound"),      # split plan: sample over the bound max_kv_len
    (1, 8, 300000, 2048, 4096, "bound"),     # split plan, longer rows: a larger sample
    (1, 130, 40000, 2048, 8192, "row")])     # streaming rows
def test_topk_sample_heavy_rows_use_exact_fallback(dsa, B, S, L, k, sample, over):
    # White-box: large scores exactly at the keys the threshold sample reads,
    # so fewer than k keys reach the estimated threshold and the exact
    # fallback must produce the result.
    r = rng(15)
    sc = r.integers(-100, 100, size=(B, S, L)).astype(np.float32)
    for s in range(S):
        n = L - S + s + 1
        pos = _sample_positions(n if over == "row" else L, sample)
        pos = pos[pos < n]
        sc[0, s, pos] = 1000.0 + r.integers(0, 50, size=pos.shape[0])
    _check(dsa, torch.from_numpy(sc), [L], k, what=f"sample-heavy/{sample}/{over}")


def test_topk_split_rows_far_below_the_bound_resample(dsa):
    # Rows much shorter than max_kv_len: the sample spread over the bound
    # leaves them too few valid keys, so their chunk workgroups sample again
    # over the row itself (and a row at most k long just lists every key).
    r = rng(21)
    L, k = 262144, 2048
    sc = torch.from_numpy(np.round(r.standard_normal((4, 2, L)) * 2100).astype(np.float32))
    _check(dsa, sc, [L, 3000, 70001, 2049], k, what="split, short rows under a long bound")


def test_topk_split_chunk_overflow_falls_back_to_exact(dsa):
    # 100 rows of 400000 keys: whole-chunk slots would exceed the workspace
    # budget, so chunks get a few times their expected candidate count.  With
    # the top keys packed into each row's most recent 12000 positions those
    # chunks overflow and the row is selected exactly from the whole row.
    r = rng(22)
    B, S, L, k = 1, 100, 400000, 2048
    sc = r.standard_normal((B, S, L)).astype(np.float32)
    for s in range(S):
        n = L - S + s + 1
        sc[0, s, n - 12000:n] += 6.0
    _check(dsa, torch.from_numpy(sc), [L], k, rows=[(0, 0), (0, 57), (0, 99)],
           what="split, overflowing chunks")


@pytest.mark.parametrize("B,S,L,k,span", [(1, 8, 262144, 2048, 3000),    # last chunks overflow their slots
                                          (2, 4, 100000, 1500, 40000)])  # spread over many chunks
def test_topk_recency_clustered_candidates(dsa, B, S, L, k, span):
    # Scores with the top-k concentrated in the most recent `span` positions
    # of each row: in the split plan the chunks there hold more candidates
    # than the select kernel loads up front, so the row takes the general
    # path that gathers every chunk's list in order.
    r = rng(16)
    sc = r.standard_normal((B, S, L)).astype(np.float32)
    kv = [L] * B
    for b in range(B):
        for s in range(S):
            n = kv[b] - S + s + 1
            sc[b, s, max(0, n - span):n] += 4.0
    _check(dsa, torch.from_numpy(sc), kv, k, what=f"recency/{span}")


def test_topk_ties_across_chunks_keep_lowest_indices(dsa):
    # 4000 keys share the top value 2.0 at random positions over the whole
    # row, the rest lie in [0, 1): the k-th largest value is 2.0 and only the
    # 3000 lowest-indexed of its keys (spread over every chunk) may be taken.
    r = rng(17)
    B, S, L, k = 1, 8, 90000, 3000
    sc = r.random((B, S, L)).astype(np.float32)
    for s in range(S):
        sc[0, s, r.choice(L - S, size=4000, replace=False)] = 2.0
    got = _check(dsa, torch.from_numpy(sc), [L], k, what="ties across chunks")
    tied = np.flatnonzero(sc[0, 0, :L - S + 1] == 2.0)
    assert np.array_equal(got[0, 0], tied[:k])


def test_topk_resident_rows_unaligned_short_and_at_capacity(dsa):
    # Few rows of at most 32768 keys: rows whose length is not a multiple of
    # 4 (element loads), rows short enough for the whole row to be the
    # threshold sample, rows with k close to their length and heavy ties
    # (candidate counts around the list capacity of 4096), and k = 1.
    r = rng(18)
    sc = torch.from_numpy(r.standard_normal((1, 8, 2101)).astype(np.float32))
    _check(dsa, sc, [2101], 2000, what="resident short, L%4=1")
    sc = torch.from_numpy(r.standard_normal((2, 8, 30001)).astype(np.float32))
    _check(dsa, sc, [30001, 15000], 2048, what="resident ragged, L%4=1")
    sc = integer_scores(r, (1, 4, 4097), -30, 30)
    _check(dsa, sc, [4097], 4000, what="resident near capacity")
    sc = torch.from_numpy(r.standard_normal((2, 8, 32768)).astype(np.float32))
    _check(dsa, sc, [32768, 9000], 1, what="resident k=1, ragged")


def test_topk_short_runtime_bound_in_a_long_cache_uses_the_resident_plan(dsa):
    # A 256K-capacity cache whose live lengths stay under 32768 keys: the
    # plan follows the runtime bound max_kv_len, and the resident workgroup
    # reads only the bound's span of each row.
    B, S, L, k = 2, 4, 262144, 2048
    plan = dsa.plan_fields(dsa.dsa_describe_plan(dsa.DSA_PLAN_TOPK, B, S, L, 30001, k=k))
    assert plan["plan"] == "resident" and plan["workspace"] == "0"
    r = rng(23)
    sc = r.standard_normal((B, S, L)).astype(np.float32)
    sc[:, :, 30001:] = np.inf                   # beyond the bound: never read
    kv = [30001, 12000]
    g_kv = torch.tensor(kv, dtype=torch.int32, device=DEV)
    for what, m in (("normal", sc), ("indexer-like", indexer_like_scores(r, (B, S, L)).numpy())):
        m = m.copy()
        m[:, :, 30001:] = np.inf
        idx = run_topk(dsa, torch.from_numpy(m).to(DEV), g_kv, k, max_kv_len=30001)
        got = idx.cpu().numpy()
        for b in range(B):
            for s in range(S):
                want = oracle.topk_row(m[b, s], kv[b] - S + s, k)
                assert np.array_equal(got[b, s], want), \
                    f"bounded resident {what} row ({b},{s}): {first_mismatch(got[b, s], want)}"


def test_topk_streaming_rows_unaligned_and_ragged(dsa):
    # The many-rows plan with row lengths that are not a multiple of 4
    # (element loads, no 16-byte path), ragged sequences, a sequence whose
    # rows hold fewer keys than k, and heavy ties.
    r = rng(20)
    sc = torch.from_numpy(r.standard_normal((2, 130, 5001)).astype(np.float32))
    _check(dsa, sc, [5001, 3333], 512, what="stream, L%4=1, ragged")
    sc = integer_scores(r, (3, 64, 9002), -15, 15)
    _check(dsa, sc, [9002, 600, 64], 700, what="stream, L%4=2, short rows, ties")
    sc = torch.from_numpy(r.standard_normal((1, 129, 20000)).astype(np.float32))
    _check(dsa, sc, [20000], 2048, what="stream, L%4=0")


def test_topk_very_long_rows(dsa):
    # Few rows of 4.5M keys: more chunks per row than the select kernel's
    # registers hold, so it takes the general path (and, with more candidates
    # than its LDS list holds, the exact selection over the whole row).
    r = rng(19)
    sc = torch.from_numpy(r.standard_normal((1, 2, 4_500_000)).astype(np.float32))
    _check(dsa, sc, [4_500_000], 2048, what="4.5M keys")



@pytest.mark.parametrize("B,S,L,k,kv,bound", [
    (1, 1, 1024, 128, [1024], 1024),                  # one decode row, 4 keys per thread
    (1, 8, 4096, 2048, [4096], 4096),                 # 16 keys per thread, k = half the row
    (1, 2, 500, 7, [500], 500),                       # 4 keys per thread, threads past the row
    (3, 50, 4000, 300, [4000, 2500, 60], 4000),       # 150 rows, ragged
    (2, 7, 3001, 1, [3001, 17], 3001),                # L % 4 = 1 (element loads), k = 1
    (1, 9, 2050, 2045, [2050], 2050),                 # k close to n, k >= n on the first rows
    (2, 4, 262144, 512, [3000, 4096], 4096)])         # a long cache under a short runtime bound
def test_topk_small_plan_short_rows(dsa, B, S, L, k, kv, bound):
    # Rows of at most 4096 keys by the runtime bound: one 256-thread
    # workgroup per row holds the row in registers and selects on its radix
    # digits directly.
    plan = dsa.plan_fields(dsa.dsa_describe_plan(dsa.DSA_PLAN_TOPK, B, S, L, bound, k=k))
    assert plan["plan"] == "small" and plan["workspace"] == "0"
    r = rng(50 + L + k)
    for what, sc in (("normal", torch.from_numpy(r.standard_normal((B, S, L)).astype(np.float32))),
                     ("ints[-3,3]", integer_scores(r, (B, S, L), -3, 3)),
                     ("indexer-like", indexer_like_scores(r, (B, S, L)))):
        g_kv = torch.tensor(kv, dtype=torch.int32, device=DEV)
        idx = run_topk(dsa, sc.to(DEV), g_kv, k, max_kv_len=bound)
        got = idx.cpu().numpy()
        for b in range(B):
            for s in range(S):
                want = oracle.topk_row(sc[b, s], kv[b] - S + s, k)
                assert np.array_equal(got[b, s], want), \
                    f"small {what} row ({b},{s}): {first_mismatch(got[b, s], want)}"


def test_topk_small_plan_exact_digits_and_deep_levels(dsa):
    # Short rows whose k-th key sits in a cluster of tied or nearly equal keys
    # under a wide key range (keys of +-1e30 at two positions), so that the
    # chosen bin holds more than 64 keys at every level down to the last
    # digit; a row of one value; a row of two values.
    r = rng(60)
    B, S, L = 1, 6, 4096
    sc = np.empty((B, S, L), dtype=np.float32)
    sc[0, 0] = 1.0 + r.integers(0, 256, size=L) * 2.0 ** -23         # low 8 bits differ
    sc[0, 1] = 1.0 + r.integers(0, 1 << 16, size=L) * 2.0 ** -23     # low 16 bits differ
    sc[0, 2] = 1.0 + r.integers(0, 1 << 24, size=L) * 2.0 ** -23     # low 24 bits differ
    for s in range(3):
        sc[0, s, 17], sc[0, s, 3000] = 1e30, -1e30
    sc[0, 3] = 7.0
    sc[0, 4] = np.where(np.arange(L) % 3 == 0, 5.0, 4.0)
    sc[0, 5] = r.standard_normal(L)
    sc = torch.from_numpy(sc)
    for k in (1, 2, 100, 1365, 1366, 1367, 4000, 4090):
        _check(dsa, sc, [L], k, what=f"small deep k={k}")


@pytest.mark.parametrize("B,S,L,k,kv", [
    (8, 8, 65536, 2048, [65536, 60000, 4000, 2049, 2048, 9, 65536, 31000]),   # 64 rows, ragged
    (1, 3, 100003, 1500, [100003]),                # 3 rows, L % 4 = 3
    (1, 1, 262144, 4096, [262144])])               # one long row, k = 4096
def test_topk_few_rows_indexer_like_and_normal(dsa, B, S, L, k, kv):
    r = rng(30 + B * S)
    _check(dsa, indexer_like_scores(r, (B, S, L)), kv, k, what="indexer-like")
    _check(dsa, torch.from_numpy(r.standard_normal((B, S, L)).astype(np.float32)), kv, k,
           what="normal")


@pytest.mark.parametrize("L", [32768, 262144])
def test_topk_repeated_calls_and_graph_replays(dsa, L):
    # No state carries from one call to the next: 40 calls in a row and 5
    # replays of a captured graph of 20 calls (one shared workspace for the
    # two-kernel plan at 256K), each result checked.
    B, S, k = 1, 8, 2048
    r = rng(40)
    sc_cpu = indexer_like_scores(r, (B, S, L))
    want = np.stack([oracle.topk_row(sc_cpu[0, s], L - S + s, k) for s in range(S)])
    sc = sc_cpu.to(DEV)
    kv = torch.tensor([L], dtype=torch.int32, device=DEV)
    outs = [torch.full((B, S, k), -7, dtype=torch.int32, device=DEV) for _ in range(40)]
    for o in outs:
        dsa.dsa_topk(sc, kv, k, o)
    torch.cuda.synchronize()
    for i, o in enumerate(outs):
        assert np.array_equal(o.cpu().numpy()[0], want), f"call {i}"
    need = dsa.dsa_topk_workspace_bytes(B, S, L, k)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV) if need > 0 else None
    gouts = [torch.full((B, S, k), -7, dtype=torch.int32, device=DEV) for _ in range(20)]
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(g, stream=stream):
            for o in gouts:
                dsa.dsa_topk(sc, kv, k, o, workspace=ws)
    for rep in range(5):
        for o in gouts:
            o.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, o in enumerate(gouts):
            assert np.array_equal(o.cpu().numpy()[0], want), f"replay {rep} call {i}"


def test_topk_two_streams_at_once(dsa):
    # Calls in flight together on two streams, each with its own workspace.
    B, S, L, k = 1, 8, 65536, 2048
    r = rng(41)
    a_cpu = indexer_like_scores(r, (B, S, L))
    b_cpu = torch.from_numpy(r.standard_normal((B, S, L)).astype(np.float32))
    kv = torch.tensor([L], dtype=torch.int32, device=DEV)
    a, b = a_cpu.to(DEV), b_cpu.to(DEV)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for rep in range(6):
        oa = torch.full((B, S, k), -7, dtype=torch.int32, device=DEV)
        ob = torch.full((B, S, k), -7, dtype=torch.int32, device=DEV)
        with torch.cuda.stream(s1):
            dsa.dsa_topk(a, kv, k, oa)
        with torch.cuda.stream(s2):
            dsa.dsa_topk(b, kv, k, ob)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    want_a = np.stack([oracle.topk_row(a_cpu[0, s], L - S + s, k) for s in range(S)])
    want_b = np.stack([oracle.topk_row(b_cpu[0, s], L - S + s, k) for s in range(S)])
    for rep, (oa, ob) in enumerate(outs):
        assert np.array_equal(oa.cpu().numpy()[0], want_a), f"stream 1, call {rep}"
        assert np.array_equal(ob.cpu().numpy()[0], want_b), f"stream 2, call {rep}"
