"""The C-ABI library loads, exports every symbol include/dsa.h declares, and
rejects invalid calls on the host before any device work (CPU only).

Every call here fails validation, so no pointer is ever dereferenced and no
kernel is launched; the fake addresses are never touched.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")
LIBPATH = os.path.join(ROOT, "sparse_gqa_attention_amd", "libdsa.so")

A16 = 0x100000          # a 16-byte-aligned fake address (never dereferenced)
MIS = 0x100004          # misaligned fake address


@pytest.fixture(scope="module")
def dsa():
    if not os.path.exists(LIBPATH):
        import __graft_entry__
        __graft_entry__.build()
    import sparse_gqa_attention_amd as m
    return m


def declared_functions(header=HEADER):
    text = open(header).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z_0-9]+)\s*\(", text)))


def test_header_and_library_agree(dsa):
    names = declared_functions()
    assert len(names) == 13
    lib = ctypes.CDLL(LIBPATH)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dsa.h but not exported"
    assert sorted(dsa.EXPORTS) == names
    version = int(re.search(r"#define DSA_ABI_VERSION (\d+)", open(HEADER).read()).group(1))
    assert dsa.dsa_abi_version() == version


def _status(name):
    return {"DSA_OK": 0, "INVALID": 1, "UNSUPPORTED": 2, "MISALIGNED": 3, "WS": 4}[name]


def test_indexer_validation(dsa):
    L = dsa.LIB
    args = dict(q=A16, w=A16, ks=A16, dt=2, kv=A16, B=1, S=8, H=16, Di=64, Lc=4096, mx=4096, sc=A16)

    def call(**kw):
        a = dict(args, **kw)
        return L.dsa_indexer_score(a["q"], a["w"], a["ks"], a["dt"], a["kv"], a["B"], a["S"],
                                   a["H"], a["Di"], a["Lc"], a["mx"], a["sc"], None)
    assert call(H=17) == _status("UNSUPPORTED")
    assert call(H=0) == _status("UNSUPPORTED")
    assert call(Di=48) == _status("UNSUPPORTED")
    assert call(dt=0) == _status("UNSUPPORTED")
    assert "BF16" in dsa.dsa_last_error()
    assert call(dt=3) == _status("UNSUPPORTED")
    assert call(mx=4097) == _status("INVALID")
    assert call(Lc=(1 << 27) + 1, mx=4096) == _status("UNSUPPORTED")   # 32-bit score offsets
    assert "2^27" in dsa.dsa_last_error()
    assert call(B=-1) == _status("INVALID")
    assert call(q=None) == _status("INVALID")
    assert "q_idx" in dsa.dsa_last_error()
    assert call(ks=MIS) == _status("MISALIGNED")
    assert call(sc=MIS) == _status("MISALIGNED")
    # empty inputs are a no-op that touches nothing
    assert call(B=0, q=None, w=None, ks=None, kv=None, sc=None) == 0
    assert call(S=0, q=None) == 0
    assert call(mx=0, q=None) == 0


def test_topk_validation(dsa):
    L = dsa.LIB
    LC = 1 << 20
    need = L.dsa_topk_workspace_bytes(1, 8, LC, 2048)
    assert need > 0                                             # few very long rows: multi plan
    assert L.dsa_topk_workspace_bytes(1, 8, 32768, 2048) == 0     # one workgroup per row
    assert L.dsa_topk_workspace_bytes(1, 2048, 131072, 2048) == 0
    assert L.dsa_topk_workspace_bytes(1, 8, LC, 2048) == need     # deterministic

    def call(k=2048, Lc=LC, mx=LC, ws=A16, wsb=None, sc=A16, B=1, S=8, idx=A16):
        return L.dsa_topk(sc, A16, B, S, Lc, mx, k, idx, ws, need if wsb is None else wsb, None)
    assert call(k=0) == _status("INVALID")
    assert call(k=-5) == _status("INVALID")
    assert call(mx=LC + 1) == _status("INVALID")
    assert call(Lc=(1 << 24) + 1, mx=0) == _status("UNSUPPORTED")
    assert call(wsb=need - 1) == _status("WS")
    assert "needed" in dsa.dsa_last_error()
    assert call(ws=None) == _status("INVALID")
    assert call(ws=MIS) == _status("MISALIGNED")
    assert call(sc=None) == _status("INVALID")
    assert call(idx=MIS) == _status("MISALIGNED")
    assert call(B=0, sc=None, idx=None, ws=None) == 0


def _attn(dsa, **kw):
    a = dsa.dsa.AttentionArgs()
    base = dict(q=A16, q_dtype=2, k_cache=A16, v_cache=A16, kv_dtype=1, k_scale=None,
                v_scale=None, indices=A16, k=2048, kv_len=A16, B=1, S=8, H_q=24, H_kv=2,
                D=128, L_cap=32768, max_kv_len=32768, softmax_scale=0.0, out=A16, out_dtype=2)
    base.update(kw)
    for f, v in base.items():
        setattr(a, f, v)
    return a


def test_attention_validation(dsa):
    L = dsa.LIB
    call = lambda a, ws=A16, wsb=1 << 30: L.dsa_attention_decode(ctypes.byref(a), ws, wsb, None)
    bad = [
        (dict(H_q=25), "INVALID"), (dict(H_kv=0), "INVALID"),
        (dict(H_q=34, H_kv=2), "UNSUPPORTED"),           # ratio 17
        (dict(D=96), "UNSUPPORTED"),
        (dict(q_dtype=0), "UNSUPPORTED"),                 # F32 query with F16 cache
        (dict(kv_dtype=0), "UNSUPPORTED"),
        (dict(out_dtype=3), "UNSUPPORTED"),
        (dict(kv_dtype=3), "INVALID"),                    # INT8 without scales
        (dict(k_scale=A16, v_scale=A16), "INVALID"),      # scales with a float cache
        (dict(k=-1), "INVALID"), (dict(max_kv_len=40000), "INVALID"),
        (dict(softmax_scale=float("nan")), "INVALID"),
        (dict(q=MIS), "MISALIGNED"), (dict(out=None), "INVALID"),
        (dict(kv_dtype=3, k_scale=A16, v_scale=MIS), "MISALIGNED"),
    ]
    aux = dict(aux_k=A16, aux_v=A16, aux_dtype=2, aux_len=8)
    bad += [
        (dict(aux_len=-1), "INVALID"),
        (dict(aux, aux_dtype=3), "UNSUPPORTED"),             # INT8 auxiliary values
        (dict(aux, q_dtype=0, kv_dtype=0, out_dtype=0), "UNSUPPORTED"),   # F32 q needs F32 aux
        (dict(aux, aux_k=MIS), "MISALIGNED"), (dict(aux, aux_v=None), "INVALID"),
        (dict(aux, aux_len=40000), "INVALID"),               # beyond L_cap
    ]
    for kw, want in bad:
        assert call(_attn(dsa, **kw)) == _status(want), (kw, dsa.dsa_last_error())
    ax = _attn(dsa, **aux)
    assert L.dsa_attention_workspace_bytes(ctypes.byref(ax), 0) > 0   # prefill + aux: partials
    assert (L.dsa_attention_workspace_bytes(ctypes.byref(ax), 1)
            > L.dsa_attention_workspace_bytes(ctypes.byref(_attn(dsa)), 1))
    a = _attn(dsa)
    need = L.dsa_attention_workspace_bytes(ctypes.byref(a), 1)
    assert need > 0
    assert L.dsa_attention_workspace_bytes(ctypes.byref(a), 0) == 0   # prefill: no workspace
    assert call(a, wsb=need - 1) == _status("WS")
    assert call(a, ws=None, wsb=need) == _status("INVALID")
    assert call(_attn(dsa, B=0, q=None, out=None)) == 0


def test_noalloc_attention_rejects_before_any_launch(dsa):
    # The allocation-free decode validates like dsa_attention_decode and
    # refuses partials beyond its built-in 16 MiB scratch, all on the host.
    L = dsa.LIB
    call = lambda a: L.dsa_attention_decode_noalloc(ctypes.byref(a), None)
    assert call(_attn(dsa, D=96)) == _status("UNSUPPORTED")
    assert call(_attn(dsa, q=MIS)) == _status("MISALIGNED")
    big = _attn(dsa, B=6, S=8, H_q=16, H_kv=1, kv_dtype=3, k_scale=A16, v_scale=A16, k=65536,
                L_cap=65536, max_kv_len=65536)          # 48 rows x 16 heads x 64 splits
    assert L.dsa_attention_workspace_bytes(ctypes.byref(big), 1) > 16 << 20
    assert call(big) == _status("WS")
    assert "scratch" in dsa.dsa_last_error()
    assert call(_attn(dsa, B=0, q=None, out=None)) == 0


def _append(dsa, **kw):
    a = dsa.dsa.CacheAppendArgs()
    base = dict(k_new=A16, v_new=A16, new_dtype=2, k_cache=A16, v_cache=A16, kv_dtype=3,
                k_scale=A16, v_scale=A16, key_state_new=A16, key_state=A16, idx_dtype=2,
                kv_len=A16, B=8, S=1, H_kv=8, D=128, D_idx=64, L_cap=65536)
    base.update(kw)
    for f, v in base.items():
        setattr(a, f, v)
    return a


def test_cache_append_validation(dsa):
    L = dsa.LIB
    call = lambda a: L.dsa_cache_append(ctypes.byref(a), None)
    bad = [
        (dict(D=96), "UNSUPPORTED"), (dict(H_kv=0), "INVALID"), (dict(L_cap=0), "INVALID"),
        (dict(B=-1), "INVALID"),
        (dict(new_dtype=3), "UNSUPPORTED"),                # INT8 new values
        (dict(kv_dtype=0), "UNSUPPORTED"),                 # F32 cache from BF16 values
        (dict(kv_dtype=5), "UNSUPPORTED"),
        (dict(kv_dtype=1), "INVALID"),                     # scales with a float cache
        (dict(k_scale=None), "INVALID"),                   # INT8 cache without scales
        (dict(v_scale=MIS), "MISALIGNED"),
        (dict(D_idx=48), "UNSUPPORTED"), (dict(idx_dtype=0), "UNSUPPORTED"),
        (dict(key_state=None), "INVALID"),                 # key-state source without target
        (dict(k_new=MIS), "MISALIGNED"), (dict(kv_len=None), "INVALID"),
    ]
    for kw, want in bad:
        assert call(_append(dsa, **kw)) == _status(want), (kw, dsa.dsa_last_error())
    assert call(_append(dsa, S=0, k_new=None, v_new=None)) == 0   # nothing to append


def _rope(dsa, **kw):
    a = dsa.dsa.RopeArgs()
    base = dict(x=A16, x_dtype=2, gamma=A16, cos_cache=A16, sin_cache=A16, kv_len=A16,
                B=1, S=8, H=24, D=128, max_pos=32768, eps=1e-6, interleaved=0, out=A16, out_dtype=1)
    base.update(kw)
    for f, v in base.items():
        setattr(a, f, v)
    return a


def test_rmsnorm_rope_validation(dsa):
    L = dsa.LIB
    call = lambda a: L.dsa_rmsnorm_rope(ctypes.byref(a), None)
    bad = [
        (dict(D=96), "UNSUPPORTED"), (dict(D=16), "UNSUPPORTED"),
        (dict(max_pos=0), "INVALID"), (dict(eps=-1.0), "INVALID"),
        (dict(eps=float("inf")), "INVALID"), (dict(x_dtype=3), "UNSUPPORTED"),
        (dict(out_dtype=3), "UNSUPPORTED"), (dict(H=-1), "INVALID"),
        (dict(gamma=None), "INVALID"), (dict(cos_cache=MIS), "MISALIGNED"),
        (dict(out=None), "INVALID"), (dict(kv_len=MIS), "MISALIGNED"),
    ]
    for kw, want in bad:
        assert call(_rope(dsa, **kw)) == _status(want), (kw, dsa.dsa_last_error())
    assert call(_rope(dsa, H=0, x=None, out=None)) == 0


def test_rmsnorm_rope_multi_validation(dsa):
    """Every job is validated (and named in the message) before any launch; the
    count must lie in [1, 4]."""
    L = dsa.LIB
    def call(*jobs, count=None):
        arr = (dsa.dsa.RopeArgs * max(1, len(jobs)))(*jobs)
        return L.dsa_rmsnorm_rope_multi(arr, len(jobs) if count is None else count, None)
    good = _rope(dsa, H=0, x=None, out=None)
    assert call(good) == 0
    assert call(good, good, good, good) == 0
    assert call(good, count=0) == _status("INVALID")
    assert call(good, good, good, good, good) == _status("INVALID")
    assert L.dsa_rmsnorm_rope_multi(None, 1, None) == _status("INVALID")
    assert call(good, _rope(dsa, D=96)) == _status("UNSUPPORTED")
    assert "job 1" in dsa.dsa_last_error()
    assert call(good, good, _rope(dsa, out=None)) == _status("INVALID")
    assert "out" in dsa.dsa_last_error()


def test_error_text_is_thread_local_and_cleared(dsa):
    import threading
    L = dsa.LIB
    L.dsa_topk(None, None, 1, 1, 16, 16, 0, None, None, 0, None)
    msg = dsa.dsa_last_error()
    assert "k=0" in msg
    seen = []
    t = threading.Thread(target=lambda: seen.append(dsa.dsa_last_error()))
    t.start()
    t.join()
    assert seen == [""]
    assert L.dsa_topk(None, None, 0, 1, 16, 16, 4, None, None, 0, None) == 0
    assert dsa.dsa_last_error() == ""


def test_roofline_probe_library_exports_its_header():
    import ctypes as C
    header = os.path.join(ROOT, "include", "dsa_roofline.h")
    lib = C.CDLL(os.path.join(ROOT, "sparse_gqa_attention_amd", "libdsa_roofline.so"))
    names = declared_functions(header)
    assert len(names) == 8
    for n in names:
        assert hasattr(lib, n), f"{n} declared in dsa_roofline.h but not exported"
    from sparse_gqa_attention_amd import roofline
    assert sorted(roofline.EXPORTS) == names
    assert lib.dsa_roofline_read(None, 0, None, None) == 2          # rejected, nothing launched
    lib.dsa_roofline_mfma_flops.restype = C.c_double
    assert lib.dsa_roofline_mfma_flops(2, 3) == 2 * 4 * 3 * 4 * 32 * 32 * 16 * 2


def test_describe_plan_names_the_launches(dsa):
    d, F = dsa.dsa_describe_plan, dsa.plan_fields
    # 32K speculative decode: decode indexer, one LDS-resident top-k workgroup
    # per row, 16 key splits per (row, KV head) and a split merge
    f = F(d(dsa.DSA_PLAN_INDEXER, 1, 8, 32768, D_idx=64))
    assert f["kernel"] == "indexer_score_kernel" and f["grid"] == "1x512x1"
    f = F(d(dsa.DSA_PLAN_TOPK, 1, 8, 32768, k=2048))
    assert f["plan"] == "resident" and f["grid"] == "8" and f["workspace"] == "0"
    a = _attn(dsa, q=None, k_cache=None, v_cache=None, indices=None, kv_len=None, out=None)
    f = F(d(dsa.DSA_PLAN_ATTENTION_DECODE, attention=a))
    assert f["grid"] == "16x2x8" and f["merge_grid"] == "192"
    assert int(f["workspace"]) == L_attn_ws(dsa, a)
    f = F(d(dsa.DSA_PLAN_ATTENTION_PREFILL, attention=a))
    assert f["schedule"] == "split" and f["grid"] == "1x2x8" and "merge_grid" not in f
    assert f["workspace"] == "0"
    # rows of at most 4096 keys (by the runtime bound): one small workgroup per row
    f = F(d(dsa.DSA_PLAN_TOPK, 1, 1, 1024, k=128))
    assert f["plan"] == "small" and f["grid"] == "1" and f["keys_per_thread"] == "4"
    f = F(d(dsa.DSA_PLAN_TOPK, 3, 50, 262144, max_kv_len=4096, k=300))
    assert f["plan"] == "small" and f["grid"] == "150" and f["keys_per_thread"] == "16"
    assert dsa.dsa_topk_workspace_bytes(1, 8, 4096, 2048) == 0
    assert F(d(dsa.DSA_PLAN_TOPK, 1, 8, 4097, k=2048))["plan"] == "resident"
    # the runtime bound, not the capacity, picks the plan
    f = F(d(dsa.DSA_PLAN_TOPK, 1, 8, 262144, max_kv_len=32768, k=2048))
    assert f["plan"] == "resident" and f["workspace"] == "0"
    # 256K decode: the two-kernel split top-k on its fast path
    f = F(d(dsa.DSA_PLAN_TOPK, 1, 8, 262144, k=2048))
    assert f["plan"] == "split" and f["chunk_grid"] == "32x8" and f["mode"] == "fast"
    assert int(f["workspace"]) == dsa.dsa_topk_workspace_bytes(1, 8, 262144, 2048)
    # the runtime bound sizes the chunk grid
    f = F(d(dsa.DSA_PLAN_TOPK, 4, 8, 262144, max_kv_len=200000, k=2048))
    assert f["chunk_grid"] == "25x32"
    f = F(d(dsa.DSA_PLAN_TOPK, 1, 4, 262144, k=9000))
    assert f["mode"] == "exact" and f["chunk_grid"] == "0x4"
    # 128K prefill: head-folded indexer, one top-k workgroup per row
    f = F(d(dsa.DSA_PLAN_INDEXER, 1, 2048, 131072, D_idx=64))
    assert f["kernel"] == "indexer_fold_kernel" and f["grid"] == "64x32x1"
    assert f["keys_per_workgroup"] == "4096"
    f = F(d(dsa.DSA_PLAN_TOPK, 1, 2048, 131072, k=2048))
    assert f["plan"] == "stream" and f["grid"] == "2048"
    # ... and whole-row attention waves (4 rows per workgroup, KV head j % 2)
    a = _attn(dsa, q=None, k_cache=None, v_cache=None, indices=None, kv_len=None, out=None,
              S=2048, L_cap=131072, max_kv_len=131072, kv_dtype=2)
    f = F(d(dsa.DSA_PLAN_ATTENTION_PREFILL, attention=a))
    assert f["schedule"] == "wave_rows" and f["grid"] == "1024" and f["workspace"] == "0"
    # 1024 (row, KV head) pairs stay on four waves per row
    a = _attn(dsa, q=None, k_cache=None, v_cache=None, indices=None, kv_len=None, out=None,
              S=512, L_cap=131072, max_kv_len=131072, kv_dtype=2)
    assert F(d(dsa.DSA_PLAN_ATTENTION_PREFILL, attention=a))["schedule"] == "split"
    # invalid queries: 0, with the reason
    with pytest.raises(dsa.DsaError):
        d(7, 1, 1, 16)
    with pytest.raises(dsa.DsaError):
        d(dsa.DSA_PLAN_TOPK, 1, 8, 32768, k=0)
    assert "k=0" in dsa.dsa_last_error()


def L_attn_ws(dsa, a):
    return dsa.LIB.dsa_attention_workspace_bytes(ctypes.byref(a), 1)
