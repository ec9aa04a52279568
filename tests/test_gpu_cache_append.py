"""GPU parity of dsa_cache_append against the CPU oracle (bit-exact).

Every case pre-fills the caches, appends through the C ABI, and compares the
whole caches with oracle.cache_oracle.cache_append: appended rows must equal
the oracle's rounding / INT8 quantisation bit for bit, every other position
must be untouched.
"""
import numpy as np
import pytest
import torch

import oracle.cache_oracle as co
from dsa_synth import make_append_inputs
from gpu_util import DEV, dsa, say, first_mismatch  # noqa: F401

pytestmark = pytest.mark.gpu


def _np(t):
    if t is None:
        return None
    t = t.cpu()
    return t.numpy() if t.dtype in (torch.int8, torch.int32, torch.float32) else t.double().numpy()


def _run_case(dsa, B, S, H_kv, D, L_cap, new_dtype, kv_dtype, kv_len, seed, D_idx=64,
              with_key_state=True, scale=1.0, edit=None):
    say(f"append B={B} S={S} H_kv={H_kv} D={D} L_cap={L_cap} new={new_dtype} cache={kv_dtype} "
        f"kv_len={kv_len} seed={seed}")
    x = make_append_inputs(B, S, H_kv, D, L_cap, new_dtype, kv_dtype, kv_len, D_idx=D_idx,
                           seed=seed, scale=scale)
    if edit is not None:
        edit(x)
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in x.items()}
    if L_cap * B > 4096:
        return _run_large(dsa, x, g, S, kv_len, L_cap, kv_dtype, with_key_state)
    dsa.dsa_cache_append(g["k_new"], g["v_new"], g["k_cache"], g["v_cache"], g["kv_len"],
                         k_scale=g["k_scale"], v_scale=g["v_scale"],
                         key_state_new=g["key_state_new"] if with_key_state else None,
                         key_state=g["key_state"] if with_key_state else None)
    torch.cuda.synchronize()
    kn = x["k_new"].float().numpy()
    vn = x["v_new"].float().numpy()
    ref = co.cache_append(_np(x["k_cache"]), _np(x["v_cache"]), kn, vn, kv_len, kv_dtype,
                          _np(x["k_scale"]), _np(x["v_scale"]),
                          _np(x["key_state"]), _np(x["key_state_new"]))
    names = ["k_cache", "v_cache", "k_scale", "v_scale", "key_state"]
    for name, want in zip(names, ref):
        if want is None:
            continue
        got = _np(g[name])
        if name == "key_state" and not with_key_state:
            want = _np(x["key_state"])
        if want.dtype == np.float32 and got.dtype == np.float32:
            ok = np.array_equal(got.view(np.uint32), want.view(np.uint32))
        else:
            ok = np.array_equal(got, want)
        assert ok, f"{name}: {first_mismatch(got, want)}"


def _run_large(dsa, x, g, S, kv_len, L_cap, kv_dtype, with_key_state):
    """Full-size shapes: appended rows against the oracle, the rest unchanged
    (checked on the GPU against a copy taken before the call)."""
    before = {n: g[n].clone() for n in ("k_cache", "v_cache", "k_scale", "v_scale", "key_state")
              if g[n] is not None}
    dsa.dsa_cache_append(g["k_new"], g["v_new"], g["k_cache"], g["v_cache"], g["kv_len"],
                         k_scale=g["k_scale"], v_scale=g["v_scale"],
                         key_state_new=g["key_state_new"] if with_key_state else None,
                         key_state=g["key_state"] if with_key_state else None)
    torch.cuda.synchronize()
    pos = co.append_positions(kv_len, S, L_cap)
    written = torch.zeros(g["k_cache"].shape[:2], dtype=torch.bool, device=DEV)
    for b, _, p in pos:
        written[b, p] = True
    for n, t0 in before.items():
        changed = (g[n] != t0).reshape(t0.shape[0], t0.shape[1], -1).any(-1)
        assert not (changed & ~written).any().item(), f"{n}: a position outside the append changed"
    kn, vn = x["k_new"].float().numpy(), x["v_new"].float().numpy()
    bi = np.array([b for b, _, _ in pos]); si = np.array([t for _, t, _ in pos])
    pi = np.array([p for _, _, p in pos])
    bt, pt = torch.from_numpy(bi).to(DEV), torch.from_numpy(pi).to(DEV)
    for src, cache, sc in ((kn, "k_cache", "k_scale"), (vn, "v_cache", "v_scale")):
        rows = src[bi, si]                                   # [N, H_kv, D]
        got = g[cache][bt, pt].cpu()
        if kv_dtype == "i8":
            codes, scales = co.quantize_rows_int8(rows)
            assert np.array_equal(got.numpy(), codes), cache
            assert np.array_equal(g[sc][bt, pt].cpu().numpy().view(np.uint32),
                                  scales.view(np.uint32)), sc
        else:
            want = co.round_to_dtype(rows, kv_dtype)
            assert np.array_equal(got.double().numpy(), want), cache
    if with_key_state:
        assert torch.equal(g["key_state"][bt, pt].cpu(), x["key_state_new"][bi, si])


COMBOS = [("bf16", "f16"), ("f16", "f16"), ("f32", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
          ("f32", "f32"), ("bf16", "i8"), ("f16", "i8"), ("f32", "i8")]


@pytest.mark.parametrize("new_dtype,kv_dtype", COMBOS, ids=[f"{a}->{b}" for a, b in COMBOS])
@pytest.mark.parametrize("D", [64, 128])
def test_append_small_ragged(dsa, new_dtype, kv_dtype, D):
    # ragged post-append lengths: full cache, kv_len == S, a middle one, and
    # one running past L_cap (its last two tokens are skipped)
    _run_case(dsa, B=4, S=5, H_kv=3, D=D, L_cap=40, new_dtype=new_dtype, kv_dtype=kv_dtype,
              kv_len=[40, 5, 17, 42], seed=D + len(new_dtype) * 7 + len(kv_dtype))


def test_append_without_key_state(dsa):
    _run_case(dsa, B=2, S=3, H_kv=2, D=128, L_cap=16, new_dtype="bf16", kv_dtype="i8",
              kv_len=[16, 9], seed=3, with_key_state=False)


@pytest.mark.parametrize("D_idx", [32, 128])
def test_append_key_state_widths(dsa, D_idx):
    _run_case(dsa, B=2, S=4, H_kv=1, D=64, L_cap=24, new_dtype="f16", kv_dtype="f16",
              kv_len=[24, 4], seed=5, D_idx=D_idx)


def _int8_edges(x):
    kn = x["k_new"]
    kn[0, 0, 0].zero_()                                   # all-zero row -> scale 0
    kn[0, 0, 1].zero_()
    kn[0, 0, 1, 7] = 3.0e4                                # one dominant value
    # amax 127 gives scale 1: x.5 values must round to even
    row = torch.tensor([127.0] + [k + 0.5 for k in range(-60, 60, 2)][:kn.shape[-1] - 1])
    kn[0, 1, 0, :row.numel()] = row.to(kn.dtype)
    x["k_new"] = kn


def test_append_int8_edge_rows(dsa):
    _run_case(dsa, B=1, S=2, H_kv=2, D=128, L_cap=8, new_dtype="f32", kv_dtype="i8",
              kv_len=[8], seed=9, edit=_int8_edges)


@pytest.mark.parametrize("scale", [1e-30, 1e30])
def test_append_int8_extreme_magnitudes(dsa, scale):
    _run_case(dsa, B=1, S=3, H_kv=2, D=64, L_cap=8, new_dtype="f32", kv_dtype="i8",
              kv_len=[8], seed=10, scale=scale)


def test_append_int8_batched_decode_64k_shape(dsa):
    # the 64K INT8 batched decode step: 8 sequences append one token each
    _run_case(dsa, B=8, S=1, H_kv=8, D=128, L_cap=65536, new_dtype="bf16", kv_dtype="i8",
              kv_len=[65536, 1000, 65535, 1, 40000, 2, 65536, 777], seed=11, with_key_state=False)


def test_append_prefill_chunk_shape(dsa):
    # a 2048-token prefill chunk appended after 129024 cached tokens (BF16 cache)
    _run_case(dsa, B=1, S=2048, H_kv=2, D=128, L_cap=131072, new_dtype="bf16", kv_dtype="bf16",
              kv_len=[131072], seed=12)
