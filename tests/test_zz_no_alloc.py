"""dsa_attention_decode_noalloc (built-in scratch, no workspace) against
dsa_attention_decode (caller workspace), through the C ABI.

Two calls in a row on one GPU, the second with a smaller problem (fewer rows,
heads and key splits) than the first, so the second call runs over a scratch
that still holds the first call's partials wherever it does not overwrite
them.  Both calls run the same kernels with the same split plan, so the
outputs must equal the workspace entry point's bit for bit; each is also held
to the oracle gate.
"""
import numpy as np
import pytest
import torch

import oracle
from dsa_synth import SPEC_DECODE_32K, make_inputs, scaled, torch_dtype
from gpu_util import DEV, dsa, say, upload  # noqa: F401
from parity import assert_output_close
from test_gpu_attention import random_selection

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 16 << 20

# (q, kv, out, D, H_q, H_kv, B, S, L, k, kv_len, seed)
CASES = [
    ("bf16", "i8", "bf16", 128, 48, 8, 8, 1, 65536, 8192, [65536] * 8, 41),   # ~8.6 MB of partials
    ("bf16", "f16", "bf16", 64, 8, 2, 2, 3, 3000, 256, [3000, 1200], 42),     # far smaller
]


def _inputs(case):
    qd, kd, od, D, H_q, H_kv, B, S, L, k, kv_len, seed = case
    w = scaled(SPEC_DECODE_32K, B=B, S=S, L=L, H_q=H_q, H_kv=H_kv, D=D, q_dtype=qd,
               kv_dtype=kd, out_dtype=od, k=k, H_idx=None, D_idx=None, seed=seed)
    x = make_inputs(w, kv_len=kv_len)
    idx = random_selection(np.random.default_rng(seed), x["kv_len"].tolist(), S, k, L)
    return x, idx, torch_dtype(od)


def test_noalloc_decode_matches_workspace_decode_twice(dsa):
    for case in CASES:
        x, idx, od = _inputs(case)
        g = upload(x)
        gi = idx.to(DEV)
        a = dsa.attention_args(g["q"], g["k_cache"], g["v_cache"], gi, g["kv_len"],
                               torch.empty(g["q"].shape, dtype=od, device=DEV),
                               g["k_scale"], g["v_scale"])
        need = dsa.dsa_attention_workspace_bytes(a, True)
        say(f"noalloc case {case[:10]}: partials {need} bytes")
        assert 0 < need <= SCRATCH_BYTES
        ref = torch.full(g["q"].shape, float("nan"), dtype=od, device=DEV)
        dsa.dsa_attention_decode(g["q"], g["k_cache"], g["v_cache"], gi, g["kv_len"], ref,
                                 k_scale=g["k_scale"], v_scale=g["v_scale"])
        out = torch.full(g["q"].shape, float("nan"), dtype=od, device=DEV)
        dsa.dsa_attention_decode_noalloc(g["q"], g["k_cache"], g["v_cache"], gi, g["kv_len"], out,
                                         k_scale=g["k_scale"], v_scale=g["v_scale"])
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), \
            f"{case[:10]}: allocation-free output differs from the workspace entry point's"
        want = oracle.sparse_attention(x["q"], x["k_cache"], x["v_cache"], idx,
                                       x["kv_len"].tolist(), k_scale=x["k_scale"],
                                       v_scale=x["v_scale"])
        rel, mx = assert_output_close(out, want, case[2], what=f"noalloc {case[:10]}")
        say(f"noalloc case {case[:10]}: bit-equal to the workspace call, rel={rel:.2e} max={mx:.2e}")


def test_noalloc_decode_rejects_partials_beyond_scratch(dsa):
    # 48 rows x 16 heads x 64 splits x (128 + 2) floats: about 25 MB of
    # partials, more than the scratch holds -- rejected on the host, nothing
    # launched, the output left untouched.
    case = ("bf16", "i8", "bf16", 128, 16, 1, 6, 8, 65536, 65536, [65536] * 6, 43)
    qd, kd, od_name, D, H_q, H_kv, B, S, L, k, kv_len, seed = case
    q = torch.zeros((B, S, H_q, D), dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros((B, L, H_kv, D), dtype=torch.int8, device=DEV)
    sc = torch.ones((B, L, H_kv), dtype=torch.float32, device=DEV)
    idx = torch.arange(k, dtype=torch.int32, device=DEV).expand(B, S, k).contiguous()
    kvl = torch.tensor(kv_len, dtype=torch.int32, device=DEV)
    out = torch.full((B, S, H_q, D), 7.0, dtype=torch.bfloat16, device=DEV)
    a = dsa.attention_args(q, kc, kc, idx, kvl, out, sc, sc)
    assert dsa.dsa_attention_workspace_bytes(a, True) > SCRATCH_BYTES
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_attention_decode_noalloc(q, kc, kc, idx, kvl, out, k_scale=sc, v_scale=sc)
    assert e.value.status == 4 and "scratch" in str(e.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
