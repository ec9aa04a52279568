"""GPU parity of dsa_rmsnorm_rope against the FP64 oracle.

The kernel computes in FP32 and rounds once; the oracle's exact result is
rounded once to the output dtype.  FP32 and FP64 intermediates can land on
opposite sides of a rounding boundary, so a 16-bit output may differ from
the rounded oracle by one ulp (plus a few FP32 ulps of the row's scale where
the rotation cancels), on a small fraction of elements; FP32 outputs must
agree to a few FP32 ulps of the row scale.  At the workload shapes the
FP16 output's relative RMSE against the exact result is also checked
against the pages' 0.0207%.
"""
import numpy as np
import pytest
import torch

import oracle.rope_oracle as ro
from dsa_synth import make_rope_inputs
from gpu_util import DEV, dsa, say  # noqa: F401

pytestmark = pytest.mark.gpu

_T = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def _ulp(v, dtype):
    t = torch.from_numpy(np.abs(v)).to(_T[dtype])
    nxt = torch.nextafter(t, torch.full_like(t, float("inf")))
    return (nxt.double() - t.double()).numpy()


def _check(dsa, B, S, H, D, max_pos, kv_len, x_dtype, out_dtype, interleaved, seed,
           in_place=False, max_flip_frac=0.01):
    say(f"rope B={B} S={S} H={H} D={D} max_pos={max_pos} kv_len={kv_len} x={x_dtype} "
        f"out={out_dtype} interleaved={interleaved} in_place={in_place}")
    x = make_rope_inputs(B, S, H, D, max_pos, x_dtype, kv_len, seed=seed)
    g = {k: v.to(DEV) for k, v in x.items()}
    if in_place:
        assert x_dtype == out_dtype
        out = g["x"]
    else:
        out = torch.full((B, S, H, D), float("nan"), dtype=_T[out_dtype], device=DEV)
    dsa.dsa_rmsnorm_rope(g["x"], g["gamma"], g["cos"], g["sin"], g["kv_len"], out, eps=1e-6,
                         interleaved=interleaved)
    torch.cuda.synchronize()
    return _compare(x, kv_len, out.cpu().double().numpy(), out_dtype, interleaved, in_place,
                    max_flip_frac)


def _compare(x, kv_len, got, out_dtype, interleaved, in_place=False, max_flip_frac=0.01):
    exact = ro.rmsnorm_rope(x["x"], x["gamma"], x["cos"], x["sin"], kv_len, 1e-6, interleaved)
    skipped = np.isnan(exact[:, :, 0, 0])
    for b, s in zip(*np.nonzero(skipped)):        # rows outside the tables stay untouched
        before = x["x"][b, s].double().numpy() if in_place else None
        if in_place:
            assert np.array_equal(got[b, s], before)
        else:
            assert np.all(np.isnan(got[b, s]))
    live = ~skipped
    e, gv = exact[live], got[live]
    if out_dtype == "f32":
        scale = np.max(np.abs(e), axis=-1, keepdims=True)
        assert np.all(np.abs(gv - e) <= 2e-6 * scale), np.max(np.abs(gv - e) / scale)
        return gv, e
    want = torch.from_numpy(e).to(_T[out_dtype]).double().numpy()
    diff = np.abs(gv - want)
    # one ulp of the rounded value, plus the FP32 arithmetic error, which is
    # relative to the row's scale (the rotation can cancel to a tiny result)
    scale = np.max(np.abs(e), axis=-1, keepdims=True)
    bound = _ulp(want, out_dtype) * 1.0000001 + 2.0 ** -20 * scale
    assert np.all(diff <= bound), f"off by {np.max(diff / bound):.2f} x the bound"
    frac = float(np.mean(diff > 0))
    assert frac <= max_flip_frac, f"{frac:.4f} of the elements differ from the rounded oracle"
    return gv, e


COMBOS = [("bf16", "f16"), ("f16", "f16"), ("f32", "f16"), ("bf16", "bf16"), ("f16", "bf16"),
          ("f32", "f32"), ("bf16", "f32")]


@pytest.mark.parametrize("x_dtype,out_dtype", COMBOS, ids=[f"{a}->{b}" for a, b in COMBOS])
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("interleaved", [False, True])
def test_rope_small(dsa, x_dtype, out_dtype, D, interleaved):
    # second sequence runs 2 positions past the tables: its last 2 rows stay untouched
    _check(dsa, B=3, S=5, H=7, D=D, max_pos=64, kv_len=[64, 66, 5], x_dtype=x_dtype,
           out_dtype=out_dtype, interleaved=interleaved, seed=D + int(interleaved))


def test_rope_in_place(dsa):
    _check(dsa, B=2, S=4, H=3, D=128, max_pos=32, kv_len=[32, 4], x_dtype="f16",
           out_dtype="f16", interleaved=False, seed=3, in_place=True)


@pytest.mark.parametrize("H,S,L", [(24, 8, 32768), (2, 8, 32768), (16, 8, 262144), (24, 2048, 131072)],
                         ids=["q_heads_32k", "k_heads_32k", "indexer_q_256k", "q_heads_prefill_128k"])
def test_rope_workload_shapes_and_pages_rmse(dsa, H, S, L):
    gv, e = _check(dsa, B=1, S=S, H=H, D=128 if H != 16 else 64, max_pos=L, kv_len=[L],
                   x_dtype="bf16", out_dtype="f16", interleaved=False, seed=H + S)
    rel = float(np.sqrt(np.sum((gv - e) ** 2) / np.sum(e ** 2)))
    say(f"rope H={H} S={S}: FP16 output relative RMSE vs exact {rel:.3e} (pages: 2.07e-4)")
    assert rel <= 1.1 * 2.07e-4


def test_rope_multi_one_launch(dsa):
    """dsa_rmsnorm_rope_multi: the query, key and indexer-query heads of a decode
    step (different H, D and dtypes; one interleaved; one job with no rows) in
    one launch, each against the oracle and bit-equal to its own single call."""
    specs = [  # B, S, H, D, max_pos, kv_len, x_dtype, out_dtype, interleaved
        (2, 8, 24, 128, 300, [300, 40], "bf16", "bf16", False),
        (2, 8, 2, 128, 300, [300, 40], "bf16", "f16", False),
        (2, 8, 0, 64, 300, [300, 40], "bf16", "bf16", False),
        (2, 8, 16, 64, 300, [302, 40], "f32", "f16", True),
    ]
    jobs, singles, inputs = [], [], []
    for i, (B, S, H, D, mp, kvl, xd, od, il) in enumerate(specs):
        say(f"rope multi job {i}: B={B} S={S} H={H} D={D} x={xd} out={od} interleaved={il}")
        x = make_rope_inputs(B, S, H, D, mp, xd, kvl, seed=40 + i)
        g = {k: v.to(DEV) for k, v in x.items()}
        out = torch.full((B, S, H, D), float("nan"), dtype=_T[od], device=DEV)
        ref = torch.full((B, S, H, D), float("nan"), dtype=_T[od], device=DEV)
        jobs.append(dict(x=g["x"], gamma=g["gamma"], cos_cache=g["cos"], sin_cache=g["sin"],
                         kv_len=g["kv_len"], out=out, eps=1e-6, interleaved=il))
        dsa.dsa_rmsnorm_rope(g["x"], g["gamma"], g["cos"], g["sin"], g["kv_len"], ref, eps=1e-6,
                             interleaved=il)
        singles.append(ref)
        inputs.append(x)
    dsa.dsa_rmsnorm_rope_multi(jobs)
    torch.cuda.synchronize()
    for i, (j, ref, x, sp) in enumerate(zip(jobs, singles, inputs, specs)):
        assert torch.equal(j["out"].isnan(), ref.isnan()), i
        assert torch.equal(torch.nan_to_num(j["out"]), torch.nan_to_num(ref)), i
        if sp[2]:
            _compare(x, sp[5], j["out"].cpu().double().numpy(), sp[7], sp[8])
