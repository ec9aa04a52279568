"""The hot path replayed from a captured HIP graph, as the bench times it.

One decode step (indexer -> top-k -> split-K attention with its merge) is
captured once.  Between replays the host runs eager work: it overwrites the
inputs with another seed's values and fills every output with garbage.  Each
replay must reproduce, bit for bit, what eager launches compute from the same
inputs: the kernels are deterministic and the library keeps no state between
calls.  The 256K shape covers the top-k plan with a workspace (three kernels)
and the streaming decode indexer.
"""
import pytest
import torch

from dsa_synth import DECODE_256K, SPEC_DECODE_32K, make_inputs
from gpu_util import DEV, dsa, say  # noqa: F401

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("wl", [SPEC_DECODE_32K, DECODE_256K], ids=lambda w: w.name)
def test_decode_step_graph_replays_match_eager(dsa, wl):
    say(f"graph replays {wl.name}")
    B, S, L = wl.B, wl.S, wl.L
    inputs = [make_inputs(wl), make_inputs(wl, seed=wl.seed + 100)]
    g = {k: (v.to(DEV) if isinstance(v, torch.Tensor) else v) for k, v in inputs[0].items()}
    scores = torch.empty((B, S, L), dtype=torch.float32, device=DEV)
    idx = torch.empty((B, S, wl.k), dtype=torch.int32, device=DEV)
    out = torch.empty((B, S, wl.H_q, wl.D), dtype=torch.bfloat16, device=DEV)
    topk_ws = torch.empty(max(dsa.dsa_topk_workspace_bytes(B, S, L, wl.k), 16), dtype=torch.uint8,
                          device=DEV)
    a = dsa.attention_args(g["q"], g["k_cache"], g["v_cache"], idx, g["kv_len"], out)
    attn_ws = torch.empty(max(dsa.dsa_attention_workspace_bytes(a, True), 16), dtype=torch.uint8,
                          device=DEV)
    assert attn_ws.numel() > 16, "the decode attention should split its keys here"

    def step():
        dsa.dsa_indexer_score(g["q_idx"], g["w_idx"], g["key_state"], g["kv_len"], scores)
        dsa.dsa_topk(scores, g["kv_len"], wl.k, idx, workspace=topk_ws)
        dsa.dsa_attention_decode(g["q"], g["k_cache"], g["v_cache"], idx, g["kv_len"], out,
                                 workspace=attn_ws)

    def load(x):
        for name in ("q_idx", "w_idx", "q"):
            g[name].copy_(x[name].to(DEV))

    def garbage():
        scores.fill_(float("nan"))
        idx.fill_(-7)
        out.fill_(float("nan"))
        topk_ws.fill_(0xA5)
        attn_ws.fill_(0x5A)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    for rep, x in enumerate([inputs[0], inputs[1], inputs[0]]):
        load(x)
        garbage()
        step()                                       # eager reference
        torch.cuda.synchronize()
        want = (scores.clone(), idx.clone(), out.clone())
        garbage()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, got, ref in zip(("scores", "indices", "out"), (scores, idx, out), want):
            assert torch.equal(got.view(torch.uint8) if got.dtype != torch.int32 else got,
                               ref.view(torch.uint8) if ref.dtype != torch.int32 else ref), \
                f"{wl.name} replay {rep}: {name} differs from eager"
        assert not torch.isnan(out.float()).any()
    say(f"graph replays {wl.name}: 3 replays bit-identical to eager")
