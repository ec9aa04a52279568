"""Benchmark of the dynamic sparse GQA attention hot path on one MI355X.

One step = the whole hot path (indexer score -> top-k -> sparse attention)
run once per "layer" over N distinct layer buffer sets whose total footprint
exceeds 1 GiB, so that no layer's key-state or KV cache is still resident in
the 256 MB Infinity Cache when it is read again.  The reported value is the
time per layer (microseconds): step time / N.

Inputs are seeded and synthetic and already resident in HBM when the timed
region starts.  By default one step is captured as a HIP graph (through
torch.cuda.CUDAGraph) and replayed, as a decode step is in a serving loop;
--eager times plain launches.  HIP events on the launch stream time K step
replays (after K untimed ones), then K replays of a graph of each stage
alone; the stage with the longest time is the dominant one, and its
algorithmic bytes per call divided by its average duration is the roofline
`achieved` figure.
The CPU baseline times the FP64 oracle on the host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/layer + achieved HBM GB/s for sparse GQA decode at 32K–256K ctx"

# HBM-side bytes per stage call, measured with rocprofv3 --pmc FETCH_SIZE and
# --pmc WRITE_SIZE (each scaled by the counts of a 256 MiB reference copy)
# for kernel sources whose digest is `sources`; the summaries are
# profiles/<workload>_hot_path_kernels.txt.  Reported only while the kernel
# sources still have that digest.
MEASURED_TRAFFIC = {
    "sources": "c5d1d07dedca146b",
    "spec_decode_32k": {"attention": 18138325, "indexer": 5435081, "topk": 1298523},
    "decode_256k": {"attention": 20355511, "indexer": 42208577, "topk": 9777949},
    "prefill_128k": {"attention": 3430403310, "indexer": 1125393242, "topk": 1089186349},
    "int8_batched_decode_64k": {"attention": 1155072974},
}


def sources_digest():
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_gqa_attention_amd", "csrc")
    for f in sorted(sum((glob.glob(os.path.join(csrc, p)) for p in ("*.hip", "*.h", "*.cpp")), [])):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]
HBM_PEAK_GBPS = 8000.0
ELT = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="spec_decode_32k")
    p.add_argument("--layers", type=int, default=0, help="layer buffer sets (0: >= 1 GiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of HIP-graph replays")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    p.add_argument("--pmc-run", action="store_true",
                   help="for counter collection: a 256 MiB reference copy, then each stage "
                        "eagerly on 4 distinct layers; prints the bytes each should move")
    return p.parse_args()


# ------------------------------------------------------------------ algorithmic bytes
def stage_bytes(w, kv_len):
    """Bytes each stage's contract must move for one layer (each byte once)."""
    B, S, k = w.B, w.S, w.k
    rows_valid = []
    for b in range(B):
        for s in range(S):
            pos = kv_len[b] - S + s
            rows_valid.append(max(0, min(k, pos + 1)))
    out = {}
    if w.has_indexer:
        key_state = sum(kv_len) * w.D_idx * ELT[w.idx_dtype]
        q_idx = B * S * w.H_idx * w.D_idx * ELT[w.idx_dtype] + B * S * w.H_idx * 4
        scores_w = B * S * w.L * 4
        out["indexer"] = key_state + q_idx + scores_w
        scores_r = sum(max(0, kv_len[b] - S + s + 1) for b in range(B) for s in range(S)) * 4
        out["topk"] = scores_r + B * S * k * 4
    row_bytes = w.H_kv * w.D * ELT[w.kv_dtype] * 2
    if w.kv_dtype == "i8":
        row_bytes += w.H_kv * 4 * 2
    gathered = sum(rows_valid) * row_bytes
    q = B * S * w.H_q * w.D * ELT[w.q_dtype]
    o = B * S * w.H_q * w.D * ELT[w.out_dtype]
    out["attention"] = gathered + q + o + B * S * k * 4
    # KV-cache append of the step's S new tokens (measured separately, not
    # part of the path below): new K/V and indexer keys read, cache rows written.
    new_elt = ELT[w.kv_dtype] if w.kv_dtype != "i8" else ELT[w.q_dtype]
    app = B * S * w.H_kv * w.D * (new_elt + ELT[w.kv_dtype]) * 2
    if w.kv_dtype == "i8":
        app += B * S * w.H_kv * 4 * 2
    if w.has_indexer:
        app += B * S * w.D_idx * ELT[w.idx_dtype] * 2
    out["cache_append"] = app
    # RMSNorm + rotary of the step's query, key and indexer-query heads
    # (measured separately): head vectors read and written, tables' rows read.
    out_elt = 2                                  # 16-bit output
    rope = B * S * (w.H_q + w.H_kv) * w.D * (ELT[w.q_dtype] + out_elt) + B * S * w.D * 4 * 2
    if w.has_indexer:
        rope += B * S * w.H_idx * w.D_idx * (ELT[w.idx_dtype] + out_elt) + B * S * w.D_idx * 4 * 2
    out["rmsnorm_rope"] = rope
    # Attention whose S newest keys come as auxiliary K/V (BF16, or F32 next
    # to an F32 cache) instead of from the cache.
    aux_elt = 4 if w.kv_dtype == "f32" else 2
    out["attention_aux"] = out["attention"] + B * S * w.H_kv * w.D * aux_elt * 2
    # Whole path without the score round trip (an artefact of the 4-call ABI).
    path = out["attention"]
    if w.has_indexer:
        path += key_state + q_idx
    out["path"] = path
    return out


# ------------------------------------------------------------------ CPU baseline
def cpu_baseline(w, x, seconds):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        cores = len(os.sched_getaffinity(0))
    kv_len = x["kv_len"].tolist()
    rows = [(b, s) for b in range(w.B) for s in range(w.S)]
    if len(rows) > 16:
        rows = rows[:: max(1, len(rows) // 16)][:16]
    t0 = time.perf_counter()
    reps = 0
    while True:
        idx = np.full((w.B, w.S, w.k), -1, dtype=np.int64)
        for b, s in rows:
            pos = kv_len[b] - w.S + s
            if w.has_indexer:
                sc = oracle.indexer_scores_row(x["q_idx"][b, s], x["w_idx"][b, s],
                                               x["key_state"][b], pos)
                idx[b, s] = oracle.topk_row(sc, pos, w.k)
            else:
                idx[b, s] = x["indices"][b, s].numpy()
        oracle.sparse_attention(x["q"], x["k_cache"], x["v_cache"], idx, kv_len,
                                k_scale=x["k_scale"], v_scale=x["v_scale"], rows=rows)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 200:
            break
    per_row = el / (reps * len(rows))
    us_per_layer = per_row * w.B * w.S * 1e6
    return {"value": round(us_per_layer, 1), "unit": "us/layer", "cores": cores, "kind": "oracle",
            "sample": f"{reps} x {len(rows)} of the {w.B * w.S} query rows of one {w.name} layer "
                      f"(FP64 scores, full-sort top-k, dense masked attention), scaled to "
                      f"all {w.B * w.S} rows; {el:.1f} s of host time"}


# ------------------------------------------------------------------ GPU bench
def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs "
              f"the hot path on a single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    import torch
    import sparse_gqa_attention_amd as dsa
    from dsa_synth import BY_NAME, make_inputs, make_new_tokens, make_rope_inputs, make_aux_inputs

    w = BY_NAME[args.workload]
    decode = w.decode_form
    mx = w.max_kv_len          # runtime capacity bound that sizes the launch grids
    x = make_inputs(w)
    kv_len = x["kv_len"].tolist()
    dev = torch.device("cuda:0")
    layer_bytes = sum(v.numel() * v.element_size() for v in x.values()
                      if isinstance(v, torch.Tensor))
    n_layers = args.layers or min(512, max(2, -(-(1 << 30) // layer_bytes)))
    layers = []
    for _ in range(n_layers):
        layers.append({kk: (v.to(dev) if isinstance(v, torch.Tensor) else v) for kk, v in x.items()})
    B, S, L = w.B, w.S, w.L
    scores = torch.empty((B, S, L), dtype=torch.float32, device=dev) if w.has_indexer else None
    idx = torch.empty((B, S, w.k), dtype=torch.int32, device=dev)
    out = torch.empty((B, S, w.H_q, w.D), dtype={"f32": torch.float32, "f16": torch.float16,
                                                  "bf16": torch.bfloat16}[w.out_dtype], device=dev)
    topk_ws = None
    if w.has_indexer:
        nb = dsa.dsa_topk_workspace_bytes(B, S, L, w.k)
        topk_ws = torch.empty(max(nb, 16), dtype=torch.uint8, device=dev)
    g0 = layers[0]
    a0 = dsa.attention_args(g0["q"], g0["k_cache"], g0["v_cache"], idx, g0["kv_len"], out,
                            g0["k_scale"], g0["v_scale"], max_kv_len=w.max_kv_len)
    attn_ws = torch.empty(max(dsa.dsa_attention_workspace_bytes(a0, decode), 16),
                          dtype=torch.uint8, device=dev)
    attn = dsa.dsa_attention_decode if decode else dsa.dsa_attention_prefill

    def stage(name, g):
        if name == "indexer":
            dsa.dsa_indexer_score(g["q_idx"], g["w_idx"], g["key_state"], g["kv_len"], scores,
                                  max_kv_len=mx)
        elif name == "topk":
            dsa.dsa_topk(scores, g["kv_len"], w.k, idx, workspace=topk_ws, max_kv_len=mx)
        else:
            ind = idx if w.has_indexer else g["indices"]
            attn(g["q"], g["k_cache"], g["v_cache"], ind, g["kv_len"], out,
                 k_scale=g["k_scale"], v_scale=g["v_scale"], workspace=attn_ws, max_kv_len=mx)

    stages = (["indexer", "topk"] if w.has_indexer else []) + ["attention"]

    # KV-cache append of the step's new tokens (timed on its own; the path's
    # step keeps the three stages above).
    new_dtype = w.kv_dtype if w.kv_dtype != "i8" else w.q_dtype
    nt = {kk: v.to(dev) for kk, v in make_new_tokens(B, S, w.H_kv, w.D, new_dtype,
                                                      D_idx=w.D_idx or 64,
                                                      idx_dtype=w.idx_dtype or "bf16").items()}

    def append_stage(g):
        dsa.dsa_cache_append(nt["k_new"], nt["v_new"], g["k_cache"], g["v_cache"], g["kv_len"],
                             k_scale=g["k_scale"], v_scale=g["v_scale"],
                             key_state_new=nt["key_state_new"] if w.has_indexer else None,
                             key_state=g["key_state"] if w.has_indexer else None)

    def layer_pass(g):
        for st in stages:
            stage(st, g)

    def step():
        for g in layers:
            layer_pass(g)

    stage_fns = {st: (lambda st=st: [stage(st, g) for g in layers]) for st in stages}
    # RMSNorm + rotary of the step's heads: query (-> q dtype of the path),
    # key (-> new K) and indexer query, FP16 output (BF16 for a BF16 path).
    rope_out = torch.float16 if w.q_dtype != "bf16" or w.kv_dtype == "f16" else torch.bfloat16
    rope_sets = []
    for H_, D_, seed_ in [(w.H_q, w.D, 21), (w.H_kv, w.D, 22)] + (
            [(w.H_idx, w.D_idx, 23)] if w.has_indexer else []):
        ri = {kk: v.to(dev) for kk, v in make_rope_inputs(
            B, S, H_, D_, L, "bf16" if w.q_dtype != "f32" else "f32", kv_len, seed=seed_).items()}
        ri["out"] = torch.empty_like(ri["x"], dtype=rope_out)
        rope_sets.append(ri)

    def rope_stage():
        for ri in rope_sets:
            dsa.dsa_rmsnorm_rope(ri["x"], ri["gamma"], ri["cos"], ri["sin"], ri["kv_len"], ri["out"])

    # Attention with the step's S newest tokens as auxiliary K/V.
    aux = {kk: v.to(dev) for kk, v in make_aux_inputs(
        B, S, w.H_kv, w.D, "f32" if w.kv_dtype == "f32" else "bf16", seed=24).items()}
    a_aux = dsa.attention_args(g0["q"], g0["k_cache"], g0["v_cache"], idx, g0["kv_len"], out,
                               g0["k_scale"], g0["v_scale"], max_kv_len=w.max_kv_len,
                               aux_k=aux["aux_k"], aux_v=aux["aux_v"])
    aux_ws = torch.empty(max(dsa.dsa_attention_workspace_bytes(a_aux, decode), 16),
                         dtype=torch.uint8, device=dev)

    def attention_aux_stage(g):
        ind = idx if w.has_indexer else g["indices"]
        attn(g["q"], g["k_cache"], g["v_cache"], ind, g["kv_len"], out,
             k_scale=g["k_scale"], v_scale=g["v_scale"], workspace=aux_ws, max_kv_len=mx,
             aux_k=aux["aux_k"], aux_v=aux["aux_v"])

    extra_fns = {"cache_append": lambda: [append_stage(g) for g in layers],
                 "rmsnorm_rope": lambda: [rope_stage() for _ in layers],
                 "attention_aux": lambda: [attention_aux_stage(g) for g in layers]}

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    K = args.steps

    if args.pmc_run:
        # Reference copy of known size: its FETCH_SIZE / WRITE_SIZE calibrate
        # the counters (bytes per KiB reported).
        ref_bytes = 256 << 20
        src = torch.empty(ref_bytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        for st in stages:
            for g in layers[:4]:
                stage(st, g)
            torch.cuda.synchronize()
        sb = stage_bytes(w, kv_len)
        print(json.dumps({"pmc_run": w.name, "reference_copy_bytes": ref_bytes,
                          "stage_bytes_per_call": {st: sb[st] for st in stages}}), flush=True)
        return

    def timed(fn, reps):
        """Average ms per fn() over `reps` calls, HIP events on the launch stream."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    mode = "eager"
    run_step, run_stage = step, dict(stage_fns, **extra_fns)
    if not args.eager:
        # One step (every layer, every stage) captured as a HIP graph and
        # replayed; each stage alone (over every layer) is a graph of its own.
        try:
            s_cap = torch.cuda.Stream()
            s_cap.wait_stream(torch.cuda.current_stream())
            graphs = {}
            with torch.cuda.stream(s_cap):
                for name, fn in [("step", step)] + list(stage_fns.items()) + list(extra_fns.items()):
                    fn()                                   # warm-up on the capture stream
                    torch.cuda.synchronize()
                    gph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gph, stream=s_cap):
                        fn()
                    graphs[name] = gph
            torch.cuda.current_stream().wait_stream(s_cap)
            torch.cuda.synchronize()
            run_step = graphs["step"].replay
            run_stage = {st: graphs[st].replay for st in list(stages) + list(extra_fns)}
            # As many untimed replays as timed ones: the first replays of a
            # step made of long memory-bound kernels (the INT8 batched
            # decode) ran about 3% slower than steady state.
            for _ in range(max(3, args.steps)):
                run_step()
            torch.cuda.synchronize()
            mode = "hip_graph"
        except Exception as ex:     # capture unsupported here: time eager launches
            print(f"graph capture failed ({ex}); timing eager launches", file=sys.stderr)
            run_step, run_stage = step, dict(stage_fns, **extra_fns)

    # ---- timed region: K steps, then K replays of each stage alone
    ms_per_step = timed(run_step, K)
    us_per_layer = ms_per_step * 1e3 / n_layers
    stage_us = {st: timed(run_stage[st], K) * 1e3 / n_layers for st in stages}
    extra_us = {st: timed(run_stage[st], K) * 1e3 / n_layers for st in extra_fns}
    dominant = max(stage_us, key=stage_us.get)
    dom_us = stage_us[dominant]
    eager_us = timed(step, max(3, K // 5)) * 1e3 / n_layers if mode != "eager" else us_per_layer
    sb = stage_bytes(w, kv_len)
    dom_gbps = sb[dominant] / (dom_us * 1e-6) / 1e9
    traffic = None
    if sources_digest() == MEASURED_TRAFFIC["sources"]:
        traffic = MEASURED_TRAFFIC.get(w.name, {}).get(dominant)
    path_gbps = sb["path"] / (us_per_layer * 1e-6) / 1e9
    result = {
        "metric": METRIC,
        "value": round(us_per_layer, 3),
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "f16", "bf16": "bf16", "i8": "i8", "f32": "f32"}[w.kv_dtype],
        "data": "synthetic",
        "config": {"workload": w.name, "B": B, "S": S, "L": L, "H_q": w.H_q, "H_kv": w.H_kv,
                   "D": w.D, "k": w.k, "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype,
                   "out_dtype": w.out_dtype, "indexer": (f"{w.H_idx}x{w.D_idx}"
                                                         if w.has_indexer else None),
                   "layers_per_step": n_layers, "attention_form": "decode" if decode else "prefill",
                   "kv_len": kv_len if w.kv_len is not None else "L for every sequence",
                   "max_kv_len": mx},
        "tokens_per_s": round(B * S / (us_per_layer * 1e-6), 1),
        "launch_mode": mode,
        "eager_us_per_layer": round(eager_us, 3),
        "path_hbm_gbps": round(path_gbps, 1),
        "stage_us": {k2: round(v, 3) for k2, v in stage_us.items()},
        "roofline": {"bound": "hbm", "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "stage": dominant, "us_per_call": round(dom_us, 3),
                     "timing": f"{mode} replays of the {dominant} stage over all layers",
                     "bytes_per_call": sb[dominant]},
        "extra_stages": {st: {"us_per_call": round(v, 3), "bytes_per_call": sb[st],
                              "hbm_gbps": round(sb[st] / (v * 1e-6) / 1e9, 1),
                              "note": {"cache_append": "KV-cache append of the step's new tokens",
                                       "rmsnorm_rope": "RMSNorm + rotary of the step's query, key "
                                                       "and indexer-query heads",
                                       "attention_aux": "attention with the step's S newest tokens "
                                                        "as auxiliary K/V"}[st]
                                      + "; measured on its own, not in value"}
                         for st, v in extra_us.items()},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, x, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
