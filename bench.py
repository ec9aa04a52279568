"""Benchmark of the dynamic sparse GQA attention hot path on one MI355X.

One step = the whole hot path (indexer score -> top-k -> sparse attention)
run once per "layer", cycling through N distinct layer buffer sets whose
total footprint exceeds 1 GiB (so that no layer's key-state or KV cache is
still resident in the 256 MB Infinity Cache when it is read again), for at
least 32 layers.  The reported value is the time per layer (microseconds):
step time / layers, on the speculative-decode workload at 32K context (B1
S8, FP16 KV).  The other four workloads (1K tiny
decode, 128K prefill chunk, INT8 batched decode at 64K, 256K decode) are
timed the same way and reported under `by_workload`.

Inputs are seeded and synthetic and already resident in HBM when the timed
region starts.  One step is captured as a HIP graph (through
torch.cuda.CUDAGraph) and replayed, as a decode step is in a serving loop
(--eager times plain launches); HIP events on the launch stream time K
replays after K untimed ones, each replay with its own event pair (mean,
p10, p90), then K replays of a graph of each stage alone.  Each stage gets a
roofline against the bound that fits it: HBM bytes for the decode stages and
the top-k, the score write for the prefill indexer (with its per-head
FLOP rate beside it), and for the prefill attention the rate at which the
same rows are gathered with no compute, measured in the same run.  Ceilings
(streaming read and copy, a BF16 MFMA loop, 256-byte row gathers, and a
graph of do-nothing kernels with the step's grids) are measured first.
The CPU baseline times the FP64 oracle on the host on a bounded sample.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "µs/layer + achieved HBM GB/s for sparse GQA decode at 32K–256K ctx"
VALUE_WORKLOAD = "spec_decode_32k"
BY_WORKLOAD = ("tiny_decode_1k", "prefill_128k", "int8_batched_decode_64k", "decode_256k")

# HBM-side bytes per stage call, measured with rocprofv3 --pmc FETCH_SIZE and
# --pmc WRITE_SIZE (each scaled by the counts of a 256 MiB reference copy)
# for kernel sources whose digest is `sources`; the summaries are
# profiles/<workload>_hot_path_kernels.txt.  Reported only while the kernel
# sources still have that digest.
MEASURED_TRAFFIC = {
    "sources": "dd5f41cca957d375",
    "tiny_decode_1k": {
        "indexer": 129082,
        "topk": 17793,
        "attention": 81911
    },
    "spec_decode_32k": {
        "indexer": 5436168,
        "topk": 1321780,
        "attention": 18115341
    },
    "prefill_128k": {
        "indexer": 1185967203,
        "topk": 1090173510,
        "attention": 1912552308
    },
    "int8_batched_decode_64k": {
        "attention": 1153657589
    },
    "decode_256k": {
        "indexer": 42208151,
        "topk": 10656706,
        "attention": 20332493
    }
}

MIN_LAYER_STEPS = 32            # layers per timed step (a deep model's step)
MIN_TOUCHED = 512 << 20         # bytes read per pass over the layer sets (2x the Infinity Cache)
MAX_SET_BYTES = 48 << 30        # device memory the layer sets may take
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense BF16/FP16 MFMA
ELT = {"f32": 4, "f16": 2, "bf16": 2, "i8": 1}


def sources_digest():
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_gqa_attention_amd", "csrc")
    for f in sorted(sum((glob.glob(os.path.join(csrc, p)) for p in ("*.hip", "*.h", "*.cpp")), [])):
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--workload", default=VALUE_WORKLOAD)
    p.add_argument("--by-workload", default="all",
                   help="'all' (the four other workloads), 'none', or a comma-separated list")
    p.add_argument("--layers", type=int, default=0, help="layer buffer sets (0: >= 1 GiB)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--eager", action="store_true",
                   help="time eager launches instead of HIP-graph replays")
    p.add_argument("--cpu-seconds", type=float, default=20.0,
                   help="rough budget of host seconds for the CPU baseline")
    p.add_argument("--pmc-run", action="store_true",
                   help="for counter collection: a 256 MiB reference copy, then each stage "
                        "eagerly on 4 distinct layers; prints the bytes each should move")
    return p.parse_args()


# ------------------------------------------------------------------ algorithmic work
def rows_of(w, kv_len):
    return [(b, s, kv_len[b] - w.S + s) for b in range(w.B) for s in range(w.S)]


def stage_work(w, kv_len):
    """What each stage's contract must move and compute for one layer.

    Bytes count each input of the call once and each output once.  Of these,
    `abi_bytes` are the score matrix the 4-call boundary materialises (the
    indexer writes it, the top-k reads it): the method itself does not need
    it, so the whole-path figure leaves it out.  FLOPs count 2 H_idx D_idx
    per causal (query, key) pair for the indexer and 4 D per (query head,
    selected key) for attention.
    """
    B, S, k = w.B, w.S, w.k
    rows = rows_of(w, kv_len)
    valid = [max(0, min(k, pos + 1)) for _, _, pos in rows]
    out = {}
    if w.has_indexer:
        ie = ELT[w.idx_dtype]
        key_state = sum(kv_len) * w.D_idx * ie
        q_idx = B * S * w.H_idx * (w.D_idx * ie + 4)
        pairs = sum(max(0, pos + 1) for _, _, pos in rows)
        scores = sum(S * kv_len[b] for b in range(B)) * 4
        out["indexer"] = {"bytes": key_state + q_idx + scores, "abi_bytes": scores,
                          "flops": 2.0 * w.H_idx * w.D_idx * pairs}
        out["topk"] = {"bytes": pairs * 4 + B * S * k * 4, "abi_bytes": pairs * 4, "flops": 0.0}
    row_bytes = w.H_kv * w.D * ELT[w.kv_dtype] * 2 + (w.H_kv * 4 * 2 if w.kv_dtype == "i8" else 0)
    q = B * S * w.H_q * w.D * ELT[w.q_dtype]
    o = B * S * w.H_q * w.D * ELT[w.out_dtype]
    out["attention"] = {"bytes": sum(valid) * row_bytes + q + o + B * S * k * 4, "abi_bytes": 0,
                        "gathered": sum(valid) * row_bytes,
                        "flops": 4.0 * w.D * w.H_q * sum(valid)}
    path = out["attention"]["bytes"] + (out["indexer"]["bytes"] - out["indexer"]["abi_bytes"]
                                        if w.has_indexer else 0)
    out["path"] = {"bytes": path}
    # Steps measured next to the path (not in the value): the KV-cache append
    # of the step's new tokens, RMSNorm + rotary of its query, key and
    # indexer-query heads, attention with the S newest tokens as auxiliary K/V.
    new_elt = ELT[w.kv_dtype] if w.kv_dtype != "i8" else ELT[w.q_dtype]
    app = B * S * w.H_kv * w.D * (new_elt + ELT[w.kv_dtype]) * 2
    if w.kv_dtype == "i8":
        app += B * S * w.H_kv * 4 * 2
    if w.has_indexer:
        app += B * S * w.D_idx * ELT[w.idx_dtype] * 2
    out["cache_append"] = {"bytes": app}
    rope = B * S * (w.H_q + w.H_kv) * w.D * (ELT[w.q_dtype] + 2) + B * S * w.D * 4 * 2
    if w.has_indexer:
        rope += B * S * w.H_idx * w.D_idx * (ELT[w.idx_dtype] + 2) + B * S * w.D_idx * 4 * 2
    out["rmsnorm_rope"] = {"bytes": rope}
    aux_elt = 4 if w.kv_dtype == "f32" else 2
    out["attention_aux"] = {"bytes": out["attention"]["bytes"] + B * S * w.H_kv * w.D * aux_elt * 2}
    return out


def stage_bound(w, stage):
    """The roofline that bounds `stage` on workload `w`.  The prefill indexer
    folds the head weights into the query, so its MFMA work is a fraction of
    the method's per-head count and its score stores bound it: HBM, like the
    decode stages (against the measured write ceiling)."""
    if stage == "attention" and not w.decode_form:
        return "gather"        # every token gathers its own 2048 rows from a cache-resident KV
    return "hbm"


def roofline_entry(w, stage, work, us, ceilings, fold_parts=0):
    bound = stage_bound(w, stage)
    sec = us * 1e-6
    e = {"bound": bound, "us_per_call": round(us, 3)}
    gbps = work["bytes"] / sec / 1e9
    e.update(achieved=round(gbps, 1), unit="GB/s", bytes_per_call=work["bytes"])
    if bound == "gather":
        # the gathered K/V rows against the rate at which the same rows,
        # in the same order, are read with nothing else to do (measured
        # in this run on this layer's indices); the query, output and
        # indices stream besides
        c = ceilings.get("attention_gather_gbps")
        gb = work["gathered"] / sec / 1e9
        e.update(achieved=round(gb, 1), bytes_per_call=work["gathered"], peak=c,
                 frac=round(gb / c, 4) if c else None, ceiling_name="attention_gather_gbps")
    else:
        e.update(peak=HBM_PEAK_GBPS, frac=round(gbps / HBM_PEAK_GBPS, 4))
        # the indexer's bytes are mostly its score stores, the others' loads
        cn = "hbm_write_gbps" if stage == "indexer" else "hbm_read_gbps"
        c = ceilings.get(cn)
        if c:
            e.update(ceiling=c, frac_of_ceiling=round(gbps / c, 4), ceiling_name=cn)
    if work.get("abi_bytes"):
        e["abi_bytes_per_call"] = work["abi_bytes"]   # score matrix of the 4-call boundary
    if stage == "attention" and work.get("flops"):
        tf = work["flops"] / sec / 1e12
        e["mfma_tflops"] = round(tf, 2)
        e["mfma_frac"] = round(tf / MFMA_PEAK_TFLOPS, 4)
    if stage == "indexer" and work.get("flops"):
        # the method's per-head FLOP count over the stage time, and the MFMA
        # work the kernel issues: the same for the per-head kernels; the
        # folded prefill kernel contracts one folded query, taken in
        # fold_parts 16-bit parts, instead of H_idx heads
        e["per_head_tflops"] = round(work["flops"] / sec / 1e12, 1)
        issued = work["flops"] * (fold_parts / w.H_idx if fold_parts else 1.0)
        e["mfma_tflops"] = round(issued / sec / 1e12, 1)
        e["mfma_frac"] = round(issued / sec / 1e12 / MFMA_PEAK_TFLOPS, 4)
        if fold_parts:
            e["mfma_note"] = (f"head weights folded into the query: {fold_parts} MFMA parts per "
                              f"(token, key) tile against {w.H_idx} heads in the per-head form")
    return e


# ------------------------------------------------------------------ CPU baseline
_CPU = {}          # inputs of the CPU baseline, set before the worker pool forks


def _cpu_row(task):
    """Oracle stages of one query row, timed (runs in a pool worker)."""
    import numpy as np
    import oracle
    from threadpoolctl import threadpool_limits
    name, b, s = task
    d = _CPU[name]
    pos = d["kv_len"][b] - d["S"] + s
    t = {}
    with threadpool_limits(1, user_api="blas"):
        if d["q_idx"] is not None:
            t0 = time.perf_counter()
            sc = oracle.indexer_scores_row(d["q_idx"][b, s], d["w_idx"][b, s], d["key_state"][b],
                                           pos)
            t["score"] = time.perf_counter() - t0
            t0 = time.perf_counter()
            idx = oracle.topk_row(sc, pos, d["k"])
            t["sort"] = time.perf_counter() - t0
        else:
            idx = np.arange(d["k"])
        t0 = time.perf_counter()
        oracle.attention_row(d["q"][b, s], d["K"][b], d["V"][b], idx, pos, d["kv_len"][b],
                             1.0 / math.sqrt(d["q"].shape[-1]))
        t["attention"] = time.perf_counter() - t0
    return t


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(workloads, inputs, budget_s):
    """The FP64 oracle on the host's cores, per workload and per stage.

    A fork-started process pool (before any GPU use) runs up to one row per
    worker at a time, each worker single-threaded; a workload's sampled rows
    run in parallel and their wall time times the number of such rounds a
    whole layer needs gives µs/layer.  Inputs are converted to FP64 NumPy
    arrays beforehand (not timed).
    """
    import multiprocessing as mp
    import numpy as np
    cores = len(os.sched_getaffinity(0))
    workers = max(1, min(cores, 16))
    t_start = time.perf_counter()
    for w in workloads:
        x = inputs[w.name]
        kv = x["kv_len"].tolist()
        # at most `workers` rows, from at most two sequences (a sequence's
        # cache in FP64 is up to 1 GiB), spread over the layer
        rows = [(b, s) for b in range(min(w.B, 2)) for s in range(w.S)]
        if len(rows) > workers:
            step = len(rows) / workers
            rows = [rows[int(i * step)] for i in range(workers)]
        bs = sorted({b for b, _ in rows})
        f64 = lambda t: t.double().numpy() if t.dtype.is_floating_point else t.numpy().astype(np.float64)
        K = {}
        V = {}
        for b in bs:
            if w.kv_dtype == "i8":
                K[b] = f64(x["k_cache"][b]) * f64(x["k_scale"][b])[..., None]
                V[b] = f64(x["v_cache"][b]) * f64(x["v_scale"][b])[..., None]
            else:
                K[b], V[b] = f64(x["k_cache"][b]), f64(x["v_cache"][b])
        _CPU[w.name] = {"S": w.S, "k": w.k, "kv_len": kv, "q": f64(x["q"]), "K": K, "V": V,
                        "q_idx": f64(x["q_idx"]) if w.has_indexer else None,
                        "w_idx": f64(x["w_idx"]) if w.has_indexer else None,
                        "key_state": ({b: f64(x["key_state"][b]) for b in bs}
                                      if w.has_indexer else None),
                        "rows": rows}
    ctx = mp.get_context("fork")
    results = {}
    with ctx.Pool(workers) as pool:
        for w in workloads:
            d = _CPU[w.name]
            tasks = [(w.name, b, s) for b, s in d["rows"]]
            pool.map(_cpu_row, tasks, chunksize=1)      # untimed: first touches of the inputs
            reps, walls, per = 0, [], []
            while True:
                t0 = time.perf_counter()
                per.extend(pool.map(_cpu_row, tasks, chunksize=1))
                walls.append(time.perf_counter() - t0)
                reps += 1
                if reps >= 10 or sum(walls) * (reps + 1) / reps > budget_s / len(workloads):
                    break
            wall = sorted(walls)[len(walls) // 2]
            rounds = math.ceil(w.B * w.S / len(tasks))
            stage_s = {st: float(np.median([p[st] for p in per])) for st in per[0]}
            results[w.name] = {
                "us_per_layer": round(wall * rounds * 1e6, 1),
                "stage_us_per_row": {st: round(v * 1e6, 1) for st, v in stage_s.items()},
                # a stage's share of the layer: its median row time per round
                "stage_us_per_layer": {st: round(v * 1e6 * rounds, 1) for st, v in stage_s.items()},
                "sampled_rows": len(tasks), "rounds_per_layer": rounds, "repeats": reps,
            }
    return {"cores": cores, "workers": workers, "cpu_model": cpu_model(),
            "host_seconds": round(time.perf_counter() - t_start, 1), "by_workload": results}


# ------------------------------------------------------------------ GPU side
def parse_grid(text, key):
    """Workgroups and threads of the launch named `key` in a plan description."""
    import sparse_gqa_attention_amd as dsa
    f = dsa.plan_fields(text)
    if key not in f:
        return None
    g = 1
    for v in f[key].split("x"):
        g *= int(v)
    return g


def measure_ceilings(torch, dev, K):
    """Measured ceilings of this GPU: HBM streaming read, write and copy, a BF16 MFMA
    loop, and uniformly random 256-byte row gathers from a 128 MiB
    (cache-resident) and a 2 GiB buffer."""
    from sparse_gqa_attention_amd import roofline as rl
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def tmin(fn, reps=max(5, K)):
        fn()
        torch.cuda.synchronize()
        best = None
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        return best

    out = {}
    big = torch.empty(2 << 30, dtype=torch.uint8, device=dev)
    big.random_(0, 255)
    out["hbm_read_gbps"] = round(big.numel() / tmin(lambda: rl.read(big, sink)) / 1e9, 1)
    out["hbm_write_gbps"] = round(big.numel() / tmin(lambda: rl.write(big)) / 1e9, 1)
    half = big.numel() // 2
    src, dst = big[:half], big[half:]
    out["hbm_copy_gbps"] = round(2 * half / tmin(lambda: rl.copy(src, dst)) / 1e9, 1)
    wgs, iters = 2048, 2000
    flops = rl.LIB.dsa_roofline_mfma_flops(wgs, iters)
    out["mfma_bf16_tflops"] = round(flops / tmin(lambda: rl.mfma(sink, wgs, iters)) / 1e12, 1)
    g = torch.Generator(device="cpu").manual_seed(7)
    n_rows = 1 << 24                                   # 4 GiB of gathered rows
    for name, nbytes in (("random_gather_128mib_gbps", 128 << 20),
                         ("random_gather_2gib_gbps", 2 << 30)):
        rows = torch.randint(0, nbytes // 256, (n_rows,), generator=g, dtype=torch.int32).to(dev)
        buf = big[:nbytes]
        out[name] = round(n_rows * 256 / tmin(lambda: rl.gather(buf, rows, sink)) / 1e9, 1)
        del rows
    del big
    torch.cuda.empty_cache()
    return out


def run_workload(w, args, torch, dev, ceilings, x, extras):
    import sparse_gqa_attention_amd as dsa
    from sparse_gqa_attention_amd import roofline as rl
    from dsa_synth import make_aux_inputs, make_new_tokens, make_rope_inputs

    decode = w.decode_form
    mx = w.max_kv_len
    kv_len = x["kv_len"].tolist()
    layer_bytes = sum(v.numel() * v.element_size() for v in x.values()
                      if isinstance(v, torch.Tensor))
    # Distinct sets: at least 1 GiB of buffers, and at least MIN_TOUCHED bytes
    # read per pass over them (key-state rows, gathered K/V rows, queries):
    # a layer reads only a fraction of its KV cache, and each set must leave
    # the Infinity Cache before it is read again.
    touched = stage_work(w, kv_len)["path"]["bytes"]
    n_layers = args.layers or min(512, max(2, -(-(1 << 30) // layer_bytes),
                                          -(-MIN_TOUCHED // max(1, touched))))
    while not args.layers and n_layers > 2 and n_layers * layer_bytes > MAX_SET_BYTES:
        n_layers -= 1
    layers = [{kk: (v.to(dev) if isinstance(v, torch.Tensor) else v) for kk, v in x.items()}
              for _ in range(n_layers)]
    # A step runs at least MIN_LAYER_STEPS layers, cycling through the
    # distinct sets (each set recurs only after every other set has passed
    # through the Infinity Cache), so that one replay's launch overhead is
    # spread over as many layers as a deep model's step has, whatever the
    # set count.
    seq = layers * max(1, -(-MIN_LAYER_STEPS // n_layers))
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
                            g0["k_scale"], g0["v_scale"], max_kv_len=mx)
    attn_ws = torch.empty(max(dsa.dsa_attention_workspace_bytes(a0, decode), 16),
                          dtype=torch.uint8, device=dev)
    attn = dsa.dsa_attention_decode if decode else dsa.dsa_attention_prefill
    plans = {}
    if w.has_indexer:
        plans["indexer"] = dsa.dsa_describe_plan(dsa.DSA_PLAN_INDEXER, B, S, L, mx, D_idx=w.D_idx)
        plans["topk"] = dsa.dsa_describe_plan(dsa.DSA_PLAN_TOPK, B, S, L, mx, k=w.k)
    plans["attention"] = dsa.dsa_describe_plan(
        dsa.DSA_PLAN_ATTENTION_DECODE if decode else dsa.DSA_PLAN_ATTENTION_PREFILL, attention=a0)

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

    def step():
        for g in seq:
            for st in stages:
                stage(st, g)

    fns = {"step": step}
    fns.update({st: (lambda st=st: [stage(st, g) for g in seq]) for st in stages})

    # The launch floor: the step's kernels as do-nothing kernels (each
    # workgroup reads one word) with the same grids, replayed the same way.
    word = torch.zeros(16, dtype=torch.int32, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    floor_launches = []
    for st in stages:
        f = dsa.plan_fields(plans[st])
        for key, tkey in (("grid", "threads"), ("chunk_grid", "chunk_threads"),
                          ("select_grid", "select_threads"), ("merge_grid", None)):
            if key in f:
                floor_launches.append((parse_grid(plans[st], key),
                                       int(f.get(tkey, "256")) if tkey else 256))
    floor_launches = [(min(g, 65535), t) for g, t in floor_launches]

    def floor_step():
        for _ in seq:
            for g, t in floor_launches:
                rl.floor(word, sink, g, t)
    fns["floor"] = floor_step

    if extras:
        new_dtype = w.kv_dtype if w.kv_dtype != "i8" else w.q_dtype
        nt = {kk: v.to(dev) for kk, v in make_new_tokens(B, S, w.H_kv, w.D, new_dtype,
                                                          D_idx=w.D_idx or 64,
                                                          idx_dtype=w.idx_dtype or "bf16").items()}

        def append_stage(g):
            dsa.dsa_cache_append(nt["k_new"], nt["v_new"], g["k_cache"], g["v_cache"], g["kv_len"],
                                 k_scale=g["k_scale"], v_scale=g["v_scale"],
                                 key_state_new=nt["key_state_new"] if w.has_indexer else None,
                                 key_state=g["key_state"] if w.has_indexer else None)
        rope_out = torch.float16 if w.q_dtype != "bf16" or w.kv_dtype == "f16" else torch.bfloat16
        rope_sets = []
        for H_, D_, seed_ in [(w.H_q, w.D, 21), (w.H_kv, w.D, 22)] + (
                [(w.H_idx, w.D_idx, 23)] if w.has_indexer else []):
            ri = {kk: v.to(dev) for kk, v in make_rope_inputs(
                B, S, H_, D_, L, "bf16" if w.q_dtype != "f32" else "f32", kv_len,
                seed=seed_).items()}
            ri["out"] = torch.empty_like(ri["x"], dtype=rope_out)
            rope_sets.append(ri)

        rope_jobs = [dict(x=ri["x"], gamma=ri["gamma"], cos_cache=ri["cos"], sin_cache=ri["sin"],
                          kv_len=ri["kv_len"], out=ri["out"]) for ri in rope_sets]

        def rope_stage():
            # the step's query, key and indexer-query heads in one launch
            dsa.dsa_rmsnorm_rope_multi(rope_jobs)
        aux = {kk: v.to(dev) for kk, v in make_aux_inputs(
            B, S, w.H_kv, w.D, "f32" if w.kv_dtype == "f32" else "bf16", seed=24).items()}
        a_aux = dsa.attention_args(g0["q"], g0["k_cache"], g0["v_cache"], idx, g0["kv_len"], out,
                                   g0["k_scale"], g0["v_scale"], max_kv_len=mx,
                                   aux_k=aux["aux_k"], aux_v=aux["aux_v"])
        aux_ws = torch.empty(max(dsa.dsa_attention_workspace_bytes(a_aux, decode), 16),
                             dtype=torch.uint8, device=dev)

        def attention_aux_stage(g):
            ind = idx if w.has_indexer else g["indices"]
            attn(g["q"], g["k_cache"], g["v_cache"], ind, g["kv_len"], out,
                 k_scale=g["k_scale"], v_scale=g["v_scale"], workspace=aux_ws, max_kv_len=mx,
                 aux_k=aux["aux_k"], aux_v=aux["aux_v"])
        fns["cache_append"] = lambda: [append_stage(g) for g in seq]
        fns["rmsnorm_rope"] = lambda: [rope_stage() for _ in seq]
        fns["attention_aux"] = lambda: [attention_aux_stage(g) for g in seq]

    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    K = args.steps

    if args.pmc_run:
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
        work = stage_work(w, kv_len)
        print(json.dumps({"pmc_run": w.name, "reference_copy_bytes": ref_bytes,
                          "stage_bytes_per_call": {st: work[st]["bytes"] + work[st]["abi_bytes"]
                                                   for st in stages},
                          "stage_flops_per_call": {st: work[st]["flops"] for st in stages},
                          "plans": plans}), flush=True)
        return None

    def dist(fn, reps):
        """Per-call times (ms) of `reps` calls, each between its own HIP events
        on the launch stream, and the mean over the whole span."""
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        torch.cuda.synchronize()
        for e0, e1 in ev:
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        each = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
        span = ev[0][0].elapsed_time(ev[-1][1]) / reps
        return {"mean": span, "p10": each[int(0.1 * (reps - 1))], "p50": each[(reps - 1) // 2],
                "p90": each[int(math.ceil(0.9 * (reps - 1)))]}

    mode = "eager"
    run = dict(fns)
    if not args.eager:
        try:
            s_cap = torch.cuda.Stream()
            s_cap.wait_stream(torch.cuda.current_stream())
            graphs = {}
            with torch.cuda.stream(s_cap):
                for name, fn in fns.items():
                    fn()
                    torch.cuda.synchronize()
                    gph = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gph, stream=s_cap):
                        fn()
                    graphs[name] = gph
            torch.cuda.current_stream().wait_stream(s_cap)
            torch.cuda.synchronize()
            run = {name: graphs[name].replay for name in fns}
            # As many untimed replays as timed ones: the first replays of a
            # step made of long memory-bound kernels ran about 3% slower
            # than steady state.
            for _ in range(max(3, K)):
                run["step"]()
            torch.cuda.synchronize()
            mode = "hip_graph"
        except Exception as ex:     # capture unsupported here: time eager launches
            print(f"graph capture failed ({ex}); timing eager launches", file=sys.stderr)
            run = dict(fns)

    # The gather ceiling of a prefill attention: the same K and V row reads,
    # in the same launch order, schedule and tiling, with nothing else to do
    # (the probe kernel), on this layer's caches and indices.
    if not decode and w.D * ELT[w.kv_dtype] == 256:
        wave_rows = dsa.plan_fields(plans["attention"]).get("schedule") == "wave_rows"
        run["step"]()
        torch.cuda.synchronize()
        ind = idx if w.has_indexer else g0["indices"]
        best = None
        for _ in range(max(5, K)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            rl.kv_gather(g0["k_cache"], g0["v_cache"], ind, S, sink, wave_rows=wave_rows)
            e1.record()
            torch.cuda.synchronize()
            t = e0.elapsed_time(e1) * 1e-3
            best = t if best is None else min(best, t)
        gathered = stage_work(w, kv_len)["attention"]["gathered"]
        ceilings = dict(ceilings, attention_gather_gbps=round(gathered / best / 1e9, 1))

    per_layer = lambda d: {kk: round(v * 1e3 / len(seq), 3) for kk, v in d.items()}
    step_d = per_layer(dist(run["step"], K))
    stage_d = {st: per_layer(dist(run[st], K)) for st in stages}
    floor_d = per_layer(dist(run["floor"], K))
    extra_d = {st: per_layer(dist(run[st], K)) for st in ("cache_append", "rmsnorm_rope",
                                                          "attention_aux") if st in run}
    eager_d = per_layer(dist(step, max(3, K // 5))) if mode != "eager" else step_d
    work = stage_work(w, kv_len)
    fold_parts = 0
    if w.has_indexer and "indexer_fold_kernel" in plans.get("indexer", ""):
        fold_parts = 3 if w.idx_dtype == "bf16" else 2
    roof = {st: roofline_entry(w, st, work[st], stage_d[st]["mean"], ceilings, fold_parts)
            for st in stages}
    measured = MEASURED_TRAFFIC.get(w.name, {}) if sources_digest() == MEASURED_TRAFFIC["sources"] else {}
    for st in stages:
        # HBM-side bytes per call from rocprofv3 FETCH_SIZE + WRITE_SIZE
        # (null once the kernel sources differ from the measured ones)
        roof[st]["traffic"] = measured.get(st)
        if roof[st]["bound"] == "gather" and measured.get(st):
            # the gathered rows' HBM-side share: measured traffic per call
            # over the stage time, against the HBM peak
            roof[st]["hbm_traffic_frac"] = round(
                measured[st] / (stage_d[st]["mean"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    path_gbps = work["path"]["bytes"] / (step_d["mean"] * 1e-6) / 1e9
    res = {
        "us_per_layer": step_d,
        "tokens_per_s": round(B * S / (step_d["mean"] * 1e-6), 1),
        "launch_mode": mode,
        "layers_per_step": len(seq),
        "layer_sets": n_layers,
        "eager_us_per_layer": eager_d["mean"],
        "stage_us": stage_d,
        "stage_roofline": roof,
        "dominant_stage": max(stage_d, key=lambda s_: stage_d[s_]["mean"]),
        "path": {"bytes_per_layer": work["path"]["bytes"], "gbps": round(path_gbps, 1),
                 "frac": round(path_gbps / HBM_PEAK_GBPS, 4),
                 "note": "whole layer, the score round trip of the 4-call boundary excluded"},
        "launch_floor_us_per_layer": floor_d["mean"],
        "launch_floor_kernels": [f"{g}x{t}" for g, t in floor_launches],
        "plans": plans,
        "config": {"workload": w.name, "B": B, "S": S, "L": L, "H_q": w.H_q, "H_kv": w.H_kv,
                   "D": w.D, "k": w.k, "q_dtype": w.q_dtype, "kv_dtype": w.kv_dtype,
                   "out_dtype": w.out_dtype,
                   "indexer": f"{w.H_idx}x{w.D_idx}" if w.has_indexer else None,
                   "attention_form": "decode" if decode else "prefill",
                   "kv_len": kv_len if w.kv_len is not None else "L for every sequence",
                   "max_kv_len": mx},
    }
    if "attention_gather_gbps" in ceilings:
        res["attention_gather_ceiling_gbps"] = ceilings["attention_gather_gbps"]
    if extra_d:
        res["extra_stages"] = {
            st: {"us_per_call": v["mean"], "p10": v["p10"], "p90": v["p90"],
                 "bytes_per_call": work[st]["bytes"],
                 "hbm_gbps": round(work[st]["bytes"] / (v["mean"] * 1e-6) / 1e9, 1),
                 "note": {"cache_append": "KV-cache append of the step's new tokens",
                          "rmsnorm_rope": "RMSNorm + rotary of the step's query, key and "
                                          "indexer-query heads",
                          "attention_aux": "attention with the step's S newest tokens as "
                                           "auxiliary K/V"}[st] + "; measured on its own, not in value"}
            for st, v in extra_d.items()}
    del seq, layers, scores, idx, out, topk_ws, attn_ws
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library runs "
              f"the hot path on a single MI355X and has no multi-GPU path.", file=sys.stderr)
        sys.exit(2)
    from dsa_synth import BY_NAME, make_inputs

    w_main = BY_NAME[args.workload]
    if args.by_workload == "none" or args.pmc_run:
        others = []
    elif args.by_workload == "all":
        others = [BY_NAME[n] for n in BY_WORKLOAD if n != w_main.name]
    else:
        others = [BY_NAME[n] for n in args.by_workload.split(",") if n and n != w_main.name]
    workloads = [w_main] + others
    inputs = {w.name: make_inputs(w) for w in workloads}

    # The CPU baseline runs first, in workers forked before any GPU use.
    cpu = None
    if not args.no_cpu_baseline and not args.pmc_run:
        cpu = cpu_baseline(workloads, inputs, args.cpu_seconds)

    import torch
    dev = torch.device("cuda:0")
    ceilings = {} if args.pmc_run else measure_ceilings(torch, dev, args.steps)
    main_res = run_workload(w_main, args, torch, dev, ceilings, inputs[w_main.name], extras=True)
    if main_res is None:          # counter-collection run
        return
    by = {}
    for w in others:
        by[w.name] = run_workload(w, args, torch, dev, ceilings, inputs.pop(w.name), extras=False)

    dom = main_res["dominant_stage"]
    droof = main_res["stage_roofline"][dom]
    traffic = None
    if sources_digest() == MEASURED_TRAFFIC["sources"]:
        traffic = MEASURED_TRAFFIC.get(w_main.name, {}).get(dom)
    roofline = {"bound": droof["bound"], "achieved": droof["achieved"], "peak": droof["peak"],
                "unit": droof["unit"], "frac": droof["frac"], "traffic": traffic, "stage": dom,
                "us_per_call": droof["us_per_call"],
                "timing": f"{main_res['launch_mode']} replays of the {dom} stage over all layers"}
    for kk in ("bytes_per_call", "flops_per_call", "abi_bytes_per_call", "ceiling",
               "frac_of_ceiling", "ceiling_name"):
        if kk in droof:
            roofline[kk] = droof[kk]
    result = {
        "metric": METRIC,
        "value": main_res["us_per_layer"]["mean"],
        "unit": "us/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["us_per_layer"]["mean"] * main_res["layers_per_step"] / 1e3, 4),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"f16": "f16", "bf16": "bf16", "i8": "i8", "f32": "f32"}[w_main.kv_dtype],
        "data": "synthetic",
        "config": main_res["config"],
        "roofline": roofline,
        "us_per_layer": main_res["us_per_layer"],
        "tokens_per_s": main_res["tokens_per_s"],
        "launch_mode": main_res["launch_mode"],
        "layers_per_step": main_res["layers_per_step"],
        "layer_sets": main_res["layer_sets"],
        "eager_us_per_layer": main_res["eager_us_per_layer"],
        "launch_floor_us_per_layer": main_res["launch_floor_us_per_layer"],
        "path": main_res["path"],
        "stage_us": main_res["stage_us"],
        "stage_roofline": main_res["stage_roofline"],
        "plans": main_res["plans"],
        "extra_stages": main_res.get("extra_stages"),
        "ceilings": ceilings,
        "by_workload": by,
    }
    if cpu is not None:
        c = cpu["by_workload"][w_main.name]
        result["cpu_baseline"] = {
            "value": c["us_per_layer"], "unit": "us/layer", "cores": cpu["workers"],
            "kind": "oracle",
            "sample": (f"{c['sampled_rows']} of the {w_main.B * w_main.S} query rows of one "
                       f"{w_main.name} layer (FP64 scores, full-sort top-k, dense masked "
                       f"attention), one row per single-threaded worker of a "
                       f"{cpu['workers']}-process pool on {cpu['cores']} affinity cores "
                       f"({cpu['cpu_model']}); median pool wall time x {c['rounds_per_layer']} "
                       f"round(s) per layer"),
            "stage_us_per_row": c["stage_us_per_row"],
            "cpu_model": cpu["cpu_model"], "affinity_cores": cpu["cores"],
            "host_seconds": cpu["host_seconds"],
            "by_workload": {n: v for n, v in cpu["by_workload"].items() if n != w_main.name},
        }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
