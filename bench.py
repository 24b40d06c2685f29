"""Benchmark of the DSA decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode-32k]

A step is one fused decode (lightning indexer -> deterministic top-k ->
sparse MLA) over a batch of 4 sequences at 32,768 tokens of context, k=2048,
64 indexer heads x 128 and 64 MLA heads over 576-d bf16 latent rows (one new
query per sequence, so tokens/step = batch). Inputs are seeded synthetic
arrays, resident in HBM before timing starts; the step cycles through
several copies of the caches so that repeats cannot be served from the
256 MB Infinity Cache.

Prints one JSON line: the metric, the decode step's roofline (its
algorithmic bytes over its measured time, against the HBM peak, with the
counted HBM traffic when a counter record of the same sources exists), a
per-kernel breakdown of the step, the indexer's own roofline, the CPU
oracle's throughput on a bounded sample, and (default workload) the same
measurements for the long-context fp8 decode, the determinism / replay
workload and the causal prefill pass.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA decode tokens/s @32K ctx, k=2048; achieved HBM GB/s vs peak"
HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFS = 2500.0  # dense bf16
MALL_BYTES = 256 << 20


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def latent_row_bytes(p) -> int:
    """Bytes of one gathered latent row: 576 elements (+4 B row scale for fp8)."""
    esz = {"bf16": 2, "f32": 4, "fp8_e4m3": 1}
    return 576 * esz[p.kv_dtype] + (4 if p.kv_dtype == "fp8_e4m3" else 0)


def attention_bytes(p) -> int:
    """Algorithmic bytes of one attention launch over k_eff keys per query:
    the selected latent rows, the indices, the queries and the outputs."""
    esz = {"bf16": 2, "f32": 4}
    k_eff = sum(min(p.k, int(x) + 1) for x in p.q_pos.astype(int))
    return (k_eff * latent_row_bytes(p) + p.R * p.k * 4 + p.R * p.H * 576 * esz[p.act_dtype]
            + p.R * p.H * (512 + 1) * 4)


def step_bytes(p) -> int:
    """Algorithmic HBM bytes of one decode step: every candidate indexer key
    (once, however many of the sequence's new tokens score it), every
    selected latent row, the queries, weights and the outputs."""
    esz = {"bf16": 2, "f32": 4, "fp8_e4m3": 1}
    n = p.seq_len.astype(int)
    keys = int(n.sum()) * p.D_I * esz[p.key_dtype] + (int(n.sum()) * 2 if p.key_dtype == "fp8_e4m3" else 0)
    k_eff = [min(p.k, int(x) + 1) for x in p.q_pos.astype(int)]
    gather = sum(k_eff) * latent_row_bytes(p)
    small = (p.R * p.H_I * p.D_I * esz[p.act_dtype] + p.R * p.H_I * 4 + p.R * p.H * 576 * esz[p.act_dtype]
             + p.R * p.H * 512 * 4 + p.R * p.H * 4 + p.R * p.k * 4)
    return keys + gather + small


def indexer_bytes(p) -> int:
    """Algorithmic bytes of one indexer launch: per candidate key its D_I
    elements (+2 B row scale for fp8) read and its fp32 score written; per
    query its H_I x D_I query and H_I weights."""
    esz = {"bf16": 2, "f32": 4, "fp8_e4m3": 1}
    n = int(p.seq_len.astype(int).sum())
    per_key = p.D_I * esz[p.key_dtype] + (2 if p.key_dtype == "fp8_e4m3" else 0) + 4 * p.tokens_per_seq
    per_query = p.H_I * p.D_I * esz[p.act_dtype] + p.H_I * 4
    return n * per_key + p.R * per_query


CSRC = os.path.join(ROOT, "sparse_attention_05_amd", "csrc")


def sources_sha() -> str:
    """sha256 over every kernel source (names and bytes, sorted by name)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        h.update(f.encode())
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"decode_step_{workload}_traffic.json")


def pmc_traffic(workload: str):
    """HBM bytes per step (and per kernel) from a committed counter record of
    the shipped sources, or None when absent or taken on other sources."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path))
        return rec if rec.get("sources_sha256") == sources_sha() else None
    except Exception:
        return None


COPY_BYTES = 256 << 20      # calibration pass for the HBM byte counters
PMC_STEPS = 20


def pmc_pass(workload: str):
    """Workload of the two rocprofv3 counter runs (FETCH_SIZE, then WRITE_SIZE):
    an elementwise negation over COPY_BYTES (reads and writes exactly that many
    bytes, to scale the counters) and PMC_STEPS fused decode steps on rotating
    input sets."""
    import torch
    from sparse_attention_05_amd import dsa, inputs
    torch.cuda.set_device(0)
    p = inputs.workload(workload, seed=0)
    max_len = int(p.seq_len.max())
    n_sets = max(2, math.ceil(2 * MALL_BYTES / step_bytes(p)))
    sets = [inputs.to_torch(p, "cuda") for _ in range(n_sets)]
    calls = [dsa.DecodeCall(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len, max_len, p.k,
                            p.scale, k_scale=d.k_scale, latent_scale=d.latent_scale, q_per_seq=p.tokens_per_seq)
             for d in sets]
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.neg(src, out=dst)
    for i in range(PMC_STEPS):
        calls[i % n_sets]()
    torch.cuda.synchronize()
    log(f"bench: pmc pass done ({PMC_STEPS} decode steps of {workload}, 3 passes over {COPY_BYTES >> 20} MiB)")


def ingest_pmc(workload: str, fetch_csv: str, write_csv: str):
    """Turn the two counter CSVs of pmc_pass into profiles/decode_step_<workload>_traffic.json:
    per kernel of the step, HBM bytes per launch (each counter scaled by bytes /
    counter of the negation pass) and launches per step; their sum per step."""
    import csv
    import statistics

    def per_dispatch(path, counter):
        vals = {}
        for row in csv.DictReader(open(path)):
            if row["Counter_Name"] != counter:
                continue
            key = (row["Kernel_Name"], row["Dispatch_Id"])
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
        by = {}
        for (name, _), v in vals.items():
            by.setdefault(name, []).append(v)
        return by

    f, w = per_dispatch(fetch_csv, "FETCH_SIZE"), per_dispatch(write_csv, "WRITE_SIZE")
    copy = [k for k in f if "neg" in k]
    kib = COPY_BYTES / 1024.0
    f_scale = kib / statistics.median(f[copy[0]])
    w_scale = kib / statistics.median(w[[k for k in w if "neg" in k][0]])
    from sparse_attention_05_amd import inputs
    p = inputs.workload(workload, seed=0)
    kernels, total = {}, 0.0
    for name in f:
        if "dsa::" not in name or name not in w:
            continue
        short = kernel_short_name(name).split("<")[0]
        per_launch = 1024.0 * (statistics.median(f[name]) * f_scale + statistics.median(w[name]) * w_scale)
        per_step = len(f[name]) / PMC_STEPS
        kernels[short] = {"bytes_per_launch": per_launch, "launches_per_step": per_step,
                          "fetch_kib": statistics.median(f[name]), "write_kib": statistics.median(w[name])}
        total += per_launch * per_step
    rec = {"workload": workload, "sources_sha256": sources_sha(), "fetch_scale": f_scale, "write_scale": w_scale,
           "bytes_per_step": total, "algorithmic_bytes_per_step": step_bytes(p), "kernels": kernels}
    json.dump(rec, open(traffic_path(workload), "w"), indent=1)
    print(json.dumps(rec, indent=1))


def kernel_short_name(full: str) -> str:
    """'void dsa::(anonymous namespace)::topk_attn_kernel<1>(dsa::TopkArgs, ...)' -> 'topk_attn_kernel<1>'."""
    s = full.replace("(anonymous namespace)::", "")
    return s.split("(")[0].split("::")[-1]


def kernel_breakdown(fn, n: int):
    """Per-kernel average device time over n calls of fn(i), from torch's
    profiler (on ROCm it traces every kernel the process launches, this
    library's included): {short name: {avg_us, launches_per_call}}."""
    import torch
    from torch.profiler import profile, ProfilerActivity
    with profile(activities=[ProfilerActivity.CUDA]) as prof:
        for i in range(n):
            fn(i)
        torch.cuda.synchronize()
    out = {}
    for e in prof.key_averages():
        if "dsa::" not in e.key or e.count == 0:
            continue
        dt = getattr(e, "device_time_total", 0.0) or getattr(e, "cuda_time_total", 0.0)
        short = kernel_short_name(e.key)
        out[short] = {"avg_us": dt / e.count, "launches_per_call": e.count / n}
    return out


def copy_gbps(nbytes: int = 1 << 30, reps: int = 20) -> float:
    """Device-to-device copy of nbytes on this GPU: (read + written) bytes per second."""
    import torch
    src = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        dst.copy_(src)
    end.record()
    torch.cuda.synchronize()
    secs = start.elapsed_time(end) * 1e-3 / reps
    del src, dst
    return 2 * nbytes / secs / 1e9


def read_probe_gbps(dsa, nbytes: int, steps: int):
    """The library's plain streaming read (dsa_read_probe) of nbytes, timed
    like the indexer: back-to-back launches over enough copies that the
    256 MB MALL cannot serve a repeat. Returns (GB/s, us per launch)."""
    import torch
    nb = (nbytes + 15) // 16 * 16
    copies = max(2, -(-(1200 << 20) // nb))
    bufs = [torch.ones(nb // 4, dtype=torch.float32, device="cuda") for _ in range(copies)]
    out = torch.empty(dsa.lib.dsa_read_probe_blocks(), dtype=torch.float32, device="cuda")
    fn = lambda i: dsa.dsa_read_probe(bufs[i], out=out)
    for i in range(2 * copies):
        fn(i % copies)
    us = timed_steps(fn, max(steps, 2 * copies), copies) * 1e3
    del bufs
    return nb / (us * 1e-6) / 1e9, us


def cpu_baseline(p, budget_s: float):
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    rows = 0
    t0 = time.perf_counter()
    while True:
        # decode: the rows in turn; prefill: positions spread over the sequence
        r = rows % p.R if p.is_decode() else (rows * 2654435761) % p.R
        O.dsa_forward(p, rows=[r])
        rows += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    dt = time.perf_counter() - t0
    what = (f"decode rows of the same workload (full indexer over {int(p.seq_len[0])} keys" if p.is_decode()
            else f"query rows at spread positions of the same {int(p.R)}-token prefill (causal indexer")
    # the same oracle on one thread, over a shorter sample
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            n1, t1 = 0, time.perf_counter()
            while True:
                r = n1 % p.R if p.is_decode() else (n1 * 2654435761) % p.R
                O.dsa_forward(p, rows=[r])
                n1 += 1
                if time.perf_counter() - t1 >= budget_s / 4:
                    break
            single = n1 / (time.perf_counter() - t1)
    except Exception:
        pass
    model = None
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return {"value": rows / dt, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "cpu_model": model, "host_cpus": os.cpu_count(),
            "sample": f"{rows} {what}, stable-sort top-k, fp64 attention), {dt:.1f} s",
            "single_thread_value": single}


def context_parallel(dsa, p, d, call, steps, P=4):
    """Key-range shards rehearsed on one device: each shard scores its keys and
    selects locally; timed are the merges that would follow the exchanges
    (the selection from the shards' candidate lists, the output from their
    partial attentions)."""
    import torch
    max_len = int(p.seq_len.max())
    edges = [int(x) // 64 * 64 for x in torch.linspace(0, max_len, P + 1).tolist()]
    edges[-1] = max_len
    q_pos = d.q_pos.long()
    ps, pi, shards = [], [], []
    for lo, hi in zip(edges[:-1], edges[1:]):
        off = (d.row_off + lo).contiguous()
        qp = (torch.minimum(q_pos, torch.full_like(q_pos, hi - 1)) - lo).to(torch.int32).contiguous()
        sc = dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, off, qp, hi - lo, k_scale=d.k_scale)
        a, b = dsa.dsa_topk_pairs(sc, dsa.dsa_topk(sc, qp, hi - lo, p.k), lo)
        ps.append(a)
        pi.append(b)
        shards.append((lo, hi, off))
    ps, pi = torch.stack(ps).contiguous(), torch.stack(pi).contiguous()
    idx = dsa.dsa_topk_merge(ps, pi)
    o_parts, l_parts = [], []
    for lo, hi, off in shards:
        o, l = dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, off, dsa.dsa_shard_indices(idx, lo, hi), p.scale,
                                       latent_scale=d.latent_scale)
        o_parts.append(o)
        l_parts.append(l)
    o_parts, l_parts = torch.stack(o_parts).contiguous(), torch.stack(l_parts).contiguous()
    out, lse = dsa.dsa_attn_merge(o_parts, l_parts)
    _, _, idx1 = call()
    torch.cuda.synchronize()
    same = bool(torch.equal(idx, idx1))
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    res = {}
    for name, fn in (("topk_merge_us", lambda: dsa.dsa_topk_merge(ps, pi, idx_out=idx)),
                     ("attn_merge_us", lambda: dsa.dsa_attn_merge(o_parts, l_parts, out=out, lse=lse))):
        for _ in range(10):
            fn()
        torch.cuda.synchronize()
        start.record()
        for _ in range(steps):
            fn()
        end.record()
        torch.cuda.synchronize()
        res[name] = start.elapsed_time(end) * 1e3 / steps
    return {"shards": P, **res, "merged_equals_unsharded": same}


def prefill_flops(p):
    """Algorithmic FLOPs of the causal indexer (2*H_I*D_I per query-key pair,
    keys 0..t for query t) and of the sparse attention (2*H*(576+512) per
    selected key, min(k, t+1) keys for query t)."""
    T = int(p.R)
    pairs = T * (T + 1) // 2
    sel = sum(min(p.k, t + 1) for t in range(T))
    return pairs * 2 * p.H_I * p.D_I, sel * 2 * p.H * (576 + 512)


def prefill_run(args, p):
    """One step = the causal prefill pass of one sequence through the three
    entry points (indexer scores for every query, top-k, sparse attention);
    the roofline is the indexer's (one kernel, timed alone with HIP events),
    bound by the matrix cores."""
    import torch
    from sparse_attention_05_amd import dsa, inputs
    d = inputs.to_torch(p, "cuda")
    T = int(p.R)
    ld = (T + 3) // 4 * 4
    scores = torch.empty((T, ld), dtype=torch.float32, device="cuda")
    idx = torch.empty((T, p.k), dtype=torch.int32, device="cuda")
    out = torch.empty((T, p.H, 512), dtype=torch.float32, device="cuda")
    lse = torch.empty((T, p.H), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(dsa.dsa_workspace_size(dsa.DSA_ENTRY_SPARSE_MLA, T, 0, p.k, p.H), 256), dtype=torch.uint8,
                     device="cuda")

    def index():
        dsa.dsa_index_scores(d.q_idx, d.head_w, d.k_idx, d.row_off, d.q_pos, T, q_seq=d.q_seq, scores=scores)

    def topk():
        dsa.dsa_topk(scores, d.q_pos, T, p.k, idx_out=idx)

    def attend():
        dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, idx, p.scale, q_seq=d.q_seq, out=out, lse=lse,
                                workspace=ws)

    def step():
        index()
        topk()
        attend()

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def timed(fn, n):
        start.record()
        for _ in range(n):
            fn()
        end.record()
        torch.cuda.synchronize()
        return start.elapsed_time(end) * 1e3 / n

    # the clocks ramp over the first second or so of load: warm up for a
    # fixed time, then the W warmup steps
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < args.prewarm_s:
        step()
        torch.cuda.synchronize()
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ms_step = timed(step, args.steps) * 1e-3
    n = max(args.steps, 20)
    att_us = timed(attend, n)
    topk_us = timed(topk, n)
    # the indexer alone: warmed up on its own for 0.5 s first (the clocks
    # settle differently under it than under the attention-heavy passes)
    t_warm = time.perf_counter()
    while time.perf_counter() - t_warm < 0.5:
        index()
        torch.cuda.synchronize()
    idx_us = timed(index, max(args.steps, 50))
    fl_idx, fl_att = prefill_flops(p)
    achieved = fl_idx / (idx_us * 1e-6) / 1e12
    log(f"bench: prefill {ms_step:.3f} ms/pass, indexer {idx_us:.1f} us = {achieved:.0f} TFLOP/s, "
        f"top-k {topk_us:.1f} us, attention {att_us:.1f} us = {fl_att / (att_us * 1e-6) / 1e12:.0f} TFLOP/s")
    return {
        "metric": "DSA causal prefill tokens/s (one 8,192-token sequence, k=2048); indexer MFMA TFLOP/s vs peak",
        "value": T / (ms_step * 1e-3), "unit": "tokens/s", "ms_per_step": ms_step, "steps": args.steps,
        "config": {"workload": "prefill-8k", "batch": 1, "context": T, "k": p.k, "indexer_heads": p.H_I,
                   "indexer_dim": p.D_I, "mla_heads": p.H, "latent_dim": 576},
        "stages_us": {"index_scores": idx_us, "topk": topk_us, "sparse_mla": att_us},
        "attention_tflops": fl_att / (att_us * 1e-6) / 1e12,
        "attention_frac_of_bf16_peak": fl_att / (att_us * 1e-6) / 1e12 / MFMA_PEAK_TFS,
        "roofline": {"kernel": "index_scores_prefill", "bound": "mfma", "achieved": achieved, "peak": MFMA_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": achieved / MFMA_PEAK_TFS, "traffic": None,
                     "flops_per_launch": fl_idx, "us_per_launch": idx_us},
    }


def timed_steps(fn, n, n_sets):
    """ms per call over n back-to-back calls fn(i), bracketed by HIP events."""
    import torch
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(n):
        fn(i % n_sets)
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n


def step_roofline(p, workload, ms_step, kernels):
    """The decode step as one roofline: its algorithmic bytes over its
    measured time against the HBM peak; counted HBM bytes per step when a
    counter record of these sources exists; the kernels of the step with
    their share of its time, the dominant one named."""
    sb = step_bytes(p)
    achieved = sb / (ms_step * 1e-3) / 1e9
    rec = pmc_traffic(workload)
    ks = []
    for name, v in sorted(kernels.items(), key=lambda kv: -kv[1]["avg_us"] * kv[1]["launches_per_call"]):
        us = v["avg_us"] * v["launches_per_call"]
        ks.append({"kernel": name, "us_per_step": us, "share_of_step": us / (ms_step * 1e3),
                   "launches_per_step": v["launches_per_call"]})
    for k in ks:
        if k["kernel"].startswith("index_scores"):
            ib = indexer_bytes(p)
            k["algorithmic_bytes"] = ib
            k["frac_of_hbm_peak"] = ib / (k["us_per_step"] * 1e-6) / 1e9 / HBM_PEAK_GBS
        if rec and k["kernel"].split("<")[0] in rec["kernels"]:
            kr = rec["kernels"][k["kernel"].split("<")[0]]
            k["counted_hbm_bytes"] = kr["bytes_per_launch"] * kr["launches_per_step"]
    return {"kernel": "decode step (all kernels, one stream)", "bound": "hbm", "achieved": achieved,
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
            "traffic": rec["bytes_per_step"] if rec else None, "bytes_per_step": sb, "us_per_step": ms_step * 1e3,
            "dominant_kernel": ks[0]["kernel"] if ks else None, "kernels": ks}


def decode_run(args, name, full):
    """Times the fused decode step of one workload; full: also the extras of
    the headline line (percentiles, graph replay, index sharing, attention
    alone, context-parallel merges, the indexer's own roofline)."""
    import torch
    from sparse_attention_05_amd import dsa, inputs
    torch.cuda.set_device(0)
    log(f"bench: generating {name}")
    p = inputs.workload(name, seed=0)
    max_len = int(p.seq_len.max())
    sb = step_bytes(p)
    n_sets = (args.sets if full and args.sets else 0) or max(2, math.ceil(2 * MALL_BYTES / sb))
    base = inputs.to_torch(p, "cuda")
    sets = [base] + [type(base)(**{k: (v.clone() if v is not None else None) for k, v in vars(base).items()})
                     for _ in range(n_sets - 1)]
    m = p.tokens_per_seq
    paged = p.block_table is not None
    calls = [dsa.DecodeCall(d.q_idx, d.head_w, d.k_idx, d.q_abs, d.latent, d.row_off, d.seq_len, max_len,
                            p.k, p.scale, k_scale=d.k_scale, latent_scale=d.latent_scale, q_per_seq=m,
                            block_table=d.block_table, page_size=p.page_size)
             for d in sets]
    log(f"bench: {n_sets} input sets of {sb / 1e6:.1f} MB algorithmic traffic per step")
    aws = torch.empty(max(dsa.dsa_workspace_size(dsa.DSA_ENTRY_SPARSE_MLA, p.R, 0, p.k, p.H), 256),
                      dtype=torch.uint8, device="cuda")
    outs = [(torch.empty_like(calls[0].out), torch.empty_like(calls[0].lse)) for _ in range(3)]

    def attn(i, layer=0, d=None, idx=None):
        d = d or sets[i % n_sets]
        dsa.dsa_sparse_mla_attn(d.q_abs, d.latent, d.row_off, calls[i % n_sets].idx if idx is None else idx,
                                p.scale, latent_scale=d.latent_scale, q_seq=d.q_seq if m > 1 else None,
                                block_table=d.block_table, page_size=p.page_size, out=outs[layer][0],
                                lse=outs[layer][1], workspace=aws)

    # determinism (not timed): two runs of set 0 with other steps between, and
    # the attention replayed over the recorded indices
    o0, l0, i0 = (x.clone() for x in calls[0]())
    for i in range(args.warmup):
        calls[i % n_sets]()
    torch.cuda.synchronize()
    o1, l1, i1 = calls[0]()
    attn(0, idx=i1)
    torch.cuda.synchronize()
    deterministic = bool(torch.equal(o0, o1) and torch.equal(l0, l1) and torch.equal(i0, i1))
    replay_equal = bool(torch.equal(outs[0][0], o1) and torch.equal(outs[0][1], l1))

    # ---- timed region: K fused decode steps ---------------------------------------------
    t0 = time.perf_counter()
    ms_step = timed_steps(lambda i: calls[i](), args.steps, n_sets)
    wall = time.perf_counter() - t0
    tok_s = p.R / (ms_step * 1e-3)
    log(f"bench: {name}: {ms_step * 1e3:.2f} us/step, {tok_s:,.0f} tokens/s (wall {wall:.3f} s)")

    try:
        kernels = kernel_breakdown(lambda i: calls[i % n_sets](), 20)
    except Exception as e:  # the profiler is diagnostic only
        log(f"bench: kernel breakdown unavailable: {e}")
        kernels = {}
    roof = step_roofline(p, name, ms_step, kernels)
    log(f"bench: {name}: step {roof['achieved']:,.0f} GB/s algorithmic = {roof['frac']:.3f} of HBM peak; "
        + ", ".join(f"{k['kernel'].split('<')[0]} {k['us_per_step']:.2f} us" for k in roof["kernels"]))
    res = {"workload": name, "ms_per_step": ms_step, "tokens_per_s": tok_s, "deterministic": deterministic,
           "replay_equal_fused": replay_equal, "step_algorithmic_bytes": sb, "step_hbm_gbps": roof["achieved"],
           "input_sets": n_sets, "roofline": roof,
           "config": {"workload": name, "batch": p.B, "context": max_len, "k": p.k, "indexer_heads": p.H_I,
                      "indexer_dim": p.D_I, "indexer_keys": p.key_dtype, "mla_heads": p.H, "latent_dim": 576,
                      "latent": p.kv_dtype, "tokens_per_seq": m, "page_size": p.page_size or None,
                      "input_sets": n_sets}}
    # ---- the indexer alone: K back-to-back launches of the step's first kernel -----------
    res["indexer_roofline"] = None
    if not paged:
        scores = [torch.empty((p.R, (max_len + 3) // 4 * 4), dtype=torch.float32, device="cuda") for _ in sets]

        def index(i):
            d = sets[i]
            dsa.dsa_index_scores_decode(d.q_idx, d.head_w, d.k_idx, d.row_off, d.seq_len, max_len, q_per_seq=m,
                                        k_scale=d.k_scale, scores=scores[i])

        # warmed up on its own for 0.5 s first, as the prefill indexer
        t_warm, i = time.perf_counter(), 0
        while time.perf_counter() - t_warm < 0.5:
            index(i % n_sets)
            i += 1
            if i % 50 == 0:
                torch.cuda.synchronize()
        idx_us = timed_steps(index, args.steps, n_sets) * 1e3
        ib = indexer_bytes(p)
        achieved = ib / (idx_us * 1e-6) / 1e9
        idx_tflops = 2.0 * p.H_I * p.D_I * sum(int(x) + 1 for x in p.q_pos.astype(int)) / (idx_us * 1e-6) / 1e12
        log(f"bench: indexer {idx_us:.2f} us/launch, {achieved:,.0f} GB/s algorithmic, {idx_tflops:.0f} TFLOP/s")
        copy = copy_gbps()
        log(f"bench: device copy {copy:,.0f} GB/s (read + write)")
        read_gbs, read_us = read_probe_gbps(dsa, ib, args.steps)
        log(f"bench: plain read of the indexer's {ib / 1e6:.1f} MB {read_us:.2f} us/launch = {read_gbs:,.0f} GB/s "
            f"(indexer at {achieved / read_gbs:.2f} of it)")
        rec = pmc_traffic(name)
        kr = rec["kernels"].get("index_scores_kernel") if rec else None
        res["indexer_roofline"] = {
            "kernel": "index_scores", "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": kr["bytes_per_launch"] if kr else None,
            "bytes_per_launch": ib, "us_per_launch": idx_us, "tflops": idx_tflops, "copy_gbps_measured": copy,
            "frac_of_copy": achieved / copy, "read_gbps_measured": read_gbs, "read_us_per_launch": read_us,
            "frac_of_read": achieved / read_gbs}
    if not full:
        del calls, sets, base, aws, outs
        torch.cuda.empty_cache()
        return p, res

    # ---- per-step percentiles: an event after every step of a second timed run -------------
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record()
    for i in range(args.steps):
        calls[i % n_sets]()
        evs[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps))
    res["step_us_percentiles"] = {"p10": per[len(per) // 10], "median": per[len(per) // 2],
                                  "p90": per[(9 * len(per)) // 10]}

    # ---- the same steps captured in a HIP graph (launch gaps vs kernel time) -------------
    res["graph_ms_per_step"], res["graph_replays_equal_eager"] = None, None
    try:
        ref = [tuple(x.clone() for x in c()) for c in calls]
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for c in calls:
                c()
        reps = max(1, args.steps // n_sets)
        g.replay()
        torch.cuda.synchronize()
        same = all(torch.equal(a, b) for c, r in zip(calls, ref) for a, b in zip((c.out, c.lse, c.idx), r))
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            g.replay()
        end.record()
        torch.cuda.synchronize()
        res["graph_ms_per_step"] = start.elapsed_time(end) / (reps * n_sets)
        g.replay()
        torch.cuda.synchronize()
        res["graph_replays_equal_eager"] = same and all(
            torch.equal(a, b) for c, r in zip(calls, ref) for a, b in zip((c.out, c.lse, c.idx), r))
        del g
        log(f"bench: graph-captured {res['graph_ms_per_step'] * 1e3:.2f} us/step "
            f"(replays equal to eager: {res['graph_replays_equal_eager']})")
    except Exception as e:  # capture unsupported here: report it, keep the eager numbers
        log(f"bench: graph capture failed: {e}")

    # ---- cross-layer index reuse: a block of 4 layers shares one selection -------------
    # Layer 0 runs the fused step (indexer, top-k, attention) and records its
    # indices; layers 1..3 run only the sparse attention over those indices,
    # each with its own queries and latent cache (another input set's).
    share_layers = 4

    def block(i):
        c = calls[i % n_sets]
        c()
        for l in range(1, share_layers):
            attn(i, layer=l - 1, d=sets[(i + l) % n_sets], idx=c.idx)

    for i in range(min(args.warmup, n_sets)):
        block(i)
    block_ms = timed_steps(block, args.steps, 10 ** 9)
    log(f"bench: index-shared block of {share_layers} layers {block_ms * 1e3:.2f} us "
        f"(vs {share_layers} fused steps {share_layers * ms_step * 1e3:.2f} us)")
    res["index_share"] = {"layers": share_layers, "ms_per_block": block_ms,
                          "tokens_per_s_per_block": p.R / (block_ms * 1e-3),
                          "speedup_vs_independent_layers": share_layers * ms_step / block_ms}

    # ---- the attention alone over recorded indices: K back-to-back launches --------------
    for i in range(min(args.warmup, n_sets)):
        attn(i)
    attn_us = timed_steps(attn, args.steps, n_sets) * 1e3
    ab = attention_bytes(p)
    log(f"bench: attention {attn_us:.2f} us/launch, {ab / (attn_us * 1e-6) / 1e9:,.0f} GB/s algorithmic")
    res["attention"] = {"us_per_launch": attn_us, "bytes_per_launch": ab, "gbps": ab / (attn_us * 1e-6) / 1e9}

    # ---- context parallelism rehearsed with 4 key-range shards: the merges ----------------
    res["context_parallel"] = None
    if m == 1 and not paged:
        cp = context_parallel(dsa, p, sets[0], calls[0], args.steps)
        log(f"bench: 4-shard top-k merge {cp['topk_merge_us']:.2f} us, output merge {cp['attn_merge_us']:.2f} us "
            f"(merged selection equals the unsharded one: {cp['merged_equals_unsharded']})")
        res["context_parallel"] = cp

    return p, res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode-32k")
    ap.add_argument("--sets", type=int, default=0, help="input copies cycled through (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--prewarm-s", type=float, default=1.5, help="prefill: seconds of untimed passes first")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", action="store_true", help="the named workload only (no other workloads)")
    ap.add_argument("--pmc-pass", action="store_true", help="run the counter workload (under rocprofv3 --pmc)")
    ap.add_argument("--ingest-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write the step's traffic record from two counter runs")
    args = ap.parse_args()
    if args.ingest_pmc:
        ingest_pmc(args.workload, *args.ingest_pmc)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not "
              "supported. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.pmc_pass:
        pmc_pass(args.workload)
        return
    import torch
    from sparse_attention_05_amd import inputs
    torch.cuda.set_device(0)

    if args.workload.startswith("prefill"):
        p = inputs.workload(args.workload, seed=0)
        rec = prefill_run(args, p)
        rec.update({"n_gpus": 1, "warmup": args.warmup, "higher_is_better": True, "scaling": "weak",
                    "vs_baseline": None, "dtype": "bf16", "data": "synthetic"})
        rec["cpu_baseline"] = None if args.no_cpu_baseline else cpu_baseline(p, args.cpu_seconds)
        print(json.dumps(rec), flush=True)
        return

    p, res = decode_run(args, args.workload, full=True)
    rec = {
        "metric": METRIC, "value": res["tokens_per_s"], "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": res["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if p.act_dtype == "bf16" else "f32", "data": "synthetic",
        "config": res["config"],
    }
    for k in ("step_us_percentiles", "step_hbm_gbps", "attention", "graph_ms_per_step", "graph_replays_equal_eager",
              "index_share", "context_parallel", "step_algorithmic_bytes", "deterministic", "replay_equal_fused"):
        rec[k] = res.get(k)
    rec["roofline"] = res["roofline"]
    rec["indexer_roofline"] = res["indexer_roofline"]

    # the other workloads of the survey, each with its own roofline (configs
    # of the long-context fp8 decode, the determinism / replay stress and the
    # causal prefill)
    if args.workload == "decode-32k" and not args.only:
        more = {}
        for w in ("decode-128k-fp8", "ties-64k"):
            _, r = decode_run(args, w, full=False)
            more[w] = r
        pp = inputs.workload("prefill-8k", seed=0)
        more["prefill-8k"] = prefill_run(args, pp)
        del pp
        torch.cuda.empty_cache()
        rec["workloads"] = more

    rec["cpu_baseline"] = None
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle")
        rec["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
