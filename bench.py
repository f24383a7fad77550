"""Benchmark of one DSA decode step at 128k context on one MI355X.

    python bench.py [--steps K] [--warmup W] [--config 3] [--no-cpu-baseline]
    python bench.py --mode prefill [--steps K]      (workload 4, reported, not the headline)

A step is the whole hot path for one new token per sequence: the FP8 lightning indexer
over every cached token and the top-k (k = 2048) -- issued as the one call dsa_index_topk,
the same result as dsa_index_scores -> dsa_topk -- then dsa_sparse_mla_decode (MLA in MQA
mode over the kept rows, split-KV combine included).  Per-stage times come from an eager
pass that issues the three calls separately.  The default workload is
batch 8 x 131072 context (128 query heads, 576-wide bf16 latent rows, 64 x 128 e4m3
indexer), synthetic N(0,1)/sqrt(d) data (seed 1003).  Inputs are resident in HBM before
timing starts; `--copies` distinct copies of the caches are rotated step by step so the
256 MB Infinity Cache cannot serve a step from the previous one.  One HIP graph holds a
step on every copy in turn (as a decode loop captures several attention layers in one
graph) and is replayed; the library never allocates or synchronises, so capture is plain.
The same steps replayed one graph per step are reported beside it
(`single_step_graph_us`: each graph launch adds a gap of several microseconds).  A graph of
back-to-back indexer launches over the copies, with HIP events around its replays, gives
the indexer's launch duration for the roofline figure; an eager pass with events around
each call gives the per-stage breakdown (host gaps included).

`--mode prefill` times one causal prefill of T = 32768 tokens (workload 4) instead: the fused
index + top-k (blocked, so no T x T score matrix exists) and the sparse MLA; the indexer and
the top-k are also timed as the two separate calls over a full score matrix allocated for
that diagnostic only.  It reports the indexer (A2) against the FP8 MFMA peak and the sparse
MLA (A6) against the bf16 MFMA peak, both as algorithmic flops over each kernel's own
event-timed duration.

Prints one JSON line (rank 0, N = 1).  The library has no multi-GPU path.
"""
from __future__ import annotations

import argparse
import dataclasses
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0   # dense MFMA, MI355X datasheet
BF16_PEAK_TFLOPS = 2500.0
METRIC = "DSA decode tokens/s & us/step at 128k ctx (indexer+top-k+sparse MLA); % roofline"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--mode", default="decode", choices=["decode", "prefill"])
    p.add_argument("--config", type=int, default=3, choices=[2, 3, 5])
    p.add_argument("--copies", type=int, default=4)
    p.add_argument("--no-graph", action="store_true")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=12.0)
    return p.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.mode == "prefill":
        return prefill(args)
    import numpy as np
    import torch

    import datagen
    import long_context_sparse_06_amd as dsa
    from datagen.device import upload_decode
    from long_context_sparse_06_amd.step import DecodeStep

    dsa.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = datagen.CONFIGS[args.config]
    t0 = time.time()
    inp = datagen.make_config(args.config)
    log(f"[bench] generated {cfg['name']} in {time.time() - t0:.1f}s")
    d0 = upload_decode(inp, dev)
    sh = inp.shapes
    scale = 1.0 / math.sqrt(sh.Dqk)
    copies = [d0] + [dataclasses.replace(d0, keys=d0.keys.clone(), k_scale=d0.k_scale.clone(),
                                         kv=d0.kv.clone()) for _ in range(1, args.copies)]
    steps = [DecodeStep.from_inputs(c, sh.k, scale, sh.Dv) for c in copies]
    torch.cuda.synchronize()
    B = inp.B
    L = inp.lengths.astype(np.int64)

    # ---- algorithmic work (bytes the method must move), per step
    idx_bytes = int(L.sum()) * (sh.dI + 4) + B * (sh.HI * sh.dI + 4 * sh.HI + 4)
    kept = np.minimum(L, sh.k)
    mla_bytes = int(kept.sum()) * (2 * sh.Dqk + 4) + B * sh.H * (2 * sh.Dqk + 2 * sh.Dv + 4)
    table_bytes = 0 if inp.block_table is None else int(((L + inp.page_size - 1) // inp.page_size).sum()) * 4 * 2
    step_bytes = idx_bytes + mla_bytes + table_bytes
    roof_us = step_bytes / (HBM_PEAK_GBS * 1e3)

    stream = torch.cuda.current_stream()
    # ---- graphs: one per copy (a single step), and one holding a step on every copy in
    # turn, as a decode loop would capture several attention layers in one graph -- launching
    # a graph per step leaves a gap of several microseconds between graphs
    use_graph = not args.no_graph
    graphs = []
    multi = None
    if use_graph:
        for st in steps:  # warm the kernels once before capture
            st.run()
        torch.cuda.synchronize()
        for st in steps:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                st.run()
            graphs.append(g)
        multi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(multi):
            for st in steps:
                st.run()
        torch.cuda.synchronize()

    def one(i):
        if use_graph:
            graphs[i % len(steps)].replay()
        else:
            steps[i % len(steps)].run()

    def run_steps(n):
        # n whole steps, in copy order: full rounds through the multi-step graph, then singles
        if not use_graph:
            for i in range(n):
                one(i)
            return
        for _ in range(n // len(steps)):
            multi.replay()
        for i in range(n % len(steps)):
            one(i)

    run_steps(args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(args.steps)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # ---- the same steps replayed one graph per step (reported beside the headline)
    single_us = None
    if use_graph:
        for i in range(len(steps)):
            one(i)
        torch.cuda.synchronize()
        ts0 = time.perf_counter()
        for i in range(args.steps):
            one(i)
        torch.cuda.synchronize()
        single_us = (time.perf_counter() - ts0) * 1e6 / args.steps

    # ---- per-step spread: HIP events around single replays (outside the wall-clock loop)
    spread = None
    if use_graph:
        n_ev = min(args.steps, 100)
        sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n_ev)]
        for i, (a, b) in enumerate(sev):
            a.record(stream)
            one(i)
            b.record(stream)
        torch.cuda.synchronize()
        per = np.array([a.elapsed_time(b) for a, b in sev]) * 1e3
        spread = {"p10": float(np.percentile(per, 10)), "p50": float(np.median(per)),
                  "p90": float(np.percentile(per, 90)), "n": n_ev}

    # ---- eager pass with HIP events around each call: the step as run() issues it (the fused
    # index + top-k, then attention), then the indexer and the top-k as two separate calls
    # (over score rows the step itself never writes), for the per-stage breakdown
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(min(args.warmup, 5)):
        steps[i % len(steps)].run()
        steps[i % len(steps)].index()
    torch.cuda.synchronize()
    te0 = time.perf_counter()
    for i in range(args.steps):
        st = steps[i % len(steps)]
        e = ev[i]
        e[0].record(stream)
        st.index_topk()
        e[1].record(stream)
        st.attend()
        e[2].record(stream)
        st.index()
        e[3].record(stream)
        st.topk()
        e[4].record(stream)
    torch.cuda.synchronize()
    te1 = time.perf_counter()
    t_fused = np.array([e[0].elapsed_time(e[1]) for e in ev]) * 1e3
    t_mla = np.array([e[1].elapsed_time(e[2]) for e in ev]) * 1e3
    t_idx = np.array([e[2].elapsed_time(e[3]) for e in ev]) * 1e3
    t_topk = np.array([e[3].elapsed_time(e[4]) for e in ev]) * 1e3
    idx_us = float(t_idx.mean())
    if use_graph:
        # the indexer's launch duration without host gaps: a graph of back-to-back indexer
        # launches, one per cache copy in turn (caches as cold as in the step), HIP events
        # around its replays on this stream
        gi = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gi):
            for st in steps:
                st.index()
        gi.replay()
        torch.cuda.synchronize()
        n_rep = max(5, args.steps // len(steps))
        ia, ib = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ia.record(stream)
        for _ in range(n_rep):
            gi.replay()
        ib.record(stream)
        torch.cuda.synchronize()
        idx_us = ia.elapsed_time(ib) * 1e3 / (n_rep * len(steps))
        del gi
    achieved = idx_bytes / (idx_us * 1e3)  # GB/s

    # ---- quick self-check of the timed path against the first copy's eager result
    ok = True
    if use_graph:
        ref = [t.clone() for t in (steps[0].idx, steps[0].out)]
        for g in (graphs[0], multi):
            g.replay()
            torch.cuda.synchronize()
            ok = ok and torch.equal(ref[0], steps[0].idx) and torch.equal(ref[1].view(torch.int16),
                                                                          steps[0].out.view(torch.int16))

    # ---- top-k on a tie storm (every score equal) beside the same call on the step's scores
    st0 = steps[0]
    storm = torch.full_like(st0.scores, 0.5)
    tie = {}
    for name, buf in (("step_scores", st0.scores), ("tie_storm", storm)):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
        for a, b in evs:
            a.record(stream)
            dsa.dsa_topk(buf, st0.ld, st0.n_valid, st0.B, st0.k, st0.idx, *st0.topk_ws, stream)
            b.record(stream)
        torch.cuda.synchronize()
        tie[name + "_us"] = float(np.mean([a.elapsed_time(b) for a, b in evs[2:]]) * 1e3)
    del storm

    # ---- achievable HBM bandwidth on this GPU: a 1 GiB device-to-device copy (read + write)
    src_b = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst_b = torch.empty_like(src_b)
    dst_b.copy_(src_b)
    ca, cb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ca.record(stream)
    for _ in range(5):
        dst_b.copy_(src_b)
    cb.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 5 * 2 * (1 << 30) / (ca.elapsed_time(cb) * 1e6)

    # ---- achievable streaming-read rate on the step's own caches: dsa_read_probe (every load
    # one contiguous 1 KB, the indexer's residency) over each copy's key cache in turn, as a
    # graph of back-to-back launches, HIP events around its replays on this stream
    sink = torch.empty(dsa.dsa_read_probe_sink_words(), dtype=torch.int32, device=dev)
    key_bufs = [c.keys for c in copies]
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for kb_ in key_bufs:
            dsa.dsa_read_probe(kb_, sink)
    gr.replay()
    torch.cuda.synchronize()
    ra, rb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ra.record(stream)
    for _ in range(10):
        gr.replay()
    rb.record(stream)
    torch.cuda.synchronize()
    read_us = ra.elapsed_time(rb) * 1e3 / (10 * len(key_bufs))
    read_gbs = key_bufs[0].numel() * key_bufs[0].element_size() / (read_us * 1e3)
    del gr, sink
    del src_b, dst_b

    # ---- the fused index + top-k call beside the two separate calls: each as a graph of one
    # call per cache copy in turn (cold caches, no host gaps), HIP events around replays
    st0 = steps[0]
    fused_cmp = {}
    outs = {}
    for name, fn in (("fused_us", lambda st: st.index_topk()),
                     ("separate_us", lambda st: (st.index(), st.topk()))):
        gf = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gf):
            for st in steps:
                fn(st)
        gf.replay()
        torch.cuda.synchronize()
        outs[name] = st0.idx.clone()
        fa, fb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        fa.record(stream)
        for _ in range(10):
            gf.replay()
        fb.record(stream)
        torch.cuda.synchronize()
        fused_cmp[name] = fa.elapsed_time(fb) * 1e3 / (10 * len(steps))
        del gf
    fused_cmp["same_result"] = bool(torch.equal(outs["fused_us"], outs["separate_us"]))

    # ---- indexer-quality diagnostic on the same step's scores and kept sets (forward only)
    qw = dsa.dsa_indexer_quality_workspace_size(B, sh.H, st0.ld)
    qws = torch.empty(qw, dtype=torch.uint8, device=dev)
    qkl = torch.empty(B, device=dev)
    qrc = torch.empty(B, device=dev)
    qkr = torch.empty(B, device=dev)
    qargs = (st0.q, st0.kv, st0.scores, st0.ld, st0.idx, st0.row_seq, st0.row_pos, B, sh.H, sh.Dqk,
             sh.k, scale, qkl, qrc, qws, qw)
    dsa.dsa_indexer_quality(*qargs, kl_rev=qkr)
    q0, q1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    q0.record(stream)
    for _ in range(3):
        dsa.dsa_indexer_quality(*qargs, kl_rev=qkr)
    q1.record(stream)
    torch.cuda.synchronize()
    q_us = q0.elapsed_time(q1) * 1e3 / 3
    q_flops = float(L.sum()) * sh.H * sh.Dqk * 2
    quality = {"us": q_us, "logit_flops": q_flops, "TFLOP_s": q_flops / (q_us * 1e6),
               "kl_mean": float(qkl.mean()), "kl_rev_mean": float(qkr.mean()),
               "recall_mean": float(qrc.mean())}
    del qws

    # ---- cache append (the step before the indexer): one new token per sequence, written
    # into scratch caches of the same row widths (timed alone; not part of the step above)
    ap_k = torch.randn(B, sh.dI, device=dev) * 0.1
    ap_v = torch.randn(B, sh.Dqk, device=dev).to(torch.bfloat16)
    ap_keys = torch.empty(B, sh.dI, dtype=torch.uint8, device=dev)
    ap_ks = torch.empty(B, dtype=torch.float32, device=dev)
    ap_kv = torch.empty(B, sh.Dqk, dtype=torch.bfloat16, device=dev)
    ap_seq = torch.arange(B, dtype=torch.int32, device=dev)
    ap_pos = torch.zeros(B, dtype=torch.int32, device=dev)
    ap_args = (ap_k, ap_v, ap_seq, ap_pos, B, sh.dI, sh.Dqk, dsa.Cache(ap_keys, ap_ks, seq_stride=1),
               dsa.Cache(ap_kv, None, seq_stride=1))
    dsa.dsa_cache_append(*ap_args)
    torch.cuda.synchronize()
    # 20 calls captured in one graph, so the host's per-call cost does not pace the GPU
    ag = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ag):
        for _ in range(20):
            dsa.dsa_cache_append(*ap_args)
    ag.replay()
    torch.cuda.synchronize()
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(5):
        ag.replay()
    a1.record(stream)
    torch.cuda.synchronize()
    append_us = a0.elapsed_time(a1) * 1e3 / 100
    append_bytes = B * (sh.dI * 4 + sh.Dqk * 2 + 8) + B * (sh.dI + 4 + sh.Dqk * 2)

    # ---- CPU oracle on this host (bounded sample of the same workload)
    cpu = None
    if not args.no_cpu_baseline:
        from oracle import pipeline
        threads = os.cpu_count()
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            pass
        tc0 = time.perf_counter()
        done = 0
        while True:  # whole sequences, repeated until the time budget is used
            pipeline.decode_step(inp, scale, rows=[done % B])
            done += 1
            if time.perf_counter() - tc0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - tc0
        cpu = {"value": done / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
               "sample": f"{done} sequence-steps of this workload (each a full {int(L.max())}-token "
                         f"index scan, top-k and sparse MLA for one sequence), numpy fp64, {el:.1f} s"}

    # HBM traffic of the indexer from the committed rocprofv3 counter record; null when the
    # kernel source has changed since the counters were taken.
    traffic = None
    traffic_detail = None
    try:
        import hashlib
        rec = json.load(open(os.path.join(ROOT, "profiles", f"index_fp8_kernel_{cfg['name']}.traffic.json")))
        src = open(os.path.join(ROOT, rec["source"]), "rb").read()
        if hashlib.sha256(src).hexdigest() == rec["source_sha256"]:
            traffic = rec["fetch_bytes"] + rec["write_bytes"]  # HBM bytes per launch
            traffic_detail = {"fetch_bytes": rec["fetch_bytes"], "write_bytes": rec["write_bytes"],
                              "instance": rec.get("instance"), "vs_alg": traffic / idx_bytes}
    except (OSError, KeyError, ValueError):
        traffic = traffic_detail = None

    out = {
        "metric": METRIC,
        "value": B / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "us_per_step": ms_per_step * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "batch": B, "context": int(L.max()),
                   "context_mean": float(L.mean()), "top_k": sh.k, "heads": sh.H,
                   "latent": sh.Dqk, "value_dim": sh.Dv, "indexer_heads": sh.HI, "indexer_dim": sh.dI,
                   "paged": inp.block_table is not None, "cache_copies": len(steps),
                   "graph": use_graph, "steps_per_graph": len(steps) if use_graph else 0,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": "index_fp8_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "traffic_detail": traffic_detail,
                     "alg_bytes_per_launch": idx_bytes, "launch_us": idx_us},
        "step_roofline": {"alg_bytes": step_bytes, "roof_us": roof_us,
                          "frac": roof_us / (ms_per_step * 1e3),
                          "achievable_copy_GBs": copy_gbs,
                          "frac_of_achievable": step_bytes / (copy_gbs * 1e3) / (ms_per_step * 1e3),
                          "index_frac_of_achievable": achieved / copy_gbs,
                          "achievable_read_GBs": read_gbs, "read_probe_us": read_us,
                          "index_frac_of_achievable_read": achieved / read_gbs},
        "step_us_spread": spread,
        "index_topk_fused_vs_separate": fused_cmp,
        "indexer_quality": quality,
        "cache_append": {"us": append_us, "alg_bytes": append_bytes,
                         "GB_s": append_bytes / (append_us * 1e3), "bound": "latency"},
        "topk_diagnostic": tie,
        "single_step_graph_us": single_us,
        "breakdown_us": {"index_topk_fused": float(t_fused.mean()), "sparse_mla": float(t_mla.mean()),
                         "index_alone": float(t_idx.mean()), "topk_alone": float(t_topk.mean()),
                         "eager_step_and_separate_calls": (te1 - te0) * 1e6 / args.steps},
        "graph_replay_matches_eager": bool(ok),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def prefill(args):
    """One causal prefill of workload 4 (T = 32768), each stage timed with HIP events."""
    import numpy as np
    import torch

    import datagen
    import long_context_sparse_06_amd as dsa
    from datagen.device import upload_prefill
    from long_context_sparse_06_amd.step import Prefill

    dsa.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cfg = datagen.CONFIGS[4]
    t0 = time.time()
    inp = datagen.make_config(4)
    log(f"[bench] generated {cfg['name']} in {time.time() - t0:.1f}s")
    sh, T = inp.shapes, inp.T
    scale = 1.0 / math.sqrt(sh.Dqk)
    pf = Prefill.from_inputs(upload_prefill(inp, dev), sh.k, scale, sh.Dv)
    del inp
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    steps = max(1, min(args.steps, 5))
    for _ in range(max(1, min(args.warmup, 2))):
        pf.run()
    torch.cuda.synchronize()
    # The step as run(): the fused index + top-k (blocked; no T x T score buffer), then attention.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev:
        e[0].record(stream)
        pf.index_topk()
        e[1].record(stream)
        pf.attend()
        e[2].record(stream)
    torch.cuda.synchronize()
    ms = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev])
    t_fused, t_mla = (float(x) for x in ms.mean(axis=0))
    total = t_fused + t_mla
    fused_idx = pf.idx.clone()
    # The indexer and the top-k as the two separate calls over the full [T, T] score matrix
    # (allocated here for this diagnostic only), for the indexer's own kernel time.
    pf.index()
    pf.topk()
    torch.cuda.synchronize()
    same = bool(torch.equal(fused_idx, pf.idx))
    del fused_idx
    ev2 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for e in ev2:
        e[0].record(stream)
        pf.index()
        e[1].record(stream)
        pf.topk()
        e[2].record(stream)
    torch.cuda.synchronize()
    ms2 = np.array([[e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])] for e in ev2])
    t_idx, t_topk = (float(x) for x in ms2.mean(axis=0))
    score_matrix_bytes = pf.scores.numel() * 4
    pf._scores = None
    pf._topk_ws = None
    torch.cuda.empty_cache()
    n = np.arange(1, T + 1, dtype=np.float64)
    idx_flops = float(n.sum()) * sh.HI * sh.dI * 2
    kept = np.minimum(n, sh.k)
    mla_flops = float(kept.sum()) * sh.H * (sh.Dqk + sh.Dv) * 2
    # Short prefill (T = 2048, every earlier token kept): sparse gather vs the dense masked form.
    Ts = 2048
    sinp = datagen.make_prefill(Ts, sh, datagen.seed_for(4) + 1)
    sq = upload_prefill(sinp, dev)
    del sinp
    sidx = torch.full((Ts, sh.k), -1, dtype=torch.int32, device=dev)
    ar = torch.arange(sh.k, dtype=torch.int32, device=dev)
    sidx = torch.where(ar[None, :] <= torch.arange(Ts, device=dev)[:, None], ar[None, :], sidx).contiguous()
    so = torch.empty(Ts, sh.H, sh.Dv, dtype=torch.bfloat16, device=dev)
    sl = torch.empty(Ts, sh.H, dtype=torch.float32, device=dev)
    short = {}
    for name, fn in (("sparse", dsa.dsa_sparse_mla_prefill), ("masked", dsa.dsa_masked_mla_prefill)):
        fn(dsa.BF16, sq.q, sq.kv, sidx, Ts, sh.H, sh.Dqk, sh.Dv, sh.k, scale, so, sl)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            fn(dsa.BF16, sq.q, sq.kv, sidx, Ts, sh.H, sh.Dqk, sh.Dv, sh.k, scale, so, sl)
        e1.record(stream)
        torch.cuda.synchronize()
        short[name + "_ms"] = e0.elapsed_time(e1) / 5
    del sq, sidx, so, sl
    idx_tf = idx_flops / (t_idx * 1e-3) / 1e12
    mla_tf = mla_flops / (t_mla * 1e-3) / 1e12
    # Counter-derived MFMA busy % of the same kernels from the committed rocprofv3 record (one
    # counter pass of this command); null when the kernel source changed since it was taken.
    counters = {"sparse_mla": None, "index": None}
    try:
        import hashlib
        rec = json.load(open(os.path.join(ROOT, "profiles", "mfma_counters_prefill_t32768.json")))
        for key, r in (("sparse_mla", rec), ("index", rec["indexer"])):
            src = open(os.path.join(ROOT, r["source"]), "rb").read()
            if hashlib.sha256(src).hexdigest() == r["source_sha256"]:
                counters[key] = {"mfma_busy_pct": r["MfmaUtil_pct"], "waves_per_simd": r["waves_per_simd"],
                                 "lds_bank_conflict_pct": r["LdsBankConflict_pct"], "instance": r["instance"],
                                 "mfma_flops_counted": r["mfma_flops_counted"]}
    except (OSError, KeyError, ValueError):
        pass
    out = {
        "metric": "DSA prefill tokens/s at T=32768 (indexer+top-k+sparse MLA); % MFMA peak",
        "value": T / (total * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "ms_per_step": total,
        "higher_is_better": True,
        "vs_baseline": None,
        "dtype": "e4m3+bf16 (fp32 accumulate)",
        "data": "synthetic",
        "config": {"workload": cfg["name"], "tokens": T, "top_k": sh.k, "heads": sh.H, "latent": sh.Dqk,
                   "value_dim": sh.Dv, "indexer_heads": sh.HI, "indexer_dim": sh.dI},
        "stages_ms": {"index_topk_fused": t_fused, "sparse_mla": t_mla,
                      "index_alone": t_idx, "topk_alone": t_topk},
        "fused_same_as_two_calls": same,
        "index_topk_workspace_bytes": pf.fused_ws_bytes,
        "score_matrix_bytes_avoided": score_matrix_bytes,
        "short_prefill_t2048_attention": short,
        "roofline": {
            "index": {"bound": "mfma", "achieved": idx_tf, "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                      "frac": idx_tf / FP8_PEAK_TFLOPS, "alg_flops": idx_flops,
                      "counters": counters["index"]},
            "sparse_mla": {"bound": "mfma", "achieved": mla_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                           "frac": mla_tf / BF16_PEAK_TFLOPS, "alg_flops": mla_flops,
                           "counters": counters["sparse_mla"]},
        },
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
