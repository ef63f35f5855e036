"""Throughput of the candidate-scoring forward pass on one MI355X.

Default workload: the CVR model at its largest batch (C4: 4096 samples, 2 interaction layers,
behaviour sequences of 256/1024/2048 positions, bf16).  One step = one cvr_score call over the
whole batch (expand, gather-pool, tokenizer, SwiGLU sequence encoding and pools, per layer the
queries, attention and token mixer, PLE experts, gates and heads), inputs resident in HBM.
After it, unless --no-extra, the two DLRM workloads (C5: 27 GB of tables, 128k candidates;
C2: 64 requests x 500 candidates) are measured the same way and reported under "configs".
Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c4] [--no-extra] [--no-cpu-baseline]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"fp16": 2500.0, "bf16": 2500.0}

WORKLOAD_TEXT = {
    "c1": "c1: 1 request x 200 candidates, 4 tables 10k x 64, fp16 MLP 256-1024x3-1",
    "c2": "c2: 64 requests x (1 user + 500 candidates), 18 fp32 tables (user-ID 10M x 64, 8 x 1M x 32, "
          "item-ID 5M x 64, 8 x 100k x 32), Zipf 1.05 ids, fp16 MLP 640-1024x5-1",
    "c5": "c5: 256 requests x (1 user + 500 candidates), 27 GB fp32 tables (100M x 64, 1M x 32, 5M x 64, 100k x 32), "
          "Zipf 1.05 + 5% cold ids, fp16 MLP 192-1024x5-1",
    "c3": "c3: CVR model, 512 samples, 1 layer, sequences 64/256/512, bf16",
    "c4": "c4: CVR model, 4096 samples, 2 layers, sequences 256/1024/2048, bf16",
}


def dlrm_output_bytes(spec, n):
    """Bytes the DLRM output stage moves per step.  The library runs the MLP over slices of the
    candidates (128 MB per activation buffer); a slice whose last hidden layer runs on the wide
    GEMM kernel (at least 256 tiles of 256 x 128) hands the output stage per-row partials of
    64 columns instead of the activations (this mirrors the library's choice)."""
    maxw, N = max(spec["mlp_hidden"]), spec["mlp_hidden"][-1]
    rows = max(256, (128 << 20) // (maxw * 2) // 256 * 256)
    total = 0
    for r0 in range(0, n, rows):
        M = min(rows, n - r0)
        fused = N % 128 == 0 and N <= 1024 and -(-M // 256) * (N // 128) >= 256
        total += (M * (N // 64) * 4 if fused else M * N * 2) + M * 4
    return total


def stage_work(spec, batch, user_block=False):
    """Algorithmic work per step, per stage: ("flop"|"byte", amount).

    FLOPs count 2*M*N*K per Linear as performed.  Bytes count what the stage
    must move: table rows once per id occurrence, the ids and offsets it reads,
    and the low-precision outputs it writes (cache hits are not subtracted).
    """
    import numpy as np
    from cvr_ranking_model_amd import synth
    shapes = synth.weight_shapes(spec)
    R = len(batch["cand_offsets"]) - 1
    n = int(batch["cand_offsets"][-1])
    lens = np.diff(batch["bag_offsets"].astype(np.int64))
    rows, out, o = 0, 0, 0
    for f in spec["features"]:
        nb = n if f["side"] == "item" else R
        dim = spec["tables"][f["table"]]["dim"]
        rows += int(lens[o:o + nb].sum()) * dim * 4
        out += nb * dim * 2
        o += nb
    work = {"gather_pool": ("byte", rows + 4 * len(batch["ids"]) + 4 * len(batch["bag_offsets"]) + out)}
    lin = lambda name: 2 * shapes[name][0] * shapes[name][1]
    if spec["model"] == "dlrm":
        work["mlp_gemm"] = ("flop", n * sum(lin(k) for k in shapes if k.startswith("mlp.") and k.endswith(".weight")
                                          and shapes[k][0] > 1))
        if user_block:
            # performed: the first layer's request-side columns once per request, not per candidate
            d_req = sum(spec["tables"][f["table"]]["dim"] for f in spec["features"] if f["side"] != "item")
            w0 = spec["mlp_hidden"][0]
            work["mlp_gemm"] = ("flop", work["mlp_gemm"][1] - 2 * (n - R) * w0 * d_req)
        work["dlrm_output"] = ("byte", dlrm_output_bytes(spec, n))
        return work
    S = len(spec["seq"]["lengths"])
    P = int(batch["seq_ids"].shape[0])
    L = spec["n_layers"]
    d = spec["d"]
    per_pos = sum(lin(f"seq.0.{x}.weight") for x in ["gate", "up", "down"])
    work["tokenize_gemm"] = ("flop", n * lin("tok.weight"))
    if spec.get("epnet_hidden"):
        work["epnet"] = ("flop", n * (lin("epnet.fc1.weight") + lin("epnet.fc2.weight")))
    work["swiglu"] = ("flop", P * per_pos)
    work["swiglu_bytes"] = ("byte", P * (sum(spec["tables"][c["table"]]["dim"] for c in spec["seq"]["columns"]) * 4
                                         + 4 * len(spec["seq"]["columns"]) + d * 2))
    work["query_gemm"] = ("flop", L * n * sum(lin(f"layer.0.query.{q}.weight") for q in range(S)))
    # each candidate reads its request's encoded positions once per layer (bf16 rows)
    so = batch["seq_offsets"].astype(np.int64)
    cand_req = np.repeat(np.arange(R), np.diff(batch["cand_offsets"]))
    pos_per_cand = sum((so[q, cand_req + 1] - so[q, cand_req]).sum() for q in range(S))
    if n >= 16 * R:
        # requests of many candidates take the MFMA kernel, which reads a request's states once
        # per 32-candidate tile: a score and a weighted sum (2d FLOP each) per (candidate, position)
        work["attention"] = ("flop", L * int(pos_per_cand) * 4 * d)
    else:
        work["attention"] = ("byte", L * int(pos_per_cand) * d * 2)
    H = spec["mixer_heads"]
    work["mixer_gemm"] = ("flop", L * n * H * (lin("layer.0.mix.0.fc1.weight") + lin("layer.0.mix.0.fc2.weight")))
    # the fused mixer reads and writes the fp32 token matrix once per layer
    T = spec["n_tokens"] + S
    work["mixer_gemm_bytes"] = ("byte", L * n * T * d * 4 * 2)
    work["ple_gemm"] = ("flop", n * spec["n_experts"] * lin("ple.expert.0.weight"))
    work["head_gemm"] = ("flop", n * spec["n_tasks"] * lin("head.0.fc1.weight"))
    return work


def measured_traffic(workload, stage):
    """HBM bytes per launch of a stage's kernel from the committed byte-counter summaries.

    Each summary under profiles/ carries "traffic-json:" lines naming the workload, the stage,
    the kernel's source file and its sha256 at the time the counters were taken; a figure whose
    source has changed since is stale and is not reported.
    """
    import glob
    import hashlib
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(path):
            if not line.startswith("traffic-json:"):
                continue
            rec = json.loads(line[len("traffic-json:"):])
            if rec.get("workload", "c2") != workload or rec.get("stage") != stage or rec.get("bytes_per_launch") is None:
                continue
            src = os.path.join(ROOT, rec["source"])
            if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest() != rec["source_sha256"]:
                return None, os.path.basename(path) + " (stale: kernel source changed)"
            return int(rec["bytes_per_launch"]), os.path.basename(path)
    return None, None


def cpu_baseline(spec, variant, weights, budget_s=10.0):
    """The oracle timed on the host's cores on a bounded sample of the same workload."""
    import numpy as np
    import oracle
    from cvr_ranking_model_amd import synth
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    tables = synth.make_tables(spec, variant)
    wl = spec["workload"]
    R = wl["requests"]
    b1 = synth.make_batch(spec, requests=1, seed_offset=99)
    t0 = time.perf_counter()
    oracle.score(spec, tables, weights, b1)
    t1 = time.perf_counter() - t0
    nreq = int(max(1, min(R, budget_s / max(t1, 1e-3))))
    b = synth.make_batch(spec, requests=nreq, seed_offset=98)
    t0 = time.perf_counter()
    oracle.score(spec, tables, weights, b)
    dt = time.perf_counter() - t0
    n = int(b["cand_offsets"][-1])
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = None
    return {"value": n / dt, "unit": "candidates/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{nreq} of {R} requests ({n} candidates) of the same workload, {dt:.1f} s, numpy fp64 dense",
            "seconds": round(dt, 2), "host_cpus": os.cpu_count(), "affinity_cpus": affinity}


def percentiles(ms):
    import numpy as np
    a = np.asarray(ms, dtype=np.float64)
    return {"median": round(float(np.median(a)), 4), "p10": round(float(np.percentile(a, 10)), 4),
            "p90": round(float(np.percentile(a, 90)), 4)}


def run_config(workload, args, steps, warmup, batch=None, candidates=None, uniform_ids=False, cpu_budget=25.0,
               gather_control=True):
    """Measure one workload; returns the fields of its JSON entry."""
    import numpy as np
    import torch
    from cvr_ranking_model_amd import synth
    from cvr_ranking_model_amd import cvr as cv

    spec = synth.load_spec(workload)
    if args.ple_task_experts:
        spec["ple_task_experts"] = [[int(e) for e in t.split(",")] for t in args.ple_task_experts.split("/")]
    if args.epnet and spec["model"] == "hyformer":
        spec["epnet_hidden"] = args.epnet
    print(f"[bench] workload {workload}: filling tables", file=sys.stderr, flush=True)
    tables = cv.device_tables(spec, args.variant)
    cached = []
    if args.cache:
        if spec["model"] != "dlrm":
            sys.exit("--cache applies to the DLRM workloads")
        # the single-id ID tables go to host memory; the HBM budget is split by table size
        cached = sorted({f["table"] for f in spec["features"] if f["name"] in ("user_id", "item_id")})
        for t in cached:
            h = torch.empty(tables[t].shape, dtype=torch.float32, pin_memory=True)
            h.copy_(tables[t])
            tables[t] = h
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
    weights = synth.make_weights(spec, args.variant)
    # the model scores on a stream of its own, as a serving process would (graph capture needs a
    # created stream, and eager calls then run on the same one)
    torch.cuda.synchronize()
    model = cv.Model(spec, tables, weights, stream=torch.cuda.Stream())
    if args.user_block and spec["model"] == "dlrm":
        model.set_option(cv.CVR_OPT_DLRM_USER_BLOCK, 1)
    cache_cfg = {}
    if cached:
        total = sum(spec["tables"][t]["rows"] * spec["tables"][t]["dim"] * 4 for t in cached)
        budget = args.cache_gb * 1e9
        for t in cached:
            rows, dim = spec["tables"][t]["rows"], spec["tables"][t]["dim"]
            share = budget * rows * dim * 4 / total
            sets = max(1, int(min(rows, share / (dim * 4)) // args.cache_ways))
            model.attach_cache(t, sets, args.cache_ways)
            cache_cfg[spec["tables"][t]["name"]] = {"sets": sets, "ways": args.cache_ways,
                                                    "hbm_GB": round(sets * args.cache_ways * dim * 4 / 1e9, 3),
                                                    "table_GB": round(rows * dim * 4 / 1e9, 3)}
    nb = args.cache_batches if cached else 1
    batches = [synth.make_batch(spec, requests=batch, candidates=candidates, uniform_ids=uniform_ids,
                                seed_offset=i) for i in range(nb)]
    dbs = [cv.DeviceBatch(b) for b in batches]
    db = dbs[0]
    n = db.n_candidates
    out = torch.empty(n * model.n_tasks, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {workload}: {n} candidates per step; warmup {warmup}", file=sys.stderr, flush=True)
    for i in range(max(warmup, nb if cached else 0)):
        model.score(dbs[i % nb], out)
    assert model.sync_status() == cv.CVR_OK
    # Instrumented pass (every stage timed, not the timed region): the per-stage table and the
    # dominant stage.  An event-carrying dispatch costs a few microseconds more than a plain one,
    # so the timed region below carries events on the dominant stage's launches only.
    model.timing_begin(steps)
    for i in range(steps):
        model.score(dbs[i % nb], out)
    stages, calls = model.timing_end()
    dom = max(stages, key=lambda k: stages[k][0])
    stats0 = {t: model.cache_stats(t) for t in cached}
    graph_dt = None
    graph_info = None
    if args.graph:
        # replays rotate over four batches of the workload (other ids, other id counts): one
        # graph per batch bucket, captured on first use
        gb = [synth.make_batch(spec, requests=batch, candidates=candidates, uniform_ids=uniform_ids,
                               seed_offset=100 + i) for i in range(4)]
        gdbs = [cv.DeviceBatch(b) for b in gb]
        big = tuple(max(x) for x in zip(*[(d.n_requests, d.n_candidates, d.n_ids, d.n_positions) for d in gdbs]))
        gout = torch.empty(max(d.n_candidates for d in gdbs) * model.n_tasks, dtype=torch.float32, device="cuda")
        for i in range(max(4, warmup)):
            model.score_graph(gdbs[i % 4], gout, ws_sizes=big)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            model.score_graph(gdbs[i % 4], gout, ws_sizes=big)
        torch.cuda.synchronize()
        graph_dt = time.perf_counter() - t0
        assert model.sync_status() == cv.CVR_OK
        held, caps = model.graph_info()
        graph_info = {"batches": 4, "graphs_held": held, "captures": caps,
                      "candidates_per_step": sum(d.n_candidates for d in gdbs) / 4}
    print(f"[bench] {workload}: timed region, {steps} steps", file=sys.stderr, flush=True)
    model.timing_begin(steps, [dom])
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        model.score(dbs[i % nb], out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    live, live_calls = model.timing_end()
    assert live_calls == steps and dom in live
    for t in cached:
        st1, st0 = model.cache_stats(t), stats0[t]
        d = {k: st1[k] - st0[k] for k in st1}
        cache_cfg[spec["tables"][t]["name"]].update(d, hit_rate=round(d["hits"] / max(d["lookups"], 1), 4))
    assert model.sync_status() == cv.CVR_OK
    eager_dt = dt
    if graph_dt is not None:
        dt = graph_dt
    # Per-step spread: the same steps again, each between two events on the model's stream.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record(model.stream)
        if args.graph:
            model.score_graph(gdbs[i % 4], gout, ws_sizes=big)
        else:
            model.score(dbs[i % nb], out)
        ev[i][1].record(model.stream)
    torch.cuda.synchronize()
    step_ms = [a.elapsed_time(b) for a, b in ev]
    # End to end from host memory: each step also copies its packed request buffer (pinned
    # host memory) to the device on the model's stream before scoring it.  Reported beside
    # the HBM-resident rate, never as the value.
    h2d_bytes = sum(b.host.numel() * 4 for b in dbs) / len(dbs)
    with torch.cuda.stream(model.stream):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            b = dbs[i % nb]
            b.dev.copy_(b.host, non_blocking=True)
            model.score(b, out)
        torch.cuda.synchronize()
        h2d_dt = time.perf_counter() - t0
    assert model.sync_status() == cv.CVR_OK
    if args.calibrate_copy:
        # reads 256 MiB and writes 256 MiB once each: the reference for FETCH_SIZE / WRITE_SIZE
        src = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)
        torch.cuda.synchronize()
        del src, dst
    ms_step = dt * 1e3 / steps
    value = (graph_info["candidates_per_step"] if graph_info else n) * steps / dt

    # per-stage rooflines from the live event timings; the dominant stage gives "roofline"
    user_blk = bool(args.user_block and spec["model"] == "dlrm")
    works = [stage_work(spec, b, user_blk) for b in batches]
    work = {k: (v[0], sum(w[k][1] for w in works) / len(works)) for k, v in works[0].items()}
    peak_f = MFMA_PEAK_TFLOPS[spec["lowp"]]
    default_shape = batch is None and candidates is None and not uniform_ids and not args.cache
    table = {}
    for st, (ms, launches) in stages.items():
        entry = {"ms_per_step": round(ms / calls, 4), "launches_per_step": launches // max(calls, 1)}
        kind = work.get(st)
        if kind:
            avg_s = ms / launches / 1e3
            per_launch = kind[1] * calls / launches
            if kind[0] == "flop":
                ach = per_launch / avg_s / 1e12
                entry.update(bound="mfma", achieved=round(ach, 1), peak=peak_f, unit="TFLOP/s", frac=round(ach / peak_f, 4))
            else:
                ach = per_launch / avg_s / 1e9
                entry.update(bound="hbm", achieved=round(ach, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                             frac=round(ach / HBM_PEAK_GBS, 4))
            entry["per_launch"] = per_launch
            entry["avg_launch_us"] = round(avg_s * 1e6, 2)
            if st == "gather_pool":
                # algorithmic bytes (every row once per id) over time: what the lookup delivers;
                # the HBM rate proper comes from the byte counters when a record exists
                entry["achieved_is"] = "effective: algorithmic bytes / kernel time (cache hits not subtracted)"
                traffic, source = measured_traffic(workload, st) if default_shape else (None, None)
                if traffic:
                    hbm = traffic / avg_s / 1e9
                    entry["hbm_counter"] = {"bytes_per_launch": traffic, "GBs": round(hbm, 1),
                                            "frac": round(hbm / HBM_PEAK_GBS, 4), "source": source}
        if st + "_bytes" in work:
            b = work[st + "_bytes"][1] * calls / launches
            entry["hbm_GBs"] = round(b / (ms / launches / 1e3) / 1e9, 1)
        table[st] = entry
    # the dominant stage's figures come from the timed region's own events
    ms, launches = live[dom]
    d_entry = dict(table[dom])
    if "bound" in d_entry:
        avg_s = ms / launches / 1e3
        per_launch = work[dom][1] * live_calls / launches
        scale = 1e12 if work[dom][0] == "flop" else 1e9
        d_entry.update(achieved=round(per_launch / avg_s / scale, 1), per_launch=per_launch,
                       avg_launch_us=round(avg_s * 1e6, 2))
        d_entry["frac"] = round(d_entry["achieved"] / d_entry["peak"], 4)
    roof = None
    if "bound" in d_entry:
        traffic, source = measured_traffic(workload, dom) if default_shape else (None, None)
        roof = {"bound": d_entry["bound"], "kernel": dom, "achieved": d_entry["achieved"], "peak": d_entry["peak"],
                "unit": d_entry["unit"], "frac": d_entry["frac"], "traffic": traffic,
                "per_launch": d_entry["per_launch"], "avg_launch_us": d_entry["avg_launch_us"]}
        if source:
            roof["traffic_source"] = source
    res = {
        "value": round(value, 1),
        "unit": "candidates/s",
        "ms_per_step": round(ms_step, 4),
        "step_ms": percentiles(step_ms),
        "value_at_median_step": round(n / (percentiles(step_ms)["median"] / 1e3), 1),
        "dtype": spec["lowp"],
        "config": dict({"workload": WORKLOAD_TEXT[workload], "candidates_per_step": n,
                        "requests_per_step": db.n_requests},
                       **({"ple_task_experts": spec["ple_task_experts"]} if args.ple_task_experts else {}),
                       **({"epnet_hidden": spec["epnet_hidden"]} if spec.get("epnet_hidden") else {}),
                       **({"user_block": "first-layer request-side columns once per request"}
                          if args.user_block and spec["model"] == "dlrm" else {}),
                       **({"hot_row_cache": cache_cfg, "distinct_batches": nb} if cached else {})),
        "roofline": roof,
        "stages": table,
        "ids": "uniform" if uniform_ids else "zipf",
        "launch": "graph replay" if args.graph else "eager",
        "with_h2d": {"value": round(n * steps / h2d_dt, 1), "unit": "candidates/s",
                     "ms_per_step": round(h2d_dt * 1e3 / steps, 4), "h2d_bytes_per_step": int(h2d_bytes),
                     "what": "each step first copies its packed request buffer from pinned host memory"},
    }
    if args.graph:
        res["eager_ms_per_step"] = round(eager_dt * 1e3 / steps, 4)
        res["roofline_pass"] = "eager steps timed right after the graph replays (events on the roofline kernel)"
        res["graph"] = graph_info
    if gather_control and not uniform_ids and not cached and "gather_pool" in table:
        # cold control: the same workload with uniform ids (no hot rows for the caches to hold)
        ub = synth.make_batch(spec, requests=batch, candidates=candidates, uniform_ids=True, seed_offset=7)
        udb = cv.DeviceBatch(ub)
        uout = torch.empty(udb.n_candidates * model.n_tasks, dtype=torch.float32, device="cuda")
        for _ in range(2):
            model.score(udb, uout)
        model.timing_begin(steps, ["gather_pool"])
        for _ in range(steps):
            model.score(udb, uout)
        ust, ucalls = model.timing_end()
        assert model.sync_status() == cv.CVR_OK
        ums, ul = ust["gather_pool"]
        ubytes = stage_work(spec, ub)["gather_pool"][1] * ucalls / ul
        ach = ubytes / (ums / ul / 1e3) / 1e9
        res["gather_uniform_ids"] = {"achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                     "frac": round(ach / HBM_PEAK_GBS, 4), "per_launch": ubytes,
                                     "avg_launch_us": round(ums / ul * 1e3, 2),
                                     "what": "gather-pool of the same workload with uniform ids (cold control)"}
        del udb, uout
    if not args.no_cpu_baseline:
        print(f"[bench] {workload}: timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(spec, args.variant, weights, budget_s=cpu_budget)
    model.close()
    del model, tables, dbs, out
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def read_ceilings(reps=10):
    """Read-bandwidth ceilings of the chip for the two streaming access patterns of the path,
    measured with the library's probe kernels (cvr_probe_stream_read, cvr_probe_row_read):
      stream       one front-to-back read of 4 GiB (the cross-attention reads each encoded
                   state once per layer: 3.49 GB at 4096 samples);
      rows_<B>_<F> uniform random whole rows of B bytes from a table of F bytes (the embedding
                   gather: fp32 rows of 32 or 64 columns, tables of 1.28 GB and 25.6 GB), 8M
                   ids per launch for 128-byte rows and 4M for 256-byte rows.
    Bytes counted: the buffer, or rows plus the 4-byte ids.  Each shape is timed over `reps`
    launches (HIP events on the launching stream) at several grid sizes, with plain loads and
    with nontemporal ones; the best is the ceiling ("nt" in "best" marks the hinted form)."""
    import torch
    from cvr_ranking_model_amd import cvr as cv
    C = cv.C
    st = torch.cuda.current_stream()
    sink = torch.empty(1 << 20, dtype=torch.int32, device="cuda")

    def timed(launch):
        for _ in range(2):
            launch()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(st)
        for _ in range(reps):
            launch()
        ev[1].record(st)
        ev[1].synchronize()
        return ev[0].elapsed_time(ev[1]) / reps

    out = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    sweep = {}
    for nt in (0, 1):
        for blocks in [4096, 16384, 65536, 262144]:
            ms = timed(lambda: cv.cvr_probe_stream_read(C.c_void_p(buf.data_ptr()), nbytes, C.c_void_p(sink.data_ptr()),
                                                        blocks, C.c_void_p(st.cuda_stream), nontemporal=nt))
            sweep[f"{blocks}{'nt' if nt else ''}"] = round(nbytes / ms / 1e6, 1)
    best = max(sweep, key=sweep.get)
    out["stream"] = {"GB/s": sweep[best], "frac": round(sweep[best] / HBM_PEAK_GBS, 4), "bytes": nbytes,
                     "best": best, "sweep_GB/s": sweep}
    del buf
    torch.cuda.empty_cache()
    gen = torch.Generator(device="cuda")
    for foot in [1.28e9, 25.6e9]:
        for row_bytes in [128, 256]:
            n_rows = int(foot // row_bytes)
            n_ids = (8 << 20) if row_bytes == 128 else (4 << 20)
            table = torch.empty(n_rows * row_bytes, dtype=torch.uint8, device="cuda")
            table.fill_(1)
            gen.manual_seed(1234 + row_bytes)
            ids = torch.randint(0, n_rows, (n_ids,), generator=gen, device="cuda", dtype=torch.int32)
            moved = n_ids * (row_bytes + 4)
            sweep = {}
            for nt in (0, 1):
                for blocks in [2048, 8192, 32768]:
                    ms = timed(lambda: cv.cvr_probe_row_read(C.c_void_p(table.data_ptr()), n_rows, row_bytes,
                                                             C.c_void_p(ids.data_ptr()), n_ids,
                                                             C.c_void_p(sink.data_ptr()), blocks,
                                                             C.c_void_p(st.cuda_stream), nontemporal=nt))
                    sweep[f"{blocks}{'nt' if nt else ''}"] = round(moved / ms / 1e6, 1)
            best = max(sweep, key=sweep.get)
            out[f"rows_{row_bytes}B_{foot / 1e9:g}GB"] = {
                "GB/s": sweep[best], "frac": round(sweep[best] / HBM_PEAK_GBS, 4), "bytes": moved,
                "n_ids": n_ids, "best": best, "sweep_GB/s": sweep}
            del table, ids
            torch.cuda.empty_cache()
    torch.cuda.synchronize()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c3", "c4", "c5"])
    ap.add_argument("--batch", type=int, default=None, help="requests per step (CVR batch sweep)")
    ap.add_argument("--candidates", type=int, default=None,
                    help="candidates per request (CVR: 1 user + C candidates sharing its sequences)")
    ap.add_argument("--variant", default="bench")
    ap.add_argument("--cache", action="store_true",
                    help="DLRM: keep the ID tables in pinned host memory behind HBM hot-row caches "
                         "(CTR article section 二) and cycle through --cache-batches distinct batches")
    ap.add_argument("--cache-gb", type=float, default=5.0, help="HBM given to the caches (the article's L0: ~5 GB)")
    ap.add_argument("--cache-ways", type=int, default=8)
    ap.add_argument("--cache-batches", type=int, default=16)
    ap.add_argument("--ple-task-experts", default=None,
                    help="CVR: experts each task's gate mixes, tasks separated by '/', e.g. 0,2/1,2 "
                         "(PLE with one task-specific expert per task and a shared one)")
    ap.add_argument("--epnet", type=int, default=0,
                    help="CVR: EPNet gate hidden width (0: off), scaling the non-sequence embedding by the "
                         "context-side scenario features (CVR article section 3.2.1)")
    ap.add_argument("--user-block", action="store_true",
                    help="DLRM: the first Linear's request-side columns once per request (CVR_OPT_DLRM_USER_BLOCK)")
    ap.add_argument("--uniform-ids", action="store_true", help="cold control: uniform ids instead of Zipf")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="measure the named workload only (no further configs, no uniform-id gather control)")
    ap.add_argument("--extra", default="c5,c2", help="configs measured after the main one (default: c5,c2)")
    ap.add_argument("--graph", action="store_true",
                    help="time graph replays (cvr_score_graph); per-stage rooflines then come from an eager pass "
                         "of the same steps that follows")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed steps, run one plain 256 MiB fp32 copy kernel (torch.neg) so a "
                         "hardware-counter run can scale its byte counters against a known size")
    ap.add_argument("--ceilings", action="store_true",
                    help="measure only the read-bandwidth ceilings (stream and random rows) and print them")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library scores on one GPU (requests would shard across GPUs "
              "with no collective, each GPU holding its own copy of tables and weights). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.ceilings:
        print(json.dumps({"read_ceilings": read_ceilings()}), flush=True)
        return
    main_res = run_config(args.workload, args, args.steps, args.warmup, batch=args.batch,
                          candidates=args.candidates, uniform_ids=args.uniform_ids,
                          gather_control=not args.no_extra)
    line = {
        "metric": "scored candidates/sec at 1 GPU",
        "value": main_res.pop("value"),
        "unit": main_res.pop("unit"),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": main_res.pop("ms_per_step"),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": main_res.pop("dtype"),
        "data": f"synthetic ({args.variant} variant: seeded hash tables, Zipf ids, Glorot weights)",
        "config": main_res.pop("config"),
        "roofline": main_res.pop("roofline"),
    }
    cpu = main_res.pop("cpu_baseline", None)
    line.update(main_res)
    line["stages_pass"] = ("instrumented pass of the same steps before the timed region (events on every launch); "
                           "the timed region carries events on the roofline kernel's launches only; step_ms from a "
                           "further pass with one event pair around each step")
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if not args.no_extra and args.batch is None and args.candidates is None and not args.uniform_ids \
            and not args.cache and not args.graph:
        configs = {}
        for w in [x for x in args.extra.split(",") if x and x != args.workload]:
            configs[w] = run_config(w, args, min(args.steps, 20), min(args.warmup, 5), cpu_budget=10.0)
        line["configs"] = configs
        line["read_ceilings"] = ceil = read_ceilings()
        # the streaming kernels against the chip's measured read ceilings
        att = line.get("stages", {}).get("attention", {}).get("achieved")
        if att:
            line["attention_of_stream_ceiling"] = round(att / ceil["stream"]["GB/s"], 4)
        for w, r in [(args.workload, line)] + list(configs.items()):
            g = r.get("gather_uniform_ids", {}).get("achieved")
            if g:
                r["gather_uniform_of_row_ceiling"] = {
                    k: round(g / v["GB/s"], 4) for k, v in ceil.items() if k.startswith("rows_")}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
