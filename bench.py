"""Throughput of the candidate-scoring forward pass on one MI355X.

Default workload: the page-2-shaped DLRM request batch (64 requests x 500
candidates, 18 fp32 tables of 4.97 GB, fp16 MLP 640 -> 5 x 1024 -> 1).  One
step = one cvr_score call over the whole batch (expand, gather-pool, every MLP
layer, output and sigmoid), inputs resident in HBM.  Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2] [--no-cpu-baseline]
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


def dense_flops_per_candidate(spec):
    """FLOPs of every Linear (2*K*N per candidate), as performed."""
    from cvr_ranking_model_amd import synth
    total = 0
    for name, shape in synth.weight_shapes(spec).items():
        if name.endswith(".weight"):
            total += 2 * shape[0] * shape[1]
    if spec["model"] == "hyformer":
        # the sequence encoders run once per position, not once per candidate
        L = sum(spec["seq"]["lengths"])
        per_pos = sum(2 * shape[0] * shape[1] for n, shape in synth.weight_shapes(spec).items()
                      if n.startswith("seq.") and n.endswith(".weight")) // len(spec["seq"]["lengths"])
        seq_total = sum(2 * shape[0] * shape[1] for n, shape in synth.weight_shapes(spec).items()
                        if n.startswith("seq.") and n.endswith(".weight"))
        total = total - seq_total + per_pos * L
    return total


def mlp_gemm_flops(spec, n):
    from cvr_ranking_model_amd import synth
    return sum(2 * n * s[0] * s[1] for k, s in synth.weight_shapes(spec).items()
               if k.startswith("mlp.") and k.endswith(".weight") and s[0] > 1)


def gather_bytes(spec, batch):
    """Algorithmic bytes of one gather-pool launch: rows once per id, ids and offsets read, fp16/bf16 out."""
    import numpy as np
    ex_lens = np.diff(batch["bag_offsets"].astype(np.int64))
    R = len(batch["cand_offsets"]) - 1
    n = int(batch["cand_offsets"][-1])
    rows = 0
    o = 0
    out = 0
    for f in spec["features"]:
        nb = n if f["side"] == "item" else R
        dim = spec["tables"][f["table"]]["dim"]
        rows += int(ex_lens[o:o + nb].sum()) * dim * 4
        out += nb * dim * 2
        o += nb
    return rows + 4 * len(batch["ids"]) + 4 * len(batch["bag_offsets"]) + out


def cpu_baseline(spec, variant, weights, budget_s=10.0):
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
    C = wl["candidates"]
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
    return {"value": n / dt, "unit": "candidates/s", "cores": int(threads), "kind": "oracle",
            "sample": f"{nreq} of {R} requests ({n} candidates) of the same workload, {dt:.1f} s, numpy fp64 dense",
            "seconds": round(dt, 2)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c5"])
    ap.add_argument("--variant", default="bench")
    ap.add_argument("--uniform-ids", action="store_true", help="cold control: uniform ids instead of Zipf")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (requests shard with no "
              "collective; see the design notes). Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from cvr_ranking_model_amd import synth
    from cvr_ranking_model_amd import cvr as cv

    spec = synth.load_spec(args.workload)
    print(f"[bench] workload {args.workload}: filling tables", file=sys.stderr, flush=True)
    tables = cv.device_tables(spec, args.variant)
    weights = synth.make_weights(spec, args.variant)
    model = cv.Model(spec, tables, weights)
    batch = synth.make_batch(spec, uniform_ids=args.uniform_ids)
    db = cv.DeviceBatch(batch)
    n = db.n_candidates
    out = torch.empty(n * model.n_tasks, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    print(f"[bench] {n} candidates per step; warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        model.score(db, out)
    assert model.sync_status() == cv.CVR_OK
    model.timing_begin(args.steps)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        model.score(db, out)
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    stages, calls = model.timing_end()
    assert model.sync_status() == cv.CVR_OK
    ms_step = dt * 1e3 / args.steps
    value = n * args.steps / dt

    # dominant kernel and its roofline
    dom = max(stages, key=lambda k: stages[k][0])
    gemm_ms, gemm_launches = stages.get("mlp_gemm", (0.0, 0))
    flops_step = mlp_gemm_flops(spec, n)
    roof = None
    if dom == "mlp_gemm" and gemm_launches:
        per_launch = flops_step * calls / gemm_launches
        avg_s = gemm_ms / gemm_launches / 1e3
        ach = per_launch / avg_s / 1e12
        roof = {"bound": "mfma", "kernel": "gemm_kernel (hidden Linear+ReLU layers)", "achieved": round(ach, 1),
                "peak": MFMA_PEAK_TFLOPS[spec["lowp"]], "unit": "TFLOP/s",
                "frac": round(ach / MFMA_PEAK_TFLOPS[spec["lowp"]], 4), "traffic": None,
                "per_launch_flops": per_launch, "avg_launch_us": round(avg_s * 1e6, 2)}
    gb = gather_bytes(spec, batch)
    g_ms, g_l = stages.get("gather_pool", (0.0, 1))
    g_avg = g_ms / max(g_l, 1) / 1e3
    gather = {"bound": "hbm", "achieved": round(gb / g_avg / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
              "frac": round(gb / g_avg / 1e9 / HBM_PEAK_GBS, 4), "per_launch_bytes": gb,
              "avg_launch_us": round(g_avg * 1e6, 2), "ids": "uniform" if args.uniform_ids else "zipf"}
    line = {
        "metric": "scored candidates/sec at 1 GPU",
        "value": round(value, 1),
        "unit": "candidates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec["lowp"],
        "data": f"synthetic ({args.variant} variant: seeded hash tables, Zipf ids, Glorot weights)",
        "config": {"workload": WORKLOAD_TEXT[args.workload], "candidates_per_step": n,
                   "requests_per_step": db.n_requests},
        "roofline": roof,
        "gather_roofline": gather,
        "stage_ms_per_step": {k: round(v[0] / calls, 4) for k, v in stages.items()},
        "dense_gflop_per_step": round(flops_step / 1e9, 2),
    }
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(spec, args.variant, weights)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
