"""Shared test fixtures: markers, tiny hand-built specs and array-backed tables."""
import copy
import json
import math
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f) if name.endswith(".json") else f.read()


def tiny_dlrm_spec(dims=(4, 4, 2, 2), sides=("user", "user", "item", "item"), hidden=(8, 8), rows=8,
                   bag_max=4, lowp="fp16"):
    tables = [{"name": f"t{i}", "rows": rows, "dim": d} for i, d in enumerate(dims)]
    feats = [{"name": f"f{i}", "table": i, "side": s, "bag_min": 1, "bag_max": bag_max, "ids": "zipf"}
             for i, s in enumerate(sides)]
    return {"name": "tiny", "model": "dlrm", "lowp": lowp, "clamp": 10.0, "tables": tables, "features": feats,
            "mlp_hidden": list(hidden),
            "workload": {"requests": 3, "candidates": 4, "seed": 7, "zipf_a": 1.05, "cold_frac": 0.0}}


def tiny_cvr_spec(d=16, n_tokens=13, heads=16, layers=1, lens=(3, 5, 4), rows=16, e_dims=(8, 8, 8, 8),
                  sides=("user", "item", "item", "context"), seq_dims=(8, 4, 2, 2), hidden=8, mixer_hidden=8,
                  experts=3, expert_dim=8, tasks=2, head_hidden=4, lowp="bf16", tau=None, epnet_hidden=0):
    assert sum(seq_dims) == d
    nf = len(e_dims)
    tables = [{"name": f"ns{i}", "rows": rows, "dim": e} for i, e in enumerate(e_dims)]
    tables += [{"name": f"sq{i}", "rows": rows, "dim": sd} for i, sd in enumerate(seq_dims)]
    feats = [{"name": f"f{i}", "table": i, "side": sides[i], "bag_min": 1, "bag_max": 3, "ids": "zipf"}
             for i in range(nf)]
    cols = [{"table": nf + i, "ids": "uniform"} for i in range(len(seq_dims))]
    return {"name": "tinycvr", "model": "hyformer", "lowp": lowp, "clamp": 10.0, "tables": tables,
            "features": feats, "seq": {"columns": cols, "lengths": list(lens)},
            "d": d, "n_tokens": n_tokens, "n_layers": layers, "swiglu_hidden": hidden,
            "tau": float(tau if tau is not None else 2.0 * math.sqrt(d)), "mixer_heads": heads,
            "mixer_hidden": mixer_hidden, "n_experts": experts, "expert_dim": expert_dim, "n_tasks": tasks,
            "head_hidden": head_hidden, "epnet_hidden": epnet_hidden,
            "workload": {"requests": 3, "candidates": 2, "seed": 11, "zipf_a": 1.05, "cold_frac": 0.0}}


def array_tables(spec, seed=0, halfwidth=1.0, dyadic=False):
    """numpy tables for a tiny spec; ``dyadic`` draws multiples of 1/64 in [-2, 2] (exact sums)."""
    rng = np.random.default_rng(seed)
    out = []
    for t in spec["tables"]:
        if dyadic:
            out.append((rng.integers(-128, 129, (t["rows"], t["dim"])) / 64.0).astype(np.float32))
        else:
            out.append(rng.uniform(-halfwidth, halfwidth, (t["rows"], t["dim"])).astype(np.float32))
    return out


@pytest.fixture
def rng():
    return np.random.default_rng(1234)


def deepcopy(x):
    return copy.deepcopy(x)
