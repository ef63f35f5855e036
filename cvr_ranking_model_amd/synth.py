"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws inputs: embedding-table values, id bags, behaviour
sequences and dense weights.  It holds none of the scoring arithmetic, so the
CPU oracle and the GPU path can both consume what it produces without sharing
any of the method's code.

Recipe (every choice below is an input-recipe decision, not part of the model):

* Table values.  Element ``i = row * dim + col`` of table ``t`` is the
  ``(i+1)``-th output of a SplitMix64 generator (Steele, Lea & Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014) seeded with
  ``table_seed(workload_seed, t)``.  The top 24 bits ``k`` of that output give
  ``fp32((k - 2**23) * (2*halfwidth / 2**24))``, computed as one fp64 product
  and rounded to fp32: a uniform value in ``[-halfwidth, halfwidth)``.  The
  GPU fills tables with its own kernel from the same definition; this module
  regenerates only the rows a CPU computation touches, so a 27 GB table never
  has to exist on the host.
* Ids.  A bounded power law over ranks ``1..V`` with exponent ``a`` drawn by
  the continuous inverse CDF, then scattered over rows by the bijection
  ``row = (P*(rank-1) + Q) mod V`` (``P`` an odd prime not dividing ``V``), so
  hot rows are spread over the table.  With probability ``cold_frac`` an id is
  replaced by a uniform row.  Bag lengths are uniform integers in
  ``[bag_min, bag_max]``.
* Sequences.  Three behaviour sequences per request, each position holding
  (item id, action type, time bucket, side-info id) row indices.
* Dense weights.  Glorot-uniform ``U(+-gain*sqrt(6/(fan_in+fan_out)))`` as the
  iQIYI article's training setup uses for dense layers (section 3.1, item 1);
  biases zero for bench data, ``U(-0.1, 0.1)`` for stress data.

Data variants: ``bench`` (tables U(-0.05, 0.05), gain 1, zero biases),
``stress`` (tables U(-1, 1), biases U(-0.1, 0.1); DLRM weights gain 2; CVR
weights gain 0.8 except the sequence encoders and query layers at gain 3,
which makes the attention strongly peaked -- the largest weight about 100x the
uniform one -- while the scores spread to a standard deviation near 0.1)
``stress1`` (the stress draws with those CVR weights at gain 1 instead of
0.8: score standard deviation near 0.2) and ``clamp`` (tables U(-50, 50) so the
+-10 clamp binds, gain 1, biases U(-0.1, 0.1)).  With bench data every score sits within a few 1e-3 of 0.5, so
parity is also checked on the other two.
"""
from __future__ import annotations

import json
import math
import os
import zlib
from dataclasses import dataclass

import numpy as np

SPEC_DIR = os.path.join(os.path.dirname(os.path.abspath(__file__)), "specs")

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

# Odd prime coprime with every table size used here (all sizes are 2^a 5^b).
ID_SCATTER_PRIME = 2654435761

VARIANTS = {
    "bench": {"halfwidth": 0.05, "gain": 1.0, "bias": 0.0},
    "stress": {"halfwidth": 1.0, "gain": 2.0, "bias": 0.1, "hyformer_gain": 0.8, "hyformer_seq_gain": 3.0},
    # the same draws as "stress" with the CVR weights outside the sequence encoders and queries at
    # gain 1 (scores spread wider; kept beside "stress" as the harder CVR parity case)
    "stress1": {"halfwidth": 1.0, "gain": 2.0, "bias": 0.1, "hyformer_gain": 1.0, "hyformer_seq_gain": 3.0},
    "clamp": {"halfwidth": 50.0, "gain": 1.0, "bias": 0.1},
}


def load_spec(name_or_path: str) -> dict:
    """Load a config spec by short name (``c1`` .. ``c5``) or by file path."""
    path = name_or_path
    if not os.path.exists(path):
        path = os.path.join(SPEC_DIR, f"{name_or_path}.json")
    with open(path) as f:
        return json.load(f)


# ----------------------------------------------------------------------------
# SplitMix64 (Steele, Lea & Flood 2014)
# ----------------------------------------------------------------------------
def splitmix64_mix(z: np.ndarray) -> np.ndarray:
    """The SplitMix64 output function on uint64 values (wrapping arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_outputs(seed: int, index: np.ndarray) -> np.ndarray:
    """Outputs number ``index+1`` (``index`` 0-based) of SplitMix64 seeded with ``seed``."""
    idx = np.asarray(index, dtype=np.uint64)
    with np.errstate(over="ignore"):
        state = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + (idx + np.uint64(1)) * _GAMMA
    return splitmix64_mix(state)


def table_seed(workload_seed: int, table_index: int) -> int:
    """Per-table generator seed (a SplitMix64 mix of workload seed and table index)."""
    key = np.array([((workload_seed & 0xFFFFFFFFFFFF) << 16) | (table_index & 0xFFFF)], dtype=np.uint64)
    return int(splitmix64_mix(key)[0])


def value_step(halfwidth: float) -> float:
    """fp64 spacing of the 2**24 table value levels for ``U[-halfwidth, halfwidth)``."""
    return (2.0 * float(halfwidth)) / 16777216.0


def hash_values(seed: int, flat_index: np.ndarray, halfwidth: float) -> np.ndarray:
    """fp32 table values for flat element indices ``row*dim+col``."""
    x = splitmix64_outputs(seed, flat_index)
    k = (x >> np.uint64(40)).astype(np.int64) - (1 << 23)
    return (k.astype(np.float64) * value_step(halfwidth)).astype(np.float32)


@dataclass
class HashTable:
    """A table whose rows are regenerated on demand from the SplitMix64 recipe.

    ``table[rows]`` returns an fp32 array ``[len(rows), dim]``; the full table
    is never held in memory unless :meth:`materialize` is called.
    """

    rows: int
    dim: int
    seed: int
    halfwidth: float

    @property
    def shape(self):
        return (self.rows, self.dim)

    def __len__(self):
        return self.rows

    def __getitem__(self, idx) -> np.ndarray:
        idx = np.asarray(idx, dtype=np.int64)
        if idx.ndim == 0:
            return self[idx.reshape(1)][0]
        if idx.size and (idx.min() < 0 or idx.max() >= self.rows):
            raise IndexError("row index out of range")
        flat = idx.reshape(-1, 1) * self.dim + np.arange(self.dim, dtype=np.int64)
        return hash_values(self.seed, flat, self.halfwidth).reshape(idx.shape + (self.dim,))

    def materialize(self) -> np.ndarray:
        return self[np.arange(self.rows)]


def make_tables(spec: dict, variant: str = "bench") -> list:
    """Hash-defined tables for a spec (cheap: nothing is generated until rows are read)."""
    hw = VARIANTS[variant]["halfwidth"]
    seed = spec["workload"]["seed"]
    return [HashTable(t["rows"], t["dim"], table_seed(seed, i), hw) for i, t in enumerate(spec["tables"])]


def table_fill_params(spec: dict, variant: str = "bench") -> list:
    """(rows, dim, seed, halfwidth) per table, for a device-side fill of the same values."""
    return [(t.rows, t.dim, t.seed, t.halfwidth) for t in make_tables(spec, variant)]


# ----------------------------------------------------------------------------
# Ids, bags and sequences
# ----------------------------------------------------------------------------
def _rng(seed: int, *keys: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *keys])))


def zipf_rows(rng: np.random.Generator, V: int, a: float, size: int, table_index: int,
              cold_frac: float = 0.0) -> np.ndarray:
    """Bounded power-law row ids in ``[0, V)`` (see the module docstring)."""
    u = rng.random(size)
    if V == 1:
        rank = np.ones(size, dtype=np.int64)
    else:
        e = 1.0 - a
        x = ((float(V) ** e - 1.0) * u + 1.0) ** (1.0 / e)
        rank = np.clip(np.floor(x).astype(np.int64), 1, V)
    P = ID_SCATTER_PRIME % V if V > 1 else 0
    Q = (table_index * 40503 + 12345) % V
    rows = (np.int64(P) * (rank - 1) + Q) % V
    if cold_frac > 0.0:
        cold = rng.random(size) < cold_frac
        rows[cold] = rng.integers(0, V, int(cold.sum()))
    return rows.astype(np.int32)


def uniform_rows(rng: np.random.Generator, V: int, size: int) -> np.ndarray:
    return rng.integers(0, V, size).astype(np.int32)


def feature_bag_counts(spec: dict, cand_counts: np.ndarray) -> list:
    """Number of bags per feature: one per request (user/context side) or per candidate (item side)."""
    R = len(cand_counts)
    n = int(np.sum(cand_counts))
    return [n if f["side"] == "item" else R for f in spec["features"]]


def make_batch(spec: dict, requests: int | None = None, candidates: int | None = None,
               seed_offset: int = 0, ragged: bool = False, cand_counts=None,
               bag_min: int | None = None, seq_lengths=None, uniform_ids: bool = False) -> dict:
    """One batch in the boundary's CSR layout (all int32 numpy arrays).

    Layout:
      cand_offsets [R+1]: request r owns candidates cand_offsets[r]..cand_offsets[r+1].
      bag_offsets [total_bags+1]: bags ordered feature-major in spec order; a
        user/context feature has R bags (request order), an item feature has n
        bags (candidate order).
      ids [bag_offsets[-1]]: table-local row ids, bag after bag.
      seq_offsets [3, R+1] (CVR only): positions of group s, request r are
        seq_offsets[s, r]..seq_offsets[s, r+1]; groups are stored one after the
        other.
      seq_ids [P, 4] (CVR only): (item, action, time bucket, side) rows.

    ``ragged`` draws varying candidate counts, bag lengths from ``bag_min``
    (default 0, so empty bags occur) and sequence lengths in [0, L_s].
    ``uniform_ids`` replaces the power law by uniform rows (cold control).
    """
    wl = spec["workload"]
    R = int(requests if requests is not None else wl["requests"])
    C = int(candidates if candidates is not None else wl["candidates"])
    seed = int(wl["seed"]) + 7919 * int(seed_offset)
    a = float(wl["zipf_a"])
    cold = float(wl.get("cold_frac", 0.0))
    rng = _rng(seed, 1)
    if cand_counts is not None:
        cc = np.asarray(cand_counts, dtype=np.int64)
        R = len(cc)
    elif ragged:
        cc = rng.integers(0 if C > 1 else 1, C + 1, R)
    else:
        cc = np.full(R, C, dtype=np.int64)
    cand_offsets = np.zeros(R + 1, dtype=np.int64)
    cand_offsets[1:] = np.cumsum(cc)
    nbags = feature_bag_counts(spec, cc)

    lens_all, ids_all = [], []
    for fi, f in enumerate(spec["features"]):
        frng = _rng(seed, 100 + fi)
        lo = f["bag_min"] if bag_min is None else min(bag_min, f["bag_min"])
        if ragged and bag_min is None:
            lo = 0
        lens = frng.integers(lo, f["bag_max"] + 1, nbags[fi])
        t = f["table"]
        V = spec["tables"][t]["rows"]
        total = int(lens.sum())
        if uniform_ids or f.get("ids") == "uniform":
            ids = uniform_rows(frng, V, total)
        else:
            ids = zipf_rows(frng, V, a, total, t, cold)
        lens_all.append(lens)
        ids_all.append(ids)
    lens = np.concatenate(lens_all) if lens_all else np.zeros(0, np.int64)
    bag_offsets = np.zeros(len(lens) + 1, dtype=np.int64)
    bag_offsets[1:] = np.cumsum(lens)
    batch = {
        "cand_offsets": cand_offsets.astype(np.int32),
        "bag_offsets": bag_offsets.astype(np.int32),
        "ids": (np.concatenate(ids_all) if ids_all else np.zeros(0)).astype(np.int32),
        "seq_offsets": None,
        "seq_ids": None,
    }
    if spec["model"] == "hyformer":
        Ls = spec["seq"]["lengths"]
        srng = _rng(seed, 2)
        seq_off = np.zeros((len(Ls), R + 1), dtype=np.int64)
        base = 0
        per_group = []
        for s, L in enumerate(Ls):
            if seq_lengths is not None:
                sl = np.asarray(seq_lengths[s], dtype=np.int64)
            elif ragged:
                sl = srng.integers(0, L + 1, R)
            else:
                sl = np.full(R, L, dtype=np.int64)
            seq_off[s, 0] = base
            seq_off[s, 1:] = base + np.cumsum(sl)
            base = int(seq_off[s, -1])
            per_group.append(int(sl.sum()))
        P = base
        cols = []
        for ci, col in enumerate(spec["seq"]["columns"]):
            crng = _rng(seed, 200 + ci)
            t = col["table"]
            V = spec["tables"][t]["rows"]
            if uniform_ids or col["ids"] == "uniform":
                cols.append(uniform_rows(crng, V, P))
            else:
                cols.append(zipf_rows(crng, V, a, P, t, cold))
        batch["seq_offsets"] = seq_off.astype(np.int32)
        batch["seq_ids"] = (np.stack(cols, axis=1) if cols else np.zeros((0, 4))).astype(np.int32)
    return batch


# ----------------------------------------------------------------------------
# Dense weights
# ----------------------------------------------------------------------------
def weight_shapes(spec: dict) -> dict:
    """Ordered ``name -> shape`` of every dense parameter (Linear weights are [out, in])."""
    shapes = {}
    if spec["model"] == "dlrm":
        d_in = sum(spec["tables"][f["table"]]["dim"] for f in spec["features"])
        widths = list(spec["mlp_hidden"]) + [1]
        for i, w in enumerate(widths):
            shapes[f"mlp.{i}.weight"] = (w, d_in)
            shapes[f"mlp.{i}.bias"] = (w,)
            d_in = w
        return shapes
    d = spec["d"]
    N = spec["n_tokens"]
    S = len(spec["seq"]["lengths"])
    e_dim = sum(spec["tables"][f["table"]]["dim"] for f in spec["features"])
    hs = spec["swiglu_hidden"]
    T = N + S
    H = spec["mixer_heads"]
    mh = spec["mixer_hidden"]
    if spec.get("epnet_hidden"):
        d_dom = sum(spec["tables"][f["table"]]["dim"] for f in spec["features"] if f["side"] == "context")
        shapes["epnet.fc1.weight"] = (spec["epnet_hidden"], d_dom + e_dim)
        shapes["epnet.fc1.bias"] = (spec["epnet_hidden"],)
        shapes["epnet.fc2.weight"] = (e_dim, spec["epnet_hidden"])
        shapes["epnet.fc2.bias"] = (e_dim,)
    shapes["tok.weight"] = (N * d, e_dim)
    shapes["tok.bias"] = (N * d,)
    for s in range(S):
        shapes[f"seq.{s}.gate.weight"] = (hs, d)
        shapes[f"seq.{s}.gate.bias"] = (hs,)
        shapes[f"seq.{s}.up.weight"] = (hs, d)
        shapes[f"seq.{s}.up.bias"] = (hs,)
        shapes[f"seq.{s}.down.weight"] = (d, hs)
        shapes[f"seq.{s}.down.bias"] = (d,)
    for l in range(spec["n_layers"]):
        for s in range(S):
            shapes[f"layer.{l}.query.{s}.weight"] = (d, (N + 1) * d)
            shapes[f"layer.{l}.query.{s}.bias"] = (d,)
        for h in range(H):
            shapes[f"layer.{l}.mix.{h}.fc1.weight"] = (mh, T * d // H)
            shapes[f"layer.{l}.mix.{h}.fc1.bias"] = (mh,)
            shapes[f"layer.{l}.mix.{h}.fc2.weight"] = (T * d // H, mh)
            shapes[f"layer.{l}.mix.{h}.fc2.bias"] = (T * d // H,)
    z_dim = T * d
    for e in range(spec["n_experts"]):
        shapes[f"ple.expert.{e}.weight"] = (spec["expert_dim"], z_dim)
        shapes[f"ple.expert.{e}.bias"] = (spec["expert_dim"],)
    te = spec.get("ple_task_experts")
    for k in range(spec["n_tasks"]):
        g = spec["n_experts"] if te is None else len(te[k])
        shapes[f"ple.gate.{k}.weight"] = (g, z_dim)
        shapes[f"ple.gate.{k}.bias"] = (g,)
    for k in range(spec["n_tasks"]):
        shapes[f"head.{k}.fc1.weight"] = (spec["head_hidden"], spec["expert_dim"])
        shapes[f"head.{k}.fc1.bias"] = (spec["head_hidden"],)
        shapes[f"head.{k}.fc2.weight"] = (1, spec["head_hidden"])
        shapes[f"head.{k}.fc2.bias"] = (1,)
    return shapes


def make_weights(spec: dict, variant: str = "bench") -> dict:
    """Glorot-uniform weights (fp32 numpy), seeded per (config, parameter name)."""
    v = VARIANTS[variant]
    seed = int(spec["workload"]["seed"])
    out = {}
    for name, shape in weight_shapes(spec).items():
        rng = _rng(seed, 10_000 + (zlib.crc32(name.encode()) & 0x7FFFFFFF), 1 if variant in ("stress", "stress1") else 0)
        if name.endswith(".weight"):
            fan_out, fan_in = shape
            gain = v["gain"]
            if spec["model"] == "hyformer" and "hyformer_gain" in v:
                seq_like = name.startswith("seq.") or ".query." in name
                gain = v["hyformer_seq_gain"] if seq_like else v["hyformer_gain"]
            lim = gain * math.sqrt(6.0 / (fan_in + fan_out))
            out[name] = rng.uniform(-lim, lim, shape).astype(np.float32)
        else:
            b = v["bias"]
            out[name] = (rng.uniform(-b, b, shape) if b > 0 else np.zeros(shape)).astype(np.float32)
    return out
