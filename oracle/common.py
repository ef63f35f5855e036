"""Batch expansion, validation and mean-pooled embedding lookup (oracle side).

Batch layout (shared with the boundary; int32 arrays):

* ``cand_offsets[R+1]`` — request ``r`` owns candidates
  ``cand_offsets[r] .. cand_offsets[r+1]-1``.  One request is one user plus
  its candidate items (CTR article, section 一; CVR article, section 3.4.5).
* ``bag_offsets[total_bags+1]`` and ``ids`` — multi-hot bags, feature-major
  in spec order.  A user- or context-side feature has one bag per request, an
  item-side feature one bag per candidate, so user features are batched per
  user and item features per item, linked by the request (CVR article,
  section 3.4.5).  Offsets are passed as data, not baked into the model (CVR
  article, section 3.3).
"""
import numpy as np


class OracleInputError(ValueError):
    """Malformed batch: the oracle refuses what the boundary reports as an error."""


def _as_i64(a, name):
    if a is None:
        raise OracleInputError(f"{name} is missing")
    a = np.asarray(a)
    if a.dtype.kind not in "iu":
        raise OracleInputError(f"{name} must be integer")
    return a.astype(np.int64)


def expand(spec, batch):
    """Step A0: check the batch CSR and map every candidate to its request.

    Returns ``R``, ``n``, ``cand_req[n]`` (int32), per-feature bag counts and
    the index of each feature's first bag.  Raises :class:`OracleInputError`
    for non-monotone offsets, offsets that do not end at ``len(ids)``, or ids
    outside their table.
    """
    co = _as_i64(batch["cand_offsets"], "cand_offsets")
    if co.ndim != 1 or co.size < 2:
        raise OracleInputError("cand_offsets needs at least one request")
    if co[0] != 0 or np.any(np.diff(co) < 0):
        raise OracleInputError("cand_offsets must start at 0 and be non-decreasing")
    R = co.size - 1
    n = int(co[-1])
    cand_req = np.repeat(np.arange(R, dtype=np.int64), np.diff(co)).astype(np.int32)

    feats = spec["features"]
    nbags = [n if f["side"] == "item" else R for f in feats]
    base = np.zeros(len(feats) + 1, dtype=np.int64)
    base[1:] = np.cumsum(nbags)
    bo = _as_i64(batch["bag_offsets"], "bag_offsets")
    ids = _as_i64(batch["ids"], "ids")
    if bo.ndim != 1 or bo.size != base[-1] + 1:
        raise OracleInputError(f"bag_offsets must have {base[-1] + 1} entries")
    if bo[0] != 0 or np.any(np.diff(bo) < 0) or bo[-1] != ids.size:
        raise OracleInputError("bag_offsets must start at 0, be non-decreasing and end at len(ids)")
    for fi, f in enumerate(feats):
        seg = ids[bo[base[fi]]:bo[base[fi + 1]]]
        rows = spec["tables"][f["table"]]["rows"]
        if seg.size and (seg.min() < 0 or seg.max() >= rows):
            raise OracleInputError(f"feature {f['name']}: id outside table of {rows} rows")

    out = {"R": R, "n": n, "cand_offsets": co.astype(np.int32), "cand_req": cand_req,
           "nbags": nbags, "bag_base": base, "bag_offsets": bo, "ids": ids}
    if spec["model"] == "hyformer":
        so = _as_i64(batch.get("seq_offsets"), "seq_offsets")
        sid = _as_i64(batch.get("seq_ids"), "seq_ids")
        S = len(spec["seq"]["lengths"])
        ncol = len(spec["seq"]["columns"])
        if so.shape != (S, R + 1):
            raise OracleInputError(f"seq_offsets must be [{S}, {R + 1}]")
        if sid.ndim != 2 or sid.shape[1] != ncol:
            raise OracleInputError(f"seq_ids must be [positions, {ncol}]")
        if np.any(np.diff(so, axis=1) < 0) or so.min() < 0 or so.max() > sid.shape[0]:
            raise OracleInputError("seq_offsets must be non-decreasing and inside seq_ids")
        # the batch layout keeps sequences apart: sequence s ends before sequence s+1 begins,
        # so no position belongs to two sequences
        if np.any(np.diff(so.reshape(-1)) < 0):
            raise OracleInputError("sequences must not overlap: seq_offsets read as one list must be non-decreasing")
        for ci, col in enumerate(spec["seq"]["columns"]):
            rows = spec["tables"][col["table"]]["rows"]
            c = sid[:, ci]
            if c.size and (c.min() < 0 or c.max() >= rows):
                raise OracleInputError(f"sequence column {ci}: id outside table of {rows} rows")
        out["seq_offsets"] = so
        out["seq_ids"] = sid
    return out


def pool_bags(table, ids, bag_offsets, bags):
    """Step A1: mean pooling of multi-hot bags, in fp32.

    The CVR article (section 3.1, item 2) pools multi-valued sparse features
    with ``mean`` instead of TorchRec's default ``sum``; the CTR article
    (section 三) keeps embeddings in FP32.  The summation order is not given;
    the reading taken is: start from zero, add the rows in the bag's own order
    in fp32, then divide once by the bag length (one correctly rounded fp32
    division).  An empty bag pools to zero.

    ``table`` is anything indexable by an int array returning fp32 rows.
    Returns fp32 ``[len(bags), dim]``.
    """
    bags = np.asarray(bags, dtype=np.int64)
    start = np.asarray(bag_offsets, dtype=np.int64)[bags]
    lens = np.asarray(bag_offsets, dtype=np.int64)[bags + 1] - start
    dim = table.shape[1]
    acc = np.zeros((bags.size, dim), dtype=np.float32)
    ids = np.asarray(ids, dtype=np.int64)
    for j in range(int(lens.max()) if lens.size else 0):
        sel = np.nonzero(lens > j)[0]
        rows = np.asarray(table[ids[start[sel] + j]], dtype=np.float32)
        acc[sel] = acc[sel] + rows
    nz = lens > 0
    acc[nz] = acc[nz] / lens[nz].astype(np.float32)[:, None]
    return acc


def clamp(x, bound):
    """The +-bound clamp applied right after lookup (CTR article, section 三).

    Inclusive bounds, computed in fp32 (exact); NaN passes through unchanged.
    """
    b = np.float32(bound)
    return np.clip(np.asarray(x, dtype=np.float32), -b, b)


def candidate_inputs(spec, tables, ex, cands, rnd):
    """Steps A1-A2 / B1 for a set of candidates.

    For each candidate ``c`` (of request ``r``) the model input is the concat,
    over features in spec order, of the feature's pooled bag — the request's
    bag for user/context features, the candidate's own bag for item features —
    clamped to +-clamp and rounded to the dense network's type by ``rnd``.
    Taking the request's bag for every candidate is the user-side repeat the
    CVR article (section 3.4.5) applies just before the concat.

    Returns (inputs fp64 ``[len(cands), D]``, dict feature -> pooled fp32 of
    the bags used, in candidate order).
    """
    cands = np.asarray(cands, dtype=np.int64)
    req = ex["cand_req"][cands].astype(np.int64)
    cols, pooled = [], {}
    for fi, f in enumerate(spec["features"]):
        local = cands if f["side"] == "item" else req
        p = pool_bags(tables[f["table"]], ex["ids"], ex["bag_offsets"], ex["bag_base"][fi] + local)
        pooled[fi] = p
        cols.append(rnd(clamp(p, spec["clamp"]).astype(np.float64)))
    D = sum(spec["tables"][f["table"]]["dim"] for f in spec["features"])
    x = np.concatenate(cols, axis=1) if cols else np.zeros((cands.size, D))
    return x, pooled


def sigmoid(z):
    """Logistic function in fp64: 1 / (1 + exp(-z))."""
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def requests_to_candidates(ex, requests):
    """Global candidate indices of the given requests (all requests when None)."""
    if requests is None:
        return np.arange(ex["n"], dtype=np.int64)
    co = ex["cand_offsets"].astype(np.int64)
    parts = [np.arange(co[r], co[r + 1], dtype=np.int64) for r in requests]
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int64)
