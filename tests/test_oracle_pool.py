"""Pins for batch expansion (A0), mean pooling (A1) and clamp (A2) in the oracle."""
import numpy as np
import pytest

import oracle
from oracle.common import clamp, pool_bags, candidate_inputs, OracleInputError
from oracle.lowp import rounder
from conftest import tiny_dlrm_spec, array_tables


def _hand_batch():
    # 3 requests with 2, 0, 3 candidates; features: f0,f1 user (3 bags each), f2,f3 item (5 bags each)
    cand_offsets = [0, 2, 2, 5]
    lens = [1, 2, 0] + [3, 1, 1] + [1, 1, 2, 1, 1] + [2, 0, 1, 1, 4]
    bag_offsets = np.concatenate([[0], np.cumsum(lens)])
    rng = np.random.default_rng(3)
    ids = rng.integers(0, 8, bag_offsets[-1])
    return {"cand_offsets": np.array(cand_offsets, np.int32), "bag_offsets": bag_offsets.astype(np.int32),
            "ids": ids.astype(np.int32), "seq_offsets": None, "seq_ids": None}


def test_expand_by_hand():
    spec = tiny_dlrm_spec()
    ex = oracle.expand(spec, _hand_batch())
    assert ex["R"] == 3 and ex["n"] == 5
    assert ex["cand_req"].tolist() == [0, 0, 2, 2, 2]
    assert ex["nbags"] == [3, 3, 5, 5]
    assert ex["bag_base"].tolist() == [0, 3, 6, 11, 16]


@pytest.mark.parametrize("mutate, msg", [
    (lambda b: b.update(cand_offsets=np.array([0, 3, 2, 5], np.int32)), "non-decreasing"),
    (lambda b: b.update(cand_offsets=np.array([1, 2, 2, 5], np.int32)), "start at 0"),
    (lambda b: b.update(bag_offsets=b["bag_offsets"][:-1]), "entries"),
    (lambda b: b.update(ids=b["ids"][:-1]), "end at len"),
    (lambda b: b["ids"].__setitem__(0, 8), "outside"),
    (lambda b: b["ids"].__setitem__(0, -1), "outside"),
])
def test_expand_rejects_malformed(mutate, msg):
    spec = tiny_dlrm_spec()
    b = _hand_batch()
    mutate(b)
    with pytest.raises(OracleInputError, match=msg):
        oracle.expand(spec, b)


def _brute_pool(table, ids, offsets, bag):
    """Scalar fp32 loop: acc = 0; acc = fl32(acc + row) for each id; fl32(acc / len)."""
    lo, hi = int(offsets[bag]), int(offsets[bag + 1])
    out = []
    for c in range(table.shape[1]):
        acc = np.float32(0.0)
        for j in range(lo, hi):
            acc = np.float32(acc + np.float32(table[ids[j], c]))
        out.append(np.float32(acc / np.float32(hi - lo)) if hi > lo else np.float32(0.0))
    return np.array(out, dtype=np.float32)


def test_pool_matches_scalar_loop_and_fp64_bound(rng):
    table = rng.uniform(-1, 1, (8, 4)).astype(np.float32)
    lens = rng.integers(0, 17, 60)
    off = np.concatenate([[0], np.cumsum(lens)])
    ids = rng.integers(0, 8, off[-1])
    got = pool_bags(table, ids, off, np.arange(60))
    for b in range(60):
        assert np.array_equal(got[b], _brute_pool(table, ids, off, b)), b
        if lens[b]:
            exact = table[ids[off[b]:off[b + 1]]].astype(np.float64).sum(0) / lens[b]
            bound = lens[b] * 2.0 ** -24 * np.abs(table[ids[off[b]:off[b + 1]]]).astype(np.float64).sum(0) / lens[b]
            assert np.all(np.abs(got[b] - exact) <= bound + np.spacing(np.float32(np.abs(exact)))), b


def test_pool_special_cases(rng):
    table = (rng.integers(-100, 101, (8, 6)) / 64.0).astype(np.float32)   # dyadic: all partial sums exact
    for k in [1, 2, 3, 4, 5, 8, 16]:
        ids = np.full(k, 5)
        got = pool_bags(table, ids, np.array([0, k]), [0])
        assert np.array_equal(got[0], table[5]), k            # mean of identical rows is the row
    got = pool_bags(table, np.array([2]), np.array([0, 1]), [0])
    assert np.array_equal(got[0], table[2])                    # single id is the row itself
    got = pool_bags(table, np.zeros(0, np.int64), np.array([0, 0]), [0])
    assert np.array_equal(got[0], np.zeros(6, np.float32))     # empty bag pools to zero
    ids = np.array([1, 2, 3])
    got = pool_bags(table, ids, np.array([0, 3]), [0])
    assert np.array_equal(got[0], ((table[1].astype(np.float64) + table[2] + table[3]) / 3).astype(np.float32))


def test_pool_order_matters_only_by_rounding(rng):
    table = rng.uniform(-1, 1, (8, 32)).astype(np.float32)
    ids = rng.integers(0, 8, 12)
    a = pool_bags(table, ids, np.array([0, 12]), [0])[0]
    b = pool_bags(table, ids[::-1].copy(), np.array([0, 12]), [0])[0]
    assert np.all(np.abs(a - b) <= 12 * np.spacing(np.float32(12.0)) / 12 * 2)


def test_clamp_bounds():
    x = np.array([-1e9, -10.0, -9.99, 0.0, 3.5, 10.0, 10.0001, 1e30, np.nan], np.float32)
    y = clamp(x, 10.0)
    assert y[:8].tolist() == [-10.0, -10.0, np.float32(-9.99), 0.0, 3.5, 10.0, 10.0, 10.0]
    assert np.isnan(y[8])
    assert y.dtype == np.float32


def test_candidate_inputs_layout_and_repeat():
    spec = tiny_dlrm_spec()
    tables = array_tables(spec, dyadic=True)
    b = _hand_batch()
    ex = oracle.expand(spec, b)
    x, pooled = candidate_inputs(spec, tables, ex, np.arange(5), rounder("fp16"))
    assert x.shape == (5, 12)
    # candidate 3 belongs to request 2: user columns come from request 2's bags, item columns from bag 3
    for fi, (lo, hi) in enumerate([(0, 4), (4, 8), (8, 10), (10, 12)]):
        bag = ex["bag_base"][fi] + (3 if fi >= 2 else 2)
        want = pool_bags(tables[fi], ex["ids"], ex["bag_offsets"], [bag])[0]
        assert np.array_equal(x[3, lo:hi], want.astype(np.float16).astype(np.float64))
    # the user part is identical for every candidate of a request (the lazy repeat)
    assert np.array_equal(x[2, :8], x[4, :8])
    # request 0's bag for f1 has two ids, request 2's has zero (empty bag -> zeros)
    assert np.array_equal(x[2, 0:4], np.zeros(4))


def test_clamp_applies_before_cast():
    spec = tiny_dlrm_spec(dims=(2, 2), sides=("user", "item"))
    tables = [np.full((8, 2), 30.0, np.float32), np.full((8, 2), -10.0004, np.float32)]
    b = {"cand_offsets": np.array([0, 1], np.int32), "bag_offsets": np.array([0, 1, 2], np.int32),
         "ids": np.array([0, 0], np.int32)}
    ex = oracle.expand(spec, b)
    x, _ = candidate_inputs(spec, tables, ex, [0], rounder("fp16"))
    assert x[0].tolist() == [10.0, 10.0, -10.0, -10.0]
