"""The sequence layout contract of the batch (no GPU): sequences may not share positions.

The workspace holds n_positions / 32 + S * R chunk descriptors of 32 positions.  For segments
that are disjoint and inside [0, P) that always suffices: sum(ceil(l_i / 32)) <=
sum(floor(l_i / 32) + 1) <= floor(sum(l_i) / 32) + S * R <= floor(P / 32) + S * R.  Overlapping
segments can exceed it, so the layout forbids them (the device raises CVR_ERR_RANGE and caps its
chunk table at the allotted count), and the oracle refuses them as well.
"""
import numpy as np
import pytest

import oracle
from oracle.common import OracleInputError
from cvr_ranking_model_amd import synth


def chunks(so, P, chunk=32):
    total = 0
    for s in range(so.shape[0]):
        for r in range(so.shape[1] - 1):
            a = min(max(int(so[s, r]), 0), P)
            e = min(max(int(so[s, r + 1]), a), P)
            total += (e - a + chunk - 1) // chunk
    return total


@pytest.mark.parametrize("seed", range(20))
def test_disjoint_layouts_fit_the_allotted_chunks(seed):
    rng = np.random.default_rng(seed)
    S, R = 3, int(rng.integers(1, 40))
    lens = rng.integers(0, 100, (S, R))
    gaps = rng.integers(0, 5, (S, R))                 # unused positions between segments are allowed
    so = np.zeros((S, R + 1), np.int64)
    pos = 0
    for s in range(S):
        so[s, 0] = pos
        for r in range(R):
            pos += gaps[s, r]
            if r == 0:
                so[s, 0] = pos
            pos += lens[s, r]
            so[s, r + 1] = pos
    P = pos + int(rng.integers(0, 40))
    assert np.all(np.diff(so.reshape(-1)) >= 0)
    assert chunks(so, P) <= P // 32 + S * R


def test_overlapping_layouts_can_exceed_it_and_the_oracle_refuses_them():
    spec = synth.load_spec("c3")
    b = synth.make_batch(spec, requests=8)
    P = b["seq_ids"].shape[0]
    every = np.stack([np.r_[0, np.full(8, P)]] * 3).astype(np.int32)
    assert chunks(every, P) > P // 32 + 3 * 8
    oracle.expand(spec, b)                           # the synthetic layout keeps the contract
    for bad in [every, np.stack([b["seq_offsets"][0]] * 3)]:
        with pytest.raises(OracleInputError, match="overlap"):
            oracle.expand(spec, dict(b, seq_offsets=bad))
