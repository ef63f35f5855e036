"""Pins for the hot-row cache oracle (CTR article section 二: HBM tier over host memory, LRU)."""
import collections
import os

import numpy as np
import pytest

from oracle import cache as oc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "murmur3_fmix32.txt")


def test_fmix32_published_vectors():
    rows = [l.split() for l in open(GOLDEN) if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for seed, want in rows:
        assert oc.fmix32(int(seed, 16)) == int(want, 16)


def test_set_of_uses_the_hash():
    c = oc.HotRowCache(sets=1000, ways=2)
    assert c.set_of(1) == 0x514E28B7 % 1000
    assert c.set_of(0xFFFFFFFF) == 0x81F16F39 % 1000


def test_hand_example_one_set_two_ways():
    c = oc.HotRowCache(sets=1, ways=2)
    hit = c.batch([(0, 5), (1, 7), (2, 5)])          # all miss; only the earliest miss (row 5) enters
    assert not hit.any()
    assert c.counters == dict(lookups=3, hits=0, misses=3, admissions=1, evictions=0)
    assert c.tags[0].tolist() == [5, -1]
    hit = c.batch([(0, 7), (1, 5)])                   # 7 misses and enters the empty way; 5 hits
    assert hit.tolist() == [False, True]
    assert c.tags[0].tolist() == [5, 7] and c.stamps[0].tolist() == [2, 2]
    hit = c.batch([(0, 9)])                           # both ways last used in batch 2: lowest way goes
    assert c.tags[0].tolist() == [9, 7]
    assert c.counters == dict(lookups=6, hits=1, misses=5, admissions=3, evictions=1)
    c.batch([(0, 7)])                                 # 7 is now the most recent ...
    c.batch([(0, 11)])                                # ... so 9 (stamp 3) is evicted, not 7 (stamp 4)
    assert sorted(c.tags[0].tolist()) == [7, 11]


@pytest.mark.parametrize("ways,universe,seed", [(1, 4, 0), (3, 6, 1), (4, 12, 2), (8, 10, 3)])
def test_one_lookup_per_batch_is_textbook_lru(ways, universe, seed):
    """With one set and one lookup per batch, the policy is plain LRU of capacity ``ways``."""
    rng = np.random.default_rng(seed)
    c = oc.HotRowCache(sets=1, ways=ways)
    lru = collections.OrderedDict()
    for step, row in enumerate(rng.integers(0, universe, 400).tolist()):
        want_hit = row in lru
        if want_hit:
            lru.move_to_end(row)
        else:
            if len(lru) == ways:
                lru.popitem(last=False)
            lru[row] = True
        got = c.batch([(0, row)])[0]
        assert got == want_hit, step
        assert sorted(t for t in c.tags[0].tolist() if t >= 0) == sorted(lru)


def test_invariants_over_random_batches():
    rng = np.random.default_rng(7)
    c = oc.HotRowCache(sets=5, ways=3)
    for t in range(1, 40):
        rows = rng.integers(-2, 60, rng.integers(0, 30)).tolist()
        before = {k: v for k, v in c.counters.items()}
        lookups = list(enumerate(rows))
        sets_missed = {c.set_of(r) for r in rows if 0 <= r < 58 and not c.contains(r)}
        hit = c.batch(lookups, rows=58)
        d = {k: c.counters[k] - before[k] for k in oc.COUNTERS}
        valid = [r for r in rows if 0 <= r < 58]
        assert d["lookups"] == len(valid) and d["hits"] + d["misses"] == d["lookups"]
        assert d["hits"] == int(hit.sum())
        assert d["admissions"] == len(sets_missed) and d["evictions"] <= d["admissions"]
        for s in range(c.sets):
            held = [x for x in c.tags[s].tolist() if x >= 0]
            assert len(held) == len(set(held))                       # a row is held once
            assert all(c.set_of(x) == s for x in held)               # in its own set
        for i, r in enumerate(rows):                                 # every hit row stays, stamped t
            if hit[i]:
                assert c.contains(r)
        assert c.epoch == t


def test_earliest_miss_is_admitted_not_the_smallest_row():
    c = oc.HotRowCache(sets=1, ways=4)
    c.batch([(10, 3), (4, 8), (7, 1)])                # positions, not order of appearance, decide
    assert c.tags[0].tolist() == [8, -1, -1, -1]
