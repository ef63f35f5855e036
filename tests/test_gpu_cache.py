"""GPU: HBM hot-row cache over host-resident tables (CTR article section 二) against the oracle.

Each scoring call is checked three ways: scores bit-identical to a model that reads the same
tables from device memory (a cache never changes a pooled value), the five counters equal to
the oracle's simulation of the same lookups, and the whole directory (row held and stamp of
every way) equal to the oracle's."""
import numpy as np
import pytest
import torch

from oracle import cache as oc
from cvr_ranking_model_amd import synth
from cvr_ranking_model_amd import cvr as cv
from gpu_common import banner, build_model, run
from conftest import tiny_dlrm_spec
from test_gpu_dlrm import check_dlrm

pytestmark = pytest.mark.gpu


def pinned(t):
    h = torch.empty(t.shape, dtype=t.dtype, pin_memory=True)
    h.copy_(t)
    return h


def check_call(m, ref, spec, b, sims, label):
    _, out, st = run(m, b)
    assert st == cv.CVR_OK
    _, want, st = run(ref, b)
    assert st == cv.CVR_OK
    assert np.array_equal(out.cpu().numpy(), want.cpu().numpy()), label
    for table, sim in sims.items():
        sim.batch(oc.table_lookups(spec, b, table), rows=spec["tables"][table]["rows"])
        got = m.cache_stats(table)
        assert got == sim.counters, (label, table, got, sim.counters)
        tags, stamps = m.cache_export(table)
        assert np.array_equal(tags, sim.tags), (label, table)
        assert np.array_equal(stamps, sim.stamps), (label, table)
    return out


def test_tiny_cache_tracks_oracle_over_batches():
    spec = tiny_dlrm_spec(dims=(16, 16, 32, 32), hidden=(64, 32), rows=300, bag_max=6)
    dev = cv.device_tables(spec, "stress")
    host = [pinned(dev[0]), dev[1], pinned(dev[2]), dev[3]]
    banner("tiny DLRM: tables 0 and 2 in pinned host memory behind 3x2 and 8x4 caches, 8 calls")
    m, _ = build_model(spec, "stress", tables=host, debug=False)
    ref, _ = build_model(spec, "stress", tables=dev, debug=False)
    m.attach_cache(0, 3, 2)
    m.attach_cache(2, 8, 4)
    sims = {0: oc.HotRowCache(3, 2), 2: oc.HotRowCache(8, 4)}
    for call in range(8):
        b = synth.make_batch(spec, requests=5, candidates=7, seed_offset=call % 5)   # calls 5-7 repeat 0-2
        check_call(m, ref, spec, b, sims, f"call {call}")
    c = sims[2].counters
    banner(f"  table 2: {c}")
    assert c["hits"] > 0 and c["evictions"] > 0


def test_c2_item_table_behind_cache():
    """C2 with its 5M-row item-ID table in host memory behind a 65,536 x 8 cache."""
    spec = synth.load_spec("c2")
    dev = cv.device_tables(spec, "stress")
    t_item = next(f["table"] for f in spec["features"] if f["name"] == "item_id")
    host = list(dev)
    host[t_item] = pinned(dev[t_item])
    banner(f"c2: item-ID table (table {t_item}) in host memory behind a 65536 x 8 cache; 4 calls of 8 requests")
    m, _ = build_model(spec, "stress", tables=host, debug=False)
    ref, _ = build_model(spec, "stress", tables=dev, debug=False)
    m.attach_cache(t_item, 65536, 8)
    sims = {t_item: oc.HotRowCache(65536, 8)}
    for call in range(4):
        b = synth.make_batch(spec, requests=8, seed_offset=call % 2)
        check_call(m, ref, spec, b, sims, f"call {call}")
    c = sims[t_item].counters
    banner(f"  counters {c}; hit rate {c['hits'] / c['lookups']:.3f}")
    assert c["hits"] > 0


def test_cached_model_matches_oracle():
    """The pooled inputs and scores of a cached model against the oracle (debug exports on)."""
    spec = tiny_dlrm_spec(dims=(16, 16, 32, 32), hidden=(64, 32), rows=300, bag_max=6)
    dev = cv.device_tables(spec, "stress")
    host = [pinned(t) for t in dev]
    m, _ = build_model(spec, "stress", tables=host)
    m.attach_cache(1, 4, 4)
    m.attach_cache(3, 5, 2)
    tables_host = [t.materialize() for t in synth.make_tables(spec, "stress")]
    for call in range(3):
        check_dlrm(spec, m, synth.make_batch(spec, requests=4, candidates=6, seed_offset=call), "stress",
                   tables_host=tables_host)


def test_graph_replay_advances_the_cache():
    spec = tiny_dlrm_spec(dims=(16, 16, 32, 32), hidden=(64, 32), rows=300, bag_max=6)
    dev = cv.device_tables(spec, "stress")
    host = [dev[0], dev[1], pinned(dev[2]), dev[3]]
    m, _ = build_model(spec, "stress", tables=host, debug=False)
    m.attach_cache(2, 8, 4)
    sim = oc.HotRowCache(8, 4)
    b = synth.make_batch(spec, requests=5, candidates=7)
    db = cv.DeviceBatch(b)
    for rep in range(4):
        m.score_graph(db)
        sim.batch(oc.table_lookups(spec, b, 2), rows=300)
        assert m.sync_status() == cv.CVR_OK
        assert m.cache_stats(2) == sim.counters, rep
        tags, stamps = m.cache_export(2)
        assert np.array_equal(tags, sim.tags) and np.array_equal(stamps, sim.stamps), rep


def test_attach_errors():
    spec = tiny_dlrm_spec(dims=(16, 16, 32, 32), hidden=(64, 32), rows=300, bag_max=6)
    dev = cv.device_tables(spec, "stress")
    m, _ = build_model(spec, "stress", tables=dev, debug=False)
    with pytest.raises(cv.CvrError):
        m.attach_cache(0, 4, 5)            # more ways than dim/4 lanes
    with pytest.raises(cv.CvrError):
        m.attach_cache(9, 4, 2)            # no such table
    m.attach_cache(0, 4, 2)
    with pytest.raises(cv.CvrError):
        m.attach_cache(0, 4, 2)            # already cached
    with pytest.raises(cv.CvrError):
        m.cache_stats(1)                   # not cached


def test_cvr_model_with_cached_table():
    """The CVR model reads a cached non-sequence table through the same gather; a
    sequence-column table cannot take a cache."""
    spec = synth.load_spec("c3")
    dev = cv.device_tables(spec, "stress")
    t0 = spec["features"][0]["table"]
    host = list(dev)
    host[t0] = pinned(dev[t0])
    banner(f"c3 stress: non-sequence table {t0} in host memory behind a 4096 x 4 cache; 3 calls")
    m, _ = build_model(spec, "stress", tables=host, debug=False)
    ref, _ = build_model(spec, "stress", tables=dev, debug=False)
    m.attach_cache(t0, 4096, 4)
    sims = {t0: oc.HotRowCache(4096, 4)}
    for call in range(3):
        b = synth.make_batch(spec, requests=16, seed_offset=call % 2)
        check_call(m, ref, spec, b, sims, f"call {call}")
    seq_table = spec["seq"]["columns"][0]["table"]
    with pytest.raises(cv.CvrError):
        m.attach_cache(seq_table, 64, 2)
