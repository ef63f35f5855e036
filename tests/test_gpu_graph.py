"""Graph replay per batch bucket (CVR article section 3.4.4) against eager scoring.

Every replay is compared bit for bit with the eager result of the same batch: the graph
holds the same kernels, run at the bucket's sizes on a padded copy of the batch, and the
padding belongs to no caller request.  Replays alternate with eager scoring of other
batches and with synchronisations; batches of other sizes inside one bucket (other ids,
other candidate counts, other id counts) replay without a new capture; another bucket
captures once and the first bucket's graph stays; malformed batches are still reported.
"""
import numpy as np
import pytest
import torch

from cvr_ranking_model_amd import synth
from cvr_ranking_model_amd import cvr as cv
from gpu_common import banner, build_model

pytestmark = pytest.mark.gpu


def _shuffled_ids(spec, batch, seed):
    """Same sizes and offsets, other ids: each feature's ids (and each sequence column) are
    permuted among themselves, so every id stays inside its table."""
    b = dict(batch)
    ids = np.array(batch["ids"], dtype=np.int32).copy()
    bo = np.asarray(batch["bag_offsets"], dtype=np.int64)
    R = len(batch["cand_offsets"]) - 1
    n = int(batch["cand_offsets"][-1])
    rng = np.random.default_rng(seed)
    o = 0
    for f in spec["features"]:
        nb = n if f["side"] == "item" else R
        seg = ids[bo[o]:bo[o + nb]]
        rng.shuffle(seg)
        ids[bo[o]:bo[o + nb]] = seg
        o += nb
    b["ids"] = ids
    if batch.get("seq_ids") is not None:
        sq = np.array(batch["seq_ids"], dtype=np.int32).copy()
        for c in range(sq.shape[1]):
            rng.shuffle(sq[:, c])
        b["seq_ids"] = sq
    return b


def _eager(m, batch):
    out = m.score(cv.DeviceBatch(batch))
    assert m.sync_status() == cv.CVR_OK
    return out.clone()


@pytest.mark.parametrize("name,requests", [("c1", None), ("c3", 8)])
def test_graph_replay_matches_eager(name, requests):
    spec = synth.load_spec(name)
    banner(f"graph replay {name}: capture, replays between eager calls, refill, recapture")
    m, _ = build_model(spec, "stress", debug=False)
    A = synth.make_batch(spec, requests=requests, seed_offset=3)
    B = synth.make_batch(spec, requests=requests, seed_offset=4)
    ref_a, ref_b = _eager(m, A), _eager(m, B)
    assert not torch.equal(ref_a[: min(len(ref_a), len(ref_b))], ref_b[: min(len(ref_a), len(ref_b))])
    da, db = cv.DeviceBatch(A), cv.DeviceBatch(B)
    out_a = torch.empty_like(ref_a)
    out_b = torch.empty_like(ref_b)
    for rep in range(4):
        out_a.fill_(-1.0)
        m.score_graph(da, out_a)
        torch.cuda.synchronize()
        assert m.sync_status() == cv.CVR_OK
        assert torch.equal(out_a, ref_a), f"replay {rep} differs from eager"
        eager_b = m.score(db)
        torch.cuda.synchronize()
        assert torch.equal(eager_b, ref_b)
    # same buffers, new contents: the replay must read them
    A2 = _shuffled_ids(spec, A, 11)
    ref_a2 = _eager(m, A2)
    assert not torch.equal(ref_a2, ref_a)
    da.refill(A2)
    m.score_graph(da, out_a)
    torch.cuda.synchronize()
    assert torch.equal(out_a, ref_a2)
    # the other batch: one more capture only if its sizes fall in another bucket
    captures = m.graph_info()[1] + (0 if _key(_sizes(A)) == _key(_sizes(B)) else 1)
    m.score_graph(db, out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_b, ref_b)
    m.score_graph(da, out_a)
    torch.cuda.synchronize()
    assert torch.equal(out_a, ref_a2)
    assert m.graph_info()[1] == captures
    banner(f"graph replay {name}: {len(ref_a)} scores equal to eager on every replay")


def bucket(x):
    """The bucket rule of cvr_score_graph: the next m * 2^k with 8 <= m <= 16 (exact below 16)."""
    if x < 16:
        return x
    k = 0
    while (x >> k) >= 16:
        k += 1
    return ((x + (1 << k) - 1) >> k) << k


def _sizes(b):
    return (len(b["cand_offsets"]) - 1, int(b["cand_offsets"][-1]), len(b["ids"]),
            0 if b.get("seq_ids") is None else int(b["seq_ids"].shape[0]))


def _key(s):
    R, n, ids, P = s
    return bucket(R + 1), bucket(n + 1), bucket(ids), bucket(P)


def _same_bucket_batches(make, want, tries=40):
    """`want` seeded batches from make(seed) with pairwise different sizes in the most common
    bucket among `tries` draws."""
    by_key = {}
    for seed in range(tries):
        b = make(seed)
        group = by_key.setdefault(_key(_sizes(b)), {})
        group.setdefault(_sizes(b), b)
    group = max(by_key.values(), key=len)
    assert len(group) >= want, "no batches in a common bucket"
    return list(group.values())[:want]


@pytest.mark.parametrize("name", ["c1", "c3"])
def test_bucket_replays_batches_of_other_sizes(name):
    """Batches of different candidate counts and id counts (and, for the CVR model, request
    counts and sequence lengths) that fall in one bucket replay one captured graph, bit for bit
    equal to eager scoring; a batch of another bucket captures once, after which the first
    bucket still replays without capturing."""
    spec = synth.load_spec(name)
    rng = np.random.default_rng(7)
    if name == "c1":
        make = lambda seed: synth.make_batch(spec, requests=1, candidates=int(rng.integers(193, 208)),
                                             seed_offset=40 + seed)
        other = synth.make_batch(spec, requests=1, candidates=60, seed_offset=99)
    else:
        make = lambda seed: synth.make_batch(spec, requests=int(rng.integers(45, 49)), seed_offset=40 + seed)
        other = synth.make_batch(spec, requests=3, seed_offset=99)
    batches = _same_bucket_batches(make, 4)
    banner(f"graph buckets {name}: sizes {[_sizes(b) for b in batches]} -> bucket {_key(_sizes(batches[0]))}")
    m, _ = build_model(spec, "stress", debug=False)
    if spec["model"] == "hyformer":
        # fix the size-dependent kernel choices so that eager and bucket calls take the same kernels
        m.set_option(cv.CVR_OPT_TOK_SHARE, 0)
        m.set_option(cv.CVR_OPT_ATTN_MQ, 0)
    refs = [_eager(m, b) for b in batches]
    big = tuple(max(s[i] for s in map(_sizes, batches + [other])) for i in range(4))
    dbs = [cv.DeviceBatch(b) for b in batches]
    assert m.graph_info() == (0, 0)
    for rep in range(2):
        for db, ref in zip(dbs, refs):
            out = torch.full_like(ref, -1.0)
            m.score_graph(db, out, ws_sizes=big)
            torch.cuda.synchronize()
            assert m.sync_status() == cv.CVR_OK
            assert torch.equal(out, ref), f"replay {rep} differs from eager"
            eager_again = m.score(cv.DeviceBatch(other))      # eager work between replays
            torch.cuda.synchronize()
    assert m.graph_info() == (1, 1)
    ref_o = _eager(m, other)
    out_o = torch.empty_like(ref_o)
    m.score_graph(cv.DeviceBatch(other), out_o, ws_sizes=big)
    torch.cuda.synchronize()
    assert torch.equal(out_o, ref_o)
    assert m.graph_info() == (2, 2)
    out = torch.empty_like(refs[0])
    m.score_graph(dbs[0], out, ws_sizes=big)
    torch.cuda.synchronize()
    assert torch.equal(out, refs[0])
    assert m.graph_info() == (2, 2)


def test_bucket_replay_reports_malformed_batches():
    """Padding a batch to its bucket keeps malformed offsets malformed: a last candidate offset
    other than n_candidates, a last bag offset other than n_ids and a sequence offset past
    n_positions are reported after a replay as after an eager call."""
    spec = synth.load_spec("c3")
    m, _ = build_model(spec, "stress", debug=False)
    b = synth.make_batch(spec, requests=6, candidates=2, seed_offset=5)
    db = cv.DeviceBatch(b)
    out = torch.empty(db.n_candidates * spec["n_tasks"], dtype=torch.float32, device="cuda")
    m.score_graph(db, out)
    assert m.sync_status() == cv.CVR_OK
    co = b["cand_offsets"].copy()
    co[-1] -= 1
    bo = b["bag_offsets"].copy()
    bo[-1] -= 1
    so = b["seq_offsets"].copy()
    so[0, 2] = b["seq_ids"].shape[0] + 1
    for name, bad in [("cand_offsets", dict(b, cand_offsets=co)), ("bag_offsets", dict(b, bag_offsets=bo)),
                      ("seq_offsets", dict(b, seq_offsets=so))]:
        banner(f"graph replay with malformed {name}")
        m.score(cv.DeviceBatch(bad))
        assert m.sync_status() == cv.CVR_ERR_RANGE, name
        m.score_graph(cv.DeviceBatch(bad), out)
        assert m.sync_status() == cv.CVR_ERR_RANGE, name
    m.score_graph(db, out)
    assert m.sync_status() == cv.CVR_OK


def test_graph_needs_created_stream():
    spec = synth.load_spec("c1")
    m, _ = build_model(spec, "stress", debug=False)
    db = cv.DeviceBatch(synth.make_batch(spec, seed_offset=5))
    ws = m.workspace(db.n_requests, db.n_candidates, db.n_ids, db.n_positions)
    out = torch.empty(db.n_candidates, dtype=torch.float32, device="cuda")
    import ctypes as C
    with pytest.raises(cv.CvrError):
        cv.cvr_score_graph(m.h, db.c, C.c_void_p(ws.data_ptr()), ws.numel(), C.c_void_p(out.data_ptr()), C.c_void_p(0))


def test_graph_replay_restores_export_state():
    """A replay leaves the handle describing the replayed call: after a debug-off graph (last
    layer's tokens written as bf16) is replayed following an eager debug-on call, the fp32 token
    export is refused instead of returning bf16 bytes read as fp32."""
    spec = synth.load_spec("c3")
    banner("graph replay c3: export state after replay")
    m, _ = build_model(spec, "stress", debug=False)
    db = cv.DeviceBatch(synth.make_batch(spec, requests=8, seed_offset=6))
    out = torch.empty(db.n_candidates * spec["n_tasks"], dtype=torch.float32, device="cuda")
    shape = (db.n_candidates, spec["n_tokens"] + 3, spec["d"])
    m.score_graph(db, out)
    torch.cuda.synchronize()
    ref = out.clone()
    m.set_debug(True)
    m.score(db)
    assert m.sync_status() == cv.CVR_OK
    m.export(cv.CVR_DBG_TOKENS, torch.float32, shape)          # fp32 tokens after the debug call
    m.set_debug(False)
    m.score_graph(db, out)                                     # replays the debug-off capture
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    with pytest.raises(cv.CvrError, match="bf16"):
        m.export(cv.CVR_DBG_TOKENS, torch.float32, shape)
