"""Graph replay of a scoring call (CVR article section 3.4.4) against eager scoring.

Every replay is compared bit for bit with the eager result of the same batch: the graph
holds the same kernels with the same arguments.  Replays alternate with eager scoring of
another batch and with synchronisations; a batch refilled in place (same buffers, other
ids) must be scored from its new contents; a different batch must recapture.
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
    # another batch recaptures, and the first one again after it
    m.score_graph(db, out_b)
    torch.cuda.synchronize()
    assert torch.equal(out_b, ref_b)
    m.score_graph(da, out_a)
    torch.cuda.synchronize()
    assert torch.equal(out_a, ref_a2)
    banner(f"graph replay {name}: {len(ref_a)} scores equal to eager on every replay")


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
