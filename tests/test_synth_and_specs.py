"""Pins for the seeded input generators and for the config specs against the pages' numbers."""
import numpy as np

from cvr_ranking_model_amd import synth
from conftest import golden


def test_splitmix64_reference_outputs():
    lines = [l for l in golden("splitmix64_seed1234567.txt").splitlines() if l and not l.startswith("#")]
    want = [int(x) for x in lines]
    assert [int(v) for v in synth.splitmix64_outputs(1234567, np.arange(5))] == want


def test_table_values_uniform_and_regenerable():
    t = synth.HashTable(rows=1000, dim=64, seed=synth.table_seed(5, 3), halfwidth=0.05)
    v = t.materialize()
    assert v.dtype == np.float32 and v.shape == (1000, 64)
    assert v.min() >= -0.05 and v.max() < 0.05
    assert abs(v.mean()) < 1e-3 and abs(v.var() - 0.05 ** 2 / 3) < 5e-5
    rows = np.array([999, 0, 17, 17])
    assert np.array_equal(t[rows], v[rows])
    # values sit on the 2**24-level grid: (k - 2**23) * step with integer k
    k = v.astype(np.float64) / synth.value_step(0.05)
    assert np.allclose(k, np.round(k), atol=1e-3)


def test_zipf_ids_follow_power_law():
    rng = np.random.default_rng(0)
    V, a = 1_000_000, 1.05
    ids = synth.zipf_rows(rng, V, a, 400_000, table_index=0)
    assert ids.min() >= 0 and ids.max() < V
    # share of draws on the top-k ranks versus the continuous CDF ((k+1)^(1-a) - 1) / (V^(1-a) - 1)
    P = synth.ID_SCATTER_PRIME % V
    Q = 12345 % V
    inv = pow(P, -1, V)
    rank = ((ids.astype(np.int64) - Q) * inv) % V + 1
    for k in [1, 10, 1000, 100_000]:
        want = ((k + 1) ** (1 - a) - 1) / (V ** (1 - a) - 1)
        assert abs(np.mean(rank <= k) - want) < 0.005, k


def test_batch_layout_and_determinism():
    spec = synth.load_spec("c2")
    b1 = synth.make_batch(spec, requests=3)
    b2 = synth.make_batch(spec, requests=3)
    for k in ["cand_offsets", "bag_offsets", "ids"]:
        assert np.array_equal(b1[k], b2[k])
    assert b1["cand_offsets"].tolist() == [0, 500, 1000, 1500]
    assert len(b1["bag_offsets"]) == 9 * 3 + 9 * 1500 + 1
    lens = np.diff(b1["bag_offsets"])
    assert np.all(lens[:3] == 1)                     # user-ID bags are single-hot
    assert lens[3:27].min() >= 1 and lens[3:27].max() <= 16
    spec4 = synth.load_spec("c4")
    b = synth.make_batch(spec4, requests=2, ragged=True)
    so = b["seq_offsets"]
    assert so.shape == (3, 3) and so[0, 0] == 0 and so[1, 0] == so[0, 2] and so[2, -1] == len(b["seq_ids"])


def test_specs_follow_the_pages():
    g = golden("pages_constants.json")
    c5 = synth.load_spec("c5")
    assert [[t["rows"], t["dim"]] for t in c5["tables"]] == g["ctr_tables"]["value"]
    sizes = [t["rows"] * t["dim"] * 4 / 1e9 for t in c5["tables"]]
    assert abs(sizes[0] + sizes[1] - g["ctr_user_side_gb"]["value"]) < 0.2
    assert abs(sizes[2] + sizes[3] - g["ctr_item_side_gb"]["value"]) < 0.05
    assert abs(sum(sizes) - g["ctr_total_gb"]["value"]) < 0.5
    lo, hi = g["candidates_per_request_range"]["value"]
    for name in ["c1", "c2", "c5"]:
        s = synth.load_spec(name)
        assert s["clamp"] == g["clamp_bound"]["value"]
        assert set(s["mlp_hidden"]) == {g["mlp_width"]["value"]}
        assert g["mlp_layers_range"]["value"][0] <= len(s["mlp_hidden"]) <= g["mlp_layers_range"]["value"][1]
        assert lo <= s["workload"]["candidates"] <= hi
    for name in ["c3", "c4"]:
        s = synth.load_spec(name)
        assert s["d"] == g["token_dim"]["value"] and s["n_tokens"] == g["n_nonseq_tokens"]["value"]
        assert len(s["seq"]["lengths"]) == g["n_queries"]["value"]
        assert s["n_experts"] == g["ple_experts"]["value"]
        assert s["n_tokens"] + len(s["seq"]["lengths"]) == g["mixer_tokens"]["value"]
        assert sum(s["tables"][c["table"]]["dim"] for c in s["seq"]["columns"]) == s["d"]
    assert synth.load_spec("c3")["n_layers"] == g["production_layers"]["value"]


def test_stress_variant_spreads_scores():
    # bench data keeps scores near 0.5; stress data must not (otherwise score parity says little)
    import oracle
    spec = synth.load_spec("c1")
    b = synth.make_batch(spec)
    bench = oracle.score(spec, synth.make_tables(spec, "bench"), synth.make_weights(spec, "bench"), b)["scores"]
    stress = oracle.score(spec, synth.make_tables(spec, "stress"), synth.make_weights(spec, "stress"), b)["scores"]
    assert bench.std() < 0.005 and stress.std() > 0.1
