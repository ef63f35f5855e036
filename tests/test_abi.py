"""The C ABI library loads and exports every entry point include/cvr.h declares; host-only checks.

No test here launches device work: these run without a GPU.
"""
import ctypes as C
import os
import re

import numpy as np
import pytest

from cvr_ranking_model_amd import synth
from cvr_ranking_model_amd import cvr as cv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cvr.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+char\s*\*|cvr_status|void)\s+(cvr_\w+)\s*\(", src, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ["cvr_create", "cvr_score", "cvr_weight_arena_bytes", "cvr_workspace_bytes", "cvr_sync_status",
                 "cvr_destroy", "cvr_debug_export", "cvr_fill_table"]:
        assert must in names


def test_library_exports_every_declared_symbol():
    lib = cv.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(cv._PROTOS) == set(declared_functions())


class _FakeTensor:
    def __init__(self, rows, dim):
        self.shape = (rows, dim)

    def data_ptr(self):
        return 0


def _spec_c(spec):
    tabs = [_FakeTensor(t["rows"], t["dim"]) for t in spec["tables"]]
    return cv.spec_to_c(spec, tabs)


def test_arena_size_matches_weight_shapes():
    for name in ["c1", "c2", "c3", "c4", "c5"]:
        spec = synth.load_spec(name)
        s, tabs, keep = _spec_c(spec)
        nbytes = cv.cvr_weight_arena_bytes(s, tabs, len(spec["tables"]))
        want = 0
        for wname, shape in synth.weight_shapes(spec).items():
            n = int(np.prod(shape))
            want += ((n * (2 if wname.endswith(".weight") else 4)) + 255) // 256 * 256
        if spec["model"] == "dlrm":
            # the first Linear's request-side and item-side columns as two more matrices
            dims = [spec["tables"][f["table"]]["dim"] for f in spec["features"]]
            d_item = sum(dmn for dmn, f in zip(dims, spec["features"]) if f["side"] == "item")
            w0 = spec["mlp_hidden"][0]
            want += (w0 * (sum(dims) - d_item) * 2 + 255) // 256 * 256 + (w0 * d_item * 2 + 255) // 256 * 256
        if spec["model"] == "hyformer":
            # one internal fp32 bias vector for the expert GEMM: expert biases, then gate biases
            gates = spec["n_tasks"] * spec["n_experts"]
            want += ((spec["n_experts"] * spec["expert_dim"] + gates) * 4 + 255) // 256 * 256
            # the tokenizer's request-side and item-side columns as two more matrices
            dims = [spec["tables"][f["table"]]["dim"] for f in spec["features"]]
            item = [f["side"] == "item" for f in spec["features"]]
            runs, prev = [], None
            for dmn, it in zip(dims, item):
                if prev is not None and it == prev:
                    runs[-1] += dmn
                else:
                    runs.append(dmn)
                prev = it
            d_item = sum(dmn for dmn, it in zip(dims, item) if it)
            d_req = sum(dims) - d_item
            if d_req and d_item and all(r % 32 == 0 for r in runs):
                rows = spec["n_tokens"] * spec["d"]
                want += (rows * d_req * 2 + 255) // 256 * 256 + (rows * d_item * 2 + 255) // 256 * 256
        assert nbytes == want, name


def test_bad_specs_are_rejected_on_the_host():
    spec = synth.load_spec("c1")
    s, tabs, keep = _spec_c(spec)
    s.model = 7
    with pytest.raises(cv.CvrError) as e:
        cv.cvr_weight_arena_bytes(s, tabs, len(spec["tables"]))
    assert e.value.status == cv.CVR_ERR_SPEC
    s, tabs, keep = _spec_c(spec)
    s.features[0].table = 9
    with pytest.raises(cv.CvrError, match="table index"):
        cv.cvr_weight_arena_bytes(s, tabs, len(spec["tables"]))
    bad = dict(spec, mlp_hidden=[1000])
    s, tabs, keep = _spec_c(bad)
    with pytest.raises(cv.CvrError) as e:
        cv.cvr_weight_arena_bytes(s, tabs, len(spec["tables"]))
    assert e.value.status == cv.CVR_ERR_UNSUPPORTED
    cvr = synth.load_spec("c3")
    s, tabs, keep = _spec_c(dict(cvr, d=64))
    with pytest.raises(cv.CvrError) as e:
        cv.cvr_weight_arena_bytes(s, tabs, len(cvr["tables"]))
    assert e.value.status == cv.CVR_ERR_UNSUPPORTED


def test_cvr_spec_in_fp16_is_rejected():
    """The CVR kernels compute in bf16 (the CVR article's BF16 inference): a CVR spec asking for
    fp16 is refused rather than scored with fp16 bit patterns read as bf16."""
    cvr = synth.load_spec("c3")
    s, tabs, keep = _spec_c(dict(cvr, lowp="fp16"))
    with pytest.raises(cv.CvrError, match="bf16") as e:
        cv.cvr_weight_arena_bytes(s, tabs, len(cvr["tables"]))
    assert e.value.status == cv.CVR_ERR_UNSUPPORTED
    s, tabs, keep = _spec_c(cvr)
    assert cv.cvr_weight_arena_bytes(s, tabs, len(cvr["tables"])) > 0


def test_epnet_spec_checks():
    cvr = synth.load_spec("c3")
    s, tabs, keep = _spec_c(dict(cvr, epnet_hidden=100))
    with pytest.raises(cv.CvrError) as e:
        cv.cvr_weight_arena_bytes(s, tabs, len(cvr["tables"]))
    assert e.value.status == cv.CVR_ERR_UNSUPPORTED
    no_ctx = dict(cvr, epnet_hidden=128, features=[dict(f, side="user") if f["side"] == "context" else f
                                                   for f in cvr["features"]])
    s, tabs, keep = _spec_c(no_ctx)
    with pytest.raises(cv.CvrError, match="context"):
        cv.cvr_weight_arena_bytes(s, tabs, len(cvr["tables"]))
    # the arena gains the two gate Linears (bf16) and their biases (fp32), and loses the
    # tokenizer's request-side and item-side copies (the scaled input is per candidate, so the
    # request-side block is no longer shared)
    base = cv.cvr_weight_arena_bytes(*_spec_c(cvr)[:2], len(cvr["tables"]))
    s, tabs, keep = _spec_c(dict(cvr, epnet_hidden=128))
    grown = cv.cvr_weight_arena_bytes(s, tabs, len(cvr["tables"]))
    r = lambda x: (x + 255) // 256 * 256
    gate = r(128 * (256 + 1280) * 2) + r(128 * 4) + r(1280 * 128 * 2) + r(1280 * 4)
    split = r(13 * 128 * 768 * 2) + r(13 * 128 * 512 * 2)
    assert grown - base == gate - split


def test_set_option_needs_a_handle_and_known_values():
    L = cv.lib()
    assert L.cvr_set_option(None, cv.CVR_OPT_ATTN_MQ, 1) == cv.CVR_ERR_ARG
    assert "null handle" in L.cvr_last_error(None).decode()


def test_fill_and_create_argument_checks():
    with pytest.raises(cv.CvrError) as e:
        cv.cvr_fill_table(None, 10, 4, 1, 0.05, None)
    assert e.value.status == cv.CVR_ERR_ARG
    spec = synth.load_spec("c1")
    s, tabs, keep = _spec_c(spec)
    with pytest.raises(cv.CvrError) as e:   # null table data is refused before any device work
        cv.cvr_create(s, tabs, len(spec["tables"]), None, 0, None, 0, None)
    assert e.value.status == cv.CVR_ERR_ARG
    assert cv.lib().cvr_status_string(cv.CVR_ERR_RANGE).decode().startswith("id or offset")


def test_cache_state_bytes_host_checks():
    small = cv.cvr_cache_state_bytes(16, 4, 32)
    assert small >= 16 * 4 * 32 * 4 and small % 256 == 0          # at least the cached rows
    assert cv.cvr_cache_state_bytes(32, 4, 32) > small
    for sets, ways, dim in [(0, 4, 32), (16, 0, 32), (16, 17, 64), (16, 4, 30), (1 << 30, 4, 32)]:
        with pytest.raises(cv.CvrError):
            cv.cvr_cache_state_bytes(sets, ways, dim)


def test_probe_argument_checks():
    """The bandwidth probes refuse null pointers, misaligned or ragged sizes, grids outside
    [1, 2^20], row widths other than 64/128/256 bytes and load forms other than 0/1 before any
    device work."""
    import ctypes as C
    fake = C.c_void_p(1 << 20)    # aligned non-null stand-in; never dereferenced on these paths
    cases = [
        lambda: cv.cvr_probe_stream_read(None, 1024, fake, 64, None),
        lambda: cv.cvr_probe_stream_read(fake, 1024, None, 64, None),
        lambda: cv.cvr_probe_stream_read(C.c_void_p((1 << 20) + 4), 1024, fake, 64, None),
        lambda: cv.cvr_probe_stream_read(fake, 1000, fake, 64, None),
        lambda: cv.cvr_probe_stream_read(fake, 1024, fake, 0, None),
        lambda: cv.cvr_probe_stream_read(fake, 1024, fake, (1 << 20) + 1, None),
        lambda: cv.cvr_probe_row_read(fake, 100, 96, fake, 10, fake, 64, None),
        lambda: cv.cvr_probe_row_read(fake, 0, 128, fake, 10, fake, 64, None),
        lambda: cv.cvr_probe_row_read(None, 100, 128, fake, 10, fake, 64, None),
        lambda: cv.cvr_probe_row_read(fake, 100, 128, fake, -1, fake, 64, None),
        lambda: cv.cvr_probe_row_read(fake, 100, 128, fake, 10, fake, 0, None),
        lambda: cv.cvr_probe_stream_read(fake, 1024, fake, 64, None, nontemporal=2),
        lambda: cv.cvr_probe_row_read(fake, 100, 128, fake, 10, fake, 64, None, nontemporal=-1),
    ]
    for call in cases:
        with pytest.raises(cv.CvrError) as e:
            call()
        assert e.value.status == cv.CVR_ERR_ARG
