"""Python binding of libcvr (ctypes).

The functions ``cvr_*`` mirror the C ABI in ``include/cvr.h`` one to one and
only marshal arguments; every step of scoring runs in the HIP library.  torch
provides device memory and streams.  :class:`Model` and :class:`DeviceBatch`
are conveniences that size and hold those buffers.

The library is loaded on first use from this package's directory; if it has
not been built the import of a function fails loudly.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcvr.so")

CVR_OK, CVR_ERR_ARG, CVR_ERR_SPEC, CVR_ERR_RANGE, CVR_ERR_WORKSPACE, CVR_ERR_HIP, CVR_ERR_UNSUPPORTED = range(7)
CVR_MODEL_DLRM, CVR_MODEL_HYFORMER = 0, 1
CVR_SIDE_USER, CVR_SIDE_ITEM, CVR_SIDE_CONTEXT = 0, 1, 2
CVR_LOWP_FP16, CVR_LOWP_BF16 = 0, 1
(CVR_DBG_CAND_REQ, CVR_DBG_POOLED, CVR_DBG_INPUT_REQ, CVR_DBG_INPUT_ITEM, CVR_DBG_LOGITS, CVR_DBG_HSEQ,
 CVR_DBG_SEQ_POOL, CVR_DBG_TOKENS, CVR_DBG_QUERY, CVR_DBG_ATTN, CVR_DBG_HIDDEN, CVR_DBG_EPNET) = range(12)
(CVR_OPT_DLRM_PASS_ROWS, CVR_OPT_TOK_SHARE, CVR_OPT_ATTN_MQ, CVR_OPT_DLRM_USER_BLOCK, CVR_OPT_HEADS_FUSED,
 CVR_OPT_STATE_STREAM) = range(6)
SIDES = {"user": CVR_SIDE_USER, "item": CVR_SIDE_ITEM, "context": CVR_SIDE_CONTEXT}


class cvr_table(C.Structure):
    _fields_ = [("data", C.c_void_p), ("rows", C.c_int64), ("dim", C.c_int32)]


class cvr_feature(C.Structure):
    _fields_ = [("table", C.c_int32), ("side", C.c_int32)]


class cvr_spec(C.Structure):
    _fields_ = [("model", C.c_int32), ("lowp", C.c_int32), ("clamp", C.c_float),
                ("n_features", C.c_int32), ("features", C.POINTER(cvr_feature)),
                ("n_hidden", C.c_int32), ("hidden", C.POINTER(C.c_int32)),
                ("d", C.c_int32), ("n_tokens", C.c_int32), ("n_layers", C.c_int32), ("n_seq", C.c_int32),
                ("n_seq_cols", C.c_int32), ("seq_tables", C.POINTER(C.c_int32)),
                ("swiglu_hidden", C.c_int32), ("tau", C.c_float), ("mixer_heads", C.c_int32),
                ("mixer_hidden", C.c_int32), ("n_experts", C.c_int32), ("expert_dim", C.c_int32),
                ("n_tasks", C.c_int32), ("head_hidden", C.c_int32), ("task_experts", C.POINTER(C.c_int32)),
                ("epnet_hidden", C.c_int32)]


class cvr_weight(C.Structure):
    _fields_ = [("name", C.c_char_p), ("data", C.c_void_p), ("numel", C.c_int64)]


class cvr_batch(C.Structure):
    _fields_ = [("n_requests", C.c_int32), ("n_candidates", C.c_int32), ("n_ids", C.c_int64),
                ("n_positions", C.c_int64), ("cand_offsets", C.c_void_p), ("bag_offsets", C.c_void_p),
                ("ids", C.c_void_p), ("seq_offsets", C.c_void_p), ("seq_ids", C.c_void_p)]


_PROTOS = {
    "cvr_weight_arena_bytes": (C.c_int, [C.POINTER(cvr_spec), C.POINTER(cvr_table), C.c_int32, C.POINTER(C.c_size_t)]),
    "cvr_create": (C.c_int, [C.POINTER(cvr_spec), C.POINTER(cvr_table), C.c_int32, C.POINTER(cvr_weight), C.c_int32,
                             C.c_void_p, C.c_size_t, C.c_void_p, C.POINTER(C.c_void_p)]),
    "cvr_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int64, C.c_int64, C.POINTER(C.c_size_t)]),
    "cvr_score": (C.c_int, [C.c_void_p, C.POINTER(cvr_batch), C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]),
    "cvr_score_graph": (C.c_int, [C.c_void_p, C.POINTER(cvr_batch), C.c_void_p, C.c_size_t, C.c_void_p, C.c_void_p]),
    "cvr_score_noalloc": (C.c_int, [C.c_void_p, C.POINTER(cvr_batch), C.c_void_p, C.c_void_p]),
    "cvr_graph_workspace_bytes": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int64, C.c_int64,
                                            C.POINTER(C.c_size_t)]),
    "cvr_graph_info": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "cvr_sync_status": (C.c_int, [C.c_void_p, C.c_void_p]),
    "cvr_set_debug": (C.c_int, [C.c_void_p, C.c_int32]),
    "cvr_set_option": (C.c_int, [C.c_void_p, C.c_int32, C.c_int64]),
    "cvr_debug_export": (C.c_int, [C.c_void_p, C.c_int32, C.c_void_p, C.c_size_t, C.POINTER(C.c_size_t), C.c_void_p]),
    "cvr_timing_begin": (C.c_int, [C.c_void_p, C.c_int32, C.c_uint32]),
    "cvr_timing_end": (C.c_int, [C.c_void_p, C.POINTER(C.c_double), C.POINTER(C.c_int32), C.c_int32,
                                 C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
    "cvr_stage_name": (C.c_char_p, [C.c_void_p, C.c_int32]),
    "cvr_fill_table": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_uint64, C.c_double, C.c_void_p]),
    "cvr_cache_state_bytes": (C.c_int, [C.c_int64, C.c_int32, C.c_int32, C.POINTER(C.c_size_t)]),
    "cvr_cache_attach": (C.c_int, [C.c_void_p, C.c_int32, C.c_int64, C.c_int32, C.c_void_p, C.c_size_t, C.c_void_p]),
    "cvr_cache_stats": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int64), C.c_void_p]),
    "cvr_cache_export": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.c_void_p]),
    "cvr_probe_stream_read": (C.c_int, [C.c_void_p, C.c_int64, C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]),
    "cvr_probe_row_read": (C.c_int, [C.c_void_p, C.c_int64, C.c_int32, C.c_void_p, C.c_int64, C.c_void_p, C.c_int32,
                                     C.c_int32, C.c_void_p]),
    "cvr_last_error": (C.c_char_p, [C.c_void_p]),
    "cvr_status_string": (C.c_char_p, [C.c_int]),
    "cvr_destroy": (None, [C.c_void_p]),
}

_lib = None


def lib():
    """The loaded libcvr (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libcvr.so is not built ({LIB_PATH}); run cvr_ranking_model_amd.build")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _PROTOS.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


class CvrError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{lib().cvr_status_string(status).decode()}: {msg}")
        self.status = status


def _check(status, handle=None):
    if status != CVR_OK:
        raise CvrError(status, lib().cvr_last_error(handle).decode())


# ---- same-name wrappers of the C entry points (argument marshalling only) ----
def cvr_weight_arena_bytes(spec_c, tables_c, n_tables):
    out = C.c_size_t(0)
    _check(lib().cvr_weight_arena_bytes(C.byref(spec_c), tables_c, n_tables, C.byref(out)))
    return out.value


def cvr_create(spec_c, tables_c, n_tables, weights_c, n_weights, arena_ptr, arena_bytes, stream):
    h = C.c_void_p()
    _check(lib().cvr_create(C.byref(spec_c), tables_c, n_tables, weights_c, n_weights, arena_ptr, arena_bytes,
                            stream, C.byref(h)))
    return h


def cvr_workspace_bytes(h, max_requests, max_candidates, max_ids, max_positions):
    out = C.c_size_t(0)
    _check(lib().cvr_workspace_bytes(h, max_requests, max_candidates, max_ids, max_positions, C.byref(out)), h)
    return out.value


def cvr_score(h, batch_c, ws_ptr, ws_bytes, out_ptr, stream):
    _check(lib().cvr_score(h, C.byref(batch_c), ws_ptr, ws_bytes, out_ptr, stream), h)


def cvr_score_graph(h, batch_c, ws_ptr, ws_bytes, out_ptr, stream):
    _check(lib().cvr_score_graph(h, C.byref(batch_c), ws_ptr, ws_bytes, out_ptr, stream), h)


def cvr_graph_workspace_bytes(h, max_requests, max_candidates, max_ids, max_positions):
    out = C.c_size_t(0)
    _check(lib().cvr_graph_workspace_bytes(h, max_requests, max_candidates, max_ids, max_positions, C.byref(out)), h)
    return out.value


def cvr_graph_info(h):
    held, caps = C.c_int64(0), C.c_int64(0)
    _check(lib().cvr_graph_info(h, C.byref(held), C.byref(caps)), h)
    return held.value, caps.value


def cvr_score_noalloc(h, batch_c, out_ptr, stream):
    _check(lib().cvr_score_noalloc(h, C.byref(batch_c), out_ptr, stream), h)


CVR_NOALLOC_SCRATCH_BYTES = 64 << 20


def cvr_sync_status(h, stream):
    """Returns the status code (CVR_ERR_RANGE is a normal outcome to report, not an exception)."""
    st = lib().cvr_sync_status(h, stream)
    if st not in (CVR_OK, CVR_ERR_RANGE):
        _check(st, h)
    return st


def cvr_set_debug(h, debug):
    _check(lib().cvr_set_debug(h, int(debug)), h)


def cvr_set_option(h, option, value):
    _check(lib().cvr_set_option(h, int(option), int(value)), h)


def cvr_debug_export(h, what, dst_ptr, dst_bytes, stream):
    written = C.c_size_t(0)
    _check(lib().cvr_debug_export(h, what, dst_ptr, dst_bytes, C.byref(written), stream), h)
    return written.value


def cvr_cache_state_bytes(sets, ways, dim):
    out = C.c_size_t(0)
    _check(lib().cvr_cache_state_bytes(sets, ways, dim, C.byref(out)))
    return out.value


def cvr_cache_attach(h, table, sets, ways, state_ptr, state_bytes, stream):
    _check(lib().cvr_cache_attach(h, table, sets, ways, state_ptr, state_bytes, stream), h)


def cvr_cache_stats(h, table, stream):
    out = (C.c_int64 * 5)()
    _check(lib().cvr_cache_stats(h, table, out, stream), h)
    return list(out)


def cvr_cache_export(h, table, entries, stream):
    tags = np.empty(entries, np.int32)
    stamps = np.empty(entries, np.int32)
    _check(lib().cvr_cache_export(h, table, tags.ctypes.data_as(C.POINTER(C.c_int32)),
                                  stamps.ctypes.data_as(C.POINTER(C.c_int32)), stream), h)
    return tags, stamps


def cvr_timing_begin(h, max_calls, stage_mask=0):
    _check(lib().cvr_timing_begin(h, max_calls, stage_mask), h)


def cvr_timing_end(h):
    """Returns ({stage name: (ms_sum, launches)}, calls)."""
    n = 32
    ms = (C.c_double * n)()
    cnt = (C.c_int32 * n)()
    ns, nc = C.c_int32(0), C.c_int32(0)
    _check(lib().cvr_timing_end(h, ms, cnt, n, C.byref(ns), C.byref(nc)), h)
    return {cvr_stage_name(h, i): (ms[i], cnt[i]) for i in range(ns.value) if cnt[i]}, nc.value


def cvr_stage_name(h, i):
    return lib().cvr_stage_name(h, i).decode()


def cvr_fill_table(ptr, rows, dim, seed, halfwidth, stream):
    _check(lib().cvr_fill_table(ptr, rows, dim, C.c_uint64(seed & 0xFFFFFFFFFFFFFFFF), halfwidth, stream))


def cvr_probe_stream_read(src, nbytes, sink, blocks, stream, nontemporal=0):
    _check(lib().cvr_probe_stream_read(src, nbytes, sink, blocks, nontemporal, stream))


def cvr_probe_row_read(table, n_rows, row_bytes, ids, n_ids, sink, blocks, stream, nontemporal=0):
    _check(lib().cvr_probe_row_read(table, n_rows, row_bytes, ids, n_ids, sink, blocks, nontemporal, stream))


def cvr_destroy(h):
    lib().cvr_destroy(h)


# ---- conveniences on top of the ABI (memory and marshalling only) ----
def _torch():
    import torch
    return torch


def _stream_ptr(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return C.c_void_p(s.cuda_stream)


def spec_to_c(spec, tables):
    """Build the cvr_spec struct (plus the arrays it points to) from a spec dict."""
    feats = (cvr_feature * len(spec["features"]))(*[cvr_feature(f["table"], SIDES[f["side"]]) for f in spec["features"]])
    keep = [feats]
    s = cvr_spec()
    s.model = CVR_MODEL_DLRM if spec["model"] == "dlrm" else CVR_MODEL_HYFORMER
    s.lowp = CVR_LOWP_FP16 if spec["lowp"] == "fp16" else CVR_LOWP_BF16
    s.clamp = float(spec["clamp"])
    s.n_features = len(spec["features"])
    s.features = feats
    if spec["model"] == "dlrm":
        hid = (C.c_int32 * max(1, len(spec["mlp_hidden"])))(*spec["mlp_hidden"])
        keep.append(hid)
        s.n_hidden = len(spec["mlp_hidden"])
        s.hidden = hid
    else:
        cols = (C.c_int32 * len(spec["seq"]["columns"]))(*[c["table"] for c in spec["seq"]["columns"]])
        keep.append(cols)
        s.d, s.n_tokens, s.n_layers = spec["d"], spec["n_tokens"], spec["n_layers"]
        s.n_seq = len(spec["seq"]["lengths"])
        s.n_seq_cols = len(spec["seq"]["columns"])
        s.seq_tables = cols
        s.swiglu_hidden, s.tau = spec["swiglu_hidden"], float(spec["tau"])
        s.mixer_heads, s.mixer_hidden = spec["mixer_heads"], spec["mixer_hidden"]
        s.n_experts, s.expert_dim = spec["n_experts"], spec["expert_dim"]
        s.n_tasks, s.head_hidden = spec["n_tasks"], spec["head_hidden"]
        s.epnet_hidden = int(spec.get("epnet_hidden") or 0)
        if spec.get("ple_task_experts") is not None:
            E = spec["n_experts"]
            mask = [0] * (spec["n_tasks"] * E)
            for k, experts in enumerate(spec["ple_task_experts"]):
                for e in experts:
                    mask[k * E + e] = 1
            te = (C.c_int32 * len(mask))(*mask)
            keep.append(te)
            s.task_experts = te
    tabs = (cvr_table * len(tables))(*[cvr_table(t.data_ptr(), t.shape[0], t.shape[1]) for t in tables])
    keep.append(tabs)
    return s, tabs, keep


def device_tables(spec, variant="bench", device="cuda"):
    """Allocate the spec's fp32 tables on the GPU and fill them with the synthetic recipe."""
    torch = _torch()
    from . import synth
    out = []
    st = _stream_ptr()
    for rows, dim, seed, hw in synth.table_fill_params(spec, variant):
        t = torch.empty((rows, dim), dtype=torch.float32, device=device)
        cvr_fill_table(C.c_void_p(t.data_ptr()), rows, dim, seed, hw, st)
        out.append(t)
    return out


class DeviceBatch:
    """A batch packed on the host into one pinned int32 buffer and copied to the GPU once."""

    @staticmethod
    def _parts(batch):
        parts = [np.ascontiguousarray(batch["cand_offsets"], np.int32), np.ascontiguousarray(batch["bag_offsets"], np.int32),
                 np.ascontiguousarray(batch["ids"], np.int32)]
        has_seq = batch.get("seq_offsets") is not None
        if has_seq:
            parts += [np.ascontiguousarray(batch["seq_offsets"], np.int32).reshape(-1),
                      np.ascontiguousarray(batch["seq_ids"], np.int32).reshape(-1)]
        return parts, has_seq

    def __init__(self, batch, device="cuda", stream=None):
        torch = _torch()
        parts, has_seq = self._parts(batch)
        sizes = [p.size for p in parts]
        # 64-element (256-byte) aligned sections
        offs, total = [], 0
        for n in sizes:
            offs.append(total)
            total += (n + 63) // 64 * 64
        host = torch.empty(max(total, 64), dtype=torch.int32, pin_memory=True)
        hn = host.numpy()
        for p, o in zip(parts, offs):
            hn[o:o + p.size] = p.reshape(-1)
        self.host = host
        self._offs, self._sizes = offs, sizes
        self.dev = host.to(device, non_blocking=True)
        base = self.dev.data_ptr()
        self.c = cvr_batch()
        self.c.n_requests = len(parts[0]) - 1
        self.c.n_candidates = int(parts[0][-1])
        self.c.n_ids = int(parts[2].size)
        self.c.cand_offsets = base + 4 * offs[0]
        self.c.bag_offsets = base + 4 * offs[1]
        self.c.ids = base + 4 * offs[2]
        if has_seq:
            self.c.n_positions = int(np.asarray(batch["seq_ids"]).shape[0])
            self.c.seq_offsets = base + 4 * offs[3]
            self.c.seq_ids = base + 4 * offs[4]
        self.n_requests = self.c.n_requests
        self.n_candidates = self.c.n_candidates
        self.n_ids = self.c.n_ids
        self.n_positions = self.c.n_positions

    def refill(self, batch):
        """Copy another batch of exactly the same section sizes into the same device buffer
        (its pointers, and so a captured scoring graph, stay valid)."""
        parts, _ = self._parts(batch)
        if [p.size for p in parts] != self._sizes:
            raise ValueError("refill needs a batch with the same sizes")
        self.host.numpy()[:] = 0
        hn = self.host.numpy()
        for p, o in zip(parts, self._offs):
            hn[o:o + p.size] = p.reshape(-1)
        self.dev.copy_(self.host, non_blocking=True)


class Model:
    """A created model plus the device buffers it needs (weight arena, workspace, outputs)."""

    def __init__(self, spec, tables, weights, stream=None, device="cuda"):
        torch = _torch()
        self.spec = spec
        self.tables = tables
        self.device = device
        self.stream = stream
        self.n_tasks = 1 if spec["model"] == "dlrm" else spec["n_tasks"]
        self._spec_c, self._tabs_c, self._keep = spec_to_c(spec, tables)
        nbytes = cvr_weight_arena_bytes(self._spec_c, self._tabs_c, len(tables))
        self.arena = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        wdev = {k: torch.as_tensor(np.ascontiguousarray(v, np.float32)).to(device) for k, v in weights.items()}
        names = [k.encode() for k in wdev]
        wc = (cvr_weight * len(wdev))(*[cvr_weight(n, t.data_ptr(), t.numel()) for n, t in zip(names, wdev.values())])
        self.h = cvr_create(self._spec_c, self._tabs_c, len(tables), wc, len(wdev), C.c_void_p(self.arena.data_ptr()),
                            self.arena.numel(), _stream_ptr(stream))
        del wdev
        self.ws = None

    def workspace(self, R, n, n_ids, P):
        torch = _torch()
        need = cvr_workspace_bytes(self.h, R, n, n_ids, P)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws

    def attach_cache(self, table, sets, ways):
        """Serve ``table`` through an HBM hot-row cache of sets x ways rows (state held here)."""
        torch = _torch()
        # an out-of-range table index is reported by the library's own check
        dim = int(self.tables[table].shape[1]) if 0 <= table < len(self.tables) else 4
        nbytes = cvr_cache_state_bytes(sets, ways, dim) if ways >= 1 and sets >= 1 else 256
        state = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        cvr_cache_attach(self.h, table, sets, ways, C.c_void_p(state.data_ptr()), nbytes, _stream_ptr(self.stream))
        if not hasattr(self, "caches"):
            self.caches = {}
        self.caches[table] = (state, sets, ways)

    def cache_stats(self, table):
        """Counters since attach: lookups, hits, misses, admissions, evictions."""
        v = cvr_cache_stats(self.h, table, _stream_ptr(self.stream))
        return dict(zip(["lookups", "hits", "misses", "admissions", "evictions"], v))

    def cache_export(self, table):
        """The cache directory as (tags, stamps), each [sets, ways] int32."""
        _, sets, ways = self.caches[table]
        tags, stamps = cvr_cache_export(self.h, table, sets * ways, _stream_ptr(self.stream))
        return tags.reshape(sets, ways), stamps.reshape(sets, ways)

    def score(self, dbatch: DeviceBatch, out=None):
        torch = _torch()
        ws = self.workspace(dbatch.n_requests, dbatch.n_candidates, dbatch.n_ids, dbatch.n_positions)
        if out is None:
            out = torch.empty(max(1, dbatch.n_candidates * self.n_tasks), dtype=torch.float32, device=self.device)
        cvr_score(self.h, dbatch.c, C.c_void_p(ws.data_ptr()), ws.numel(), C.c_void_p(out.data_ptr()),
                  _stream_ptr(self.stream))
        return out

    def score_noalloc(self, dbatch: DeviceBatch, out=None):
        """cvr_score_noalloc on the model's stream: the library's own scratch array as workspace."""
        torch = _torch()
        if out is None:
            out = torch.empty(max(1, dbatch.n_candidates * self.n_tasks), dtype=torch.float32, device=self.device)
        cvr_score_noalloc(self.h, dbatch.c, C.c_void_p(out.data_ptr()), _stream_ptr(self.stream))
        return out

    def graph_workspace(self, R, n, n_ids, P):
        torch = _torch()
        need = cvr_graph_workspace_bytes(self.h, R, n, n_ids, P)
        if self.ws is None or self.ws.numel() < need:
            self.ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return self.ws

    def graph_info(self):
        """(graphs held, graphs captured since creation)."""
        return cvr_graph_info(self.h)

    def score_graph(self, dbatch: DeviceBatch, out=None, ws_sizes=None):
        """cvr_score_graph on the model's stream (or a private one ordered after the current
        stream: graph capture needs a created stream).  ws_sizes: (R, n, ids, P) to size the
        workspace for (default: this batch's own)."""
        torch = _torch()
        sizes = ws_sizes or (dbatch.n_requests, dbatch.n_candidates, dbatch.n_ids, dbatch.n_positions)
        ws = self.graph_workspace(*sizes)
        if out is None:
            out = torch.empty(max(1, dbatch.n_candidates * self.n_tasks), dtype=torch.float32, device=self.device)
        s = self.stream
        if s is None:
            if getattr(self, "_gstream", None) is None:
                self._gstream = torch.cuda.Stream()
            s = self._gstream
            s.wait_stream(torch.cuda.current_stream())
        cvr_score_graph(self.h, dbatch.c, C.c_void_p(ws.data_ptr()), ws.numel(), C.c_void_p(out.data_ptr()),
                        C.c_void_p(s.cuda_stream))
        if self.stream is None:
            torch.cuda.current_stream().wait_stream(s)
        return out

    def sync_status(self):
        return cvr_sync_status(self.h, _stream_ptr(self.stream))

    def set_debug(self, on=True):
        cvr_set_debug(self.h, 1 if on else 0)

    def set_option(self, option, value):
        cvr_set_option(self.h, option, value)

    def export(self, what, dtype, shape):
        torch = _torch()
        dst = torch.empty(shape, dtype=dtype, device=self.device)
        n = cvr_debug_export(self.h, what, C.c_void_p(dst.data_ptr()), dst.numel() * dst.element_size(),
                             _stream_ptr(self.stream))
        assert n <= dst.numel() * dst.element_size()
        return dst

    def stage_names(self):
        """Stage names in cvr_stage_name order (bit s of a timing mask is stage s)."""
        names = []
        while True:
            nm = cvr_stage_name(self.h, len(names))
            if not nm:
                return names
            names.append(nm)

    def timing_begin(self, max_calls, stages=None):
        """Arm per-stage event timing for the next max_calls scoring calls; stages: names of
        the stages to time (None = all of them)."""
        mask = 0
        if stages:
            names = self.stage_names()
            for st in stages:
                mask |= 1 << names.index(st)
        cvr_timing_begin(self.h, max_calls, mask)

    def timing_end(self):
        return cvr_timing_end(self.h)

    def close(self):
        if getattr(self, "h", None):
            cvr_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
