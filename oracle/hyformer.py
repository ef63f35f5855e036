"""The CVR model of the iQIYI article (oracle side).

The CVR article (section 3.2) builds the model in three levels: feature
input, feature interaction (HyFormer-style Query Decoding and Query Boosting)
and multi-task prediction (PLE experts with MLP heads).  The article's
tokenization formula and both figures were lost from the page; the readings
taken for every open point are listed with the function that applies them.

Precision (section 3.4.3 runs the dense network in BF16 to cut memory traffic
and compute).  Reading: ``rnd`` rounds to bf16 every Linear weight matrix and
every Linear *input*, and the encoded sequence states, which are stored once
and read again by the attention; the small per-candidate tensors that are not
Linear inputs (tokens and their residual stream, queries, attention outputs,
expert outputs, gate values) stay at full precision.  Rounding those as well
made two bf16 evaluations of the same model that differ only in summation
order disagree by up to 6e-3 on stress-data scores, so this reading is the one
that keeps the method reproducible to the scores' tolerance.
"""
import numpy as np

from .common import expand, candidate_inputs, clamp, sigmoid, requests_to_candidates, OracleInputError
from .lowp import rounder


def matmul64(a, b):
    """A Linear's products summed in fp64 (the oracle's default)."""
    return np.asarray(a, dtype=np.float64) @ np.asarray(b, dtype=np.float64)


def matmul32(a, b):
    """The same products summed in fp32.  The operands are low-precision values, so every
    product is exact in fp32 and only the summation is rounded: this is what a device that
    accumulates in fp32 computes, up to the order of its additions.  Used to measure how far
    two valid evaluations of the precision plan can sit apart."""
    return (np.asarray(a, dtype=np.float32) @ np.asarray(b, dtype=np.float32)).astype(np.float64)


def _w(weights, name, rnd):
    return rnd(np.asarray(weights[name], dtype=np.float32).astype(np.float64))


def _b(weights, name):
    return np.asarray(weights[name], dtype=np.float32).astype(np.float64)


def silu(x):
    """SiLU(x) = x * sigmoid(x), the gate nonlinearity of SwiGLU."""
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def softmax(x, axis=-1):
    """Softmax with the row maximum subtracted first (same value, no overflow)."""
    x = np.asarray(x, dtype=np.float64)
    m = np.max(x, axis=axis, keepdims=True)
    e = np.exp(x - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def domain_columns(spec):
    """Columns of the model input that hold the scenario (domain) features: the context-side
    features, in spec order."""
    cols, c = [], 0
    for f in spec["features"]:
        dim = spec["tables"][f["table"]]["dim"]
        if f["side"] == "context":
            cols.extend(range(c, c + dim))
        c += dim
    return np.array(cols, dtype=np.int64)


def epnet(spec, weights, e, rnd, mm=matmul64):
    """Optional step before B2: EPNet, the scenario-aware non-sequence embedding.

    The CVR article (section 3.2.1) obtains the non-sequence embedding through EPNet, which
    models several scenarios, but prints no formula.  Reading: EPNet as PEPNet defines it
    (Chang et al., KDD 2023): a gate unit turns the scenario features' embedding, concatenated
    with the general embedding, into a per-element scale delta = gamma * sigmoid(W2 ReLU(W1
    [e_domain, e] + b1) + b2) with gamma = 2, and the general embedding is multiplied by it
    element by element.  The scenario features are the spec's context-side features; the gate's
    hidden width is the spec's ``epnet_hidden``.  Both gate Linears take low-precision inputs,
    and the scaled embedding, the tokenizer's input, is rounded again.  ``e`` is [c, D].
    """
    x = rnd(np.concatenate([e[:, domain_columns(spec)], e], axis=1))
    h = rnd(np.maximum(mm(x, _w(weights, "epnet.fc1.weight", rnd).T) + _b(weights, "epnet.fc1.bias"), 0.0))
    g = mm(h, _w(weights, "epnet.fc2.weight", rnd).T) + _b(weights, "epnet.fc2.bias")
    with np.errstate(over="ignore"):             # exp(-g) = inf for g << 0 gives delta = 0
        delta = 2.0 / (1.0 + np.exp(-g))
    return rnd(delta * e)


def tokenize(spec, weights, e, rnd, mm=matmul64):
    """Step B2: non-sequence tokens.

    The CVR article (sections 3.2.2-3.2.3) splits the concatenated user, item
    and context embedding "in latent space" into N heads; the formula itself
    is missing from the page.  Reading: one Linear from the concatenated
    embedding to N*d outputs (with bias, no activation), reshaped row-major to
    N tokens of width d (token i = outputs i*d .. i*d+d-1).  A plain split
    cannot work: 1280 input columns do not divide into 13 tokens of 128.
    """
    N, d = spec["n_tokens"], spec["d"]
    y = mm(e, _w(weights, "tok.weight", rnd).T) + _b(weights, "tok.bias")
    return y.reshape(e.shape[0], N, d)


def sequence_rows(spec, tables, ex, s, requests):
    """Step B3 (gather): the per-position embedding of sequence group ``s``.

    The CVR article (section 3.2.1) represents each behaviour as the concat of
    its item-ID, action-type, timestamp and side-info embeddings; the three
    sequences share the underlying tables and are assembled per group.
    Returns fp32 rows for the positions of ``requests`` (in request order) and
    the per-request lengths.
    """
    so = ex["seq_offsets"]
    pos = [np.arange(so[s, r], so[s, r + 1], dtype=np.int64) for r in requests]
    lens = np.array([p.size for p in pos], dtype=np.int64)
    pos = np.concatenate(pos) if pos else np.zeros(0, dtype=np.int64)
    cols = [np.asarray(tables[c["table"]][ex["seq_ids"][pos, ci]], dtype=np.float32).reshape(pos.size, -1)
            for ci, c in enumerate(spec["seq"]["columns"])]
    return np.concatenate(cols, axis=1), lens


def swiglu(weights, s, E, rnd, mm=matmul64):
    """Step B4: the per-position SwiGLU encoder of sequence ``s``.

    The CVR article (sections 3.2.2-3.2.3) maps each of the three sequences
    into the common latent space with its own SwiGLU network, position by
    position.  Reading: H = W_down (SiLU(W_gate e + b_gate) * (W_up e + b_up))
    + b_down, no residual and no normalisation.  The product is the input of
    the down projection, so it is rounded to the low-precision type.
    """
    g = mm(E, _w(weights, f"seq.{s}.gate.weight", rnd).T) + _b(weights, f"seq.{s}.gate.bias")
    u = mm(E, _w(weights, f"seq.{s}.up.weight", rnd).T) + _b(weights, f"seq.{s}.up.bias")
    a = rnd(silu(g) * u)
    return rnd(mm(a, _w(weights, f"seq.{s}.down.weight", rnd).T) + _b(weights, f"seq.{s}.down.bias"))


def mean_pool(H):
    """Step B5: the sequence's mean ("uniform pooling") vector; zero for an empty sequence."""
    if H.shape[0] == 0:
        return np.zeros(H.shape[1])
    return H.sum(axis=0) / H.shape[0]


def query(weights, l, s, X, p, rnd, mm=matmul64):
    """Step B6: one global query per sequence.

    The CVR article (section 3.2.3, Query Decoding) concatenates the N
    non-sequence tokens with the sequence's pooled vector and feeds them to
    "one FFN layer" producing one query token, with separate parameters per
    sequence.  Reading: a single Linear (N+1)*d -> d with bias, no
    activation, separate per sequence and per stacked layer.
    ``X`` is [c, N, d], ``p`` is [c, d].
    """
    inp = rnd(np.concatenate([X.reshape(X.shape[0], -1), p], axis=1))
    return mm(inp, _w(weights, f"layer.{l}.query.{s}.weight", rnd).T) + _b(weights, f"layer.{l}.query.{s}.bias")


def cross_attention(H, q, tau, rnd, mm=matmul64):
    """Step B7: one query attending over one sequence's hidden states.

    The CVR article (section 3.2.3) takes the SwiGLU-encoded states directly
    as keys and values and scales the dot products by a temperature chosen so
    the softmax does not collapse to one-hot.  Reading: single head, no key or
    value projection, weights = softmax(H q / tau) over the valid positions,
    output = sum_t weight_t H[t].  An empty sequence gives a zero output.
    Returns (output, weights).
    """
    if H.shape[0] == 0:
        return np.zeros(H.shape[1]), np.zeros(0)
    a = softmax(mm(H, q) / tau)
    return mm(a, H), a


def token_mix(Y, heads):
    """Split -> Mixing of the token mixer (step B8).

    The CVR article (section 3.2.3, Query Boosting) sends the N+3 tokens
    through a TokenMixer-Large-style Split -> Mixing -> Reverting block in
    which every token interacts with every other.  Reading: split each token
    of width d into ``heads`` chunks of width w = d/heads; mixed token h is the
    concat, over tokens t in order, of chunk h of token t:
    ``M[h, t*w + j] = Y[t, h*w + j]``.  ``Y`` is [..., T, d].
    """
    T, d = Y.shape[-2], Y.shape[-1]
    if d % heads:
        raise OracleInputError("token width must divide into the mixer heads")
    w = d // heads
    lead = Y.shape[:-2]
    return Y.reshape(lead + (T, heads, w)).swapaxes(-3, -2).reshape(lead + (heads, T * w))


def token_revert(F, tokens):
    """Reverting: the inverse of :func:`token_mix`, ``R[t, h*w + j] = F[h, t*w + j]``."""
    Hh, Tw = F.shape[-2], F.shape[-1]
    w = Tw // tokens
    lead = F.shape[:-2]
    return F.reshape(lead + (Hh, tokens, w)).swapaxes(-3, -2).reshape(lead + (tokens, Hh * w))


def mixer(spec, weights, l, Y, rnd, mm=matmul64):
    """Step B8: Z = Y + Revert(FFN_h(Mix(Y)_h)) for one stacked layer.

    Reading: one FFN per mixed token (Linear -> ReLU -> Linear with biases,
    hidden width ``mixer_hidden``), separate weights per mixed token; the
    residual add follows the revert, no normalisation.  ``Y`` is [c, T, d].
    """
    H = spec["mixer_heads"]
    M = rnd(token_mix(Y, H))
    F = np.empty_like(M)
    for h in range(H):
        hid = rnd(np.maximum(mm(M[:, h, :], _w(weights, f"layer.{l}.mix.{h}.fc1.weight", rnd).T)
                             + _b(weights, f"layer.{l}.mix.{h}.fc1.bias"), 0.0))
        F[:, h, :] = mm(hid, _w(weights, f"layer.{l}.mix.{h}.fc2.weight", rnd).T) + _b(weights, f"layer.{l}.mix.{h}.fc2.bias")
    return Y + token_revert(F, Y.shape[1])


def task_experts(spec):
    """Experts mixed by each task's gate: every expert (shared experts only) unless the spec
    lists them per task (PLE with task-specific experts)."""
    lists = spec.get("ple_task_experts")
    if lists is None:
        return [list(range(spec["n_experts"])) for _ in range(spec["n_tasks"])]
    return [sorted(int(e) for e in lst) for lst in lists]


def ple_heads(spec, weights, z, rnd, mm=matmul64):
    """Steps B10-B11: PLE experts, per-task gates and two-layer heads.

    The CVR article (section 3.2.4) predicts each scenario's pCVR with
    PLE + MLP heads: three experts that are single fully-connected layers and
    heads of two fully-connected layers with a nonlinearity; section 3.2 also
    calls the prediction level an MMoE-style expert structure.  Reading: the
    experts are ReLU(Linear) layers; each task mixes a set of them with its
    own softmax gate (a Linear with one output per expert in its set), and
    each head is Linear -> ReLU -> Linear -> sigmoid, the sigmoid in fp32.
    By default every task mixes all experts — single-level PLE with shared
    experts only, which is exactly MMoE.  With ``ple_task_experts`` a task
    mixes only the listed experts, e.g. its own task-specific expert plus a
    shared one (PLE proper).
    ``z`` is the flattened last-layer token matrix [c, T*d].
    Returns (logits [c, tasks], gated task inputs list).
    """
    E = spec["n_experts"]
    z = rnd(z)
    experts = [np.maximum(mm(z, _w(weights, f"ple.expert.{e}.weight", rnd).T) + _b(weights, f"ple.expert.{e}.bias"), 0.0)
               for e in range(E)]
    logits, tin = [], []
    for k, mixed in enumerate(task_experts(spec)):
        g = softmax(mm(z, _w(weights, f"ple.gate.{k}.weight", rnd).T) + _b(weights, f"ple.gate.{k}.bias"))
        t = rnd(sum(g[:, i:i + 1] * experts[e] for i, e in enumerate(mixed)))
        u = rnd(np.maximum(mm(t, _w(weights, f"head.{k}.fc1.weight", rnd).T) + _b(weights, f"head.{k}.fc1.bias"), 0.0))
        y = mm(u, _w(weights, f"head.{k}.fc2.weight", rnd).T) + _b(weights, f"head.{k}.fc2.bias")
        logits.append(y[:, 0])
        tin.append(t)
    return np.stack(logits, axis=1), tin


def hyformer_forward(spec, tables, weights, batch, requests=None, exact=False, trace=False, accumulate="fp64"):
    """Steps B0-B11 for all candidates (or those of the listed requests).

    Sequences belong to the request (the user's behaviour); every candidate of
    a request attends to the same encoded sequences.  Layers stack like
    decoder layers (CVR article, section 3.2.3): layer l+1 takes the first N
    tokens of layer l's output as its non-sequence tokens, the encoded
    sequences and their pooled vectors are shared by all layers, and the
    prediction level reads the last layer's full token matrix.

    ``accumulate="fp32"`` sums every Linear's (and the attention's) products in fp32 instead
    of fp64 (see :func:`matmul32`); the default is fp64.

    Returns ``scores`` fp32 [c, tasks], ``logits`` fp64 [c, tasks], ``cand``;
    with ``trace`` also the intermediates (``e_in`` the pooled inputs, ``e`` the tokenizer's
    input (``e_in`` scaled by EPNet when the spec has it), ``X0``, ``H``, ``p``, ``q``, ``o``,
    ``Z``, ``attn``).
    """
    if spec["model"] != "hyformer":
        raise OracleInputError("not a CVR spec")
    rnd = rounder(spec["lowp"], exact)
    if accumulate not in ("fp64", "fp32"):
        raise OracleInputError("accumulate must be fp64 or fp32")
    mm = matmul32 if accumulate == "fp32" else matmul64
    ex = expand(spec, batch)
    R = ex["R"]
    reqs = list(range(R)) if requests is None else [int(r) for r in requests]
    cands = requests_to_candidates(ex, reqs)
    cand_req = ex["cand_req"][cands].astype(np.int64)
    S = len(spec["seq"]["lengths"])
    d, N = spec["d"], spec["n_tokens"]
    tau = float(spec["tau"])

    # B1-B2: non-sequence input and tokens, per candidate.
    e_in, pooled = candidate_inputs(spec, tables, ex, cands, rnd)
    e = epnet(spec, weights, e_in, rnd, mm) if spec.get("epnet_hidden") else e_in
    X = tokenize(spec, weights, e, rnd, mm)

    # B3-B5: per request and sequence.
    Hs, ps = {}, {}
    for s in range(S):
        rows, lens = sequence_rows(spec, tables, ex, s, reqs)
        Eseq = rnd(clamp(rows, spec["clamp"]).astype(np.float64))
        Hall = swiglu(weights, s, Eseq, rnd, mm) if rows.shape[0] else np.zeros((0, d))
        off = np.concatenate([[0], np.cumsum(lens)])
        for i, r in enumerate(reqs):
            Hs[(s, r)] = Hall[off[i]:off[i + 1]]
            ps[(s, r)] = mean_pool(Hs[(s, r)])

    tr = {"e_in": e_in, "e": e, "X0": X.copy(), "H": Hs, "p": ps, "q": [], "o": [], "Z": [], "attn": [], "pooled": pooled}
    nc = cands.size
    Z = None
    for l in range(spec["n_layers"]):
        outs = []
        ql, al = [], []
        for s in range(S):
            p = np.stack([ps[(s, int(r))] for r in cand_req]) if nc else np.zeros((0, d))
            q = query(weights, l, s, X, p, rnd, mm)
            o = np.zeros((nc, d))
            att = []
            for i in range(nc):
                o[i], a = cross_attention(Hs[(s, int(cand_req[i]))], q[i], tau, rnd, mm)
                att.append(a)
            outs.append(o)
            ql.append(q)
            al.append(att)
        Y = np.concatenate([X, np.stack(outs, axis=1)], axis=1)
        Z = mixer(spec, weights, l, Y, rnd, mm)
        X = Z[:, :N, :]
        tr["q"].append(ql)
        tr["o"].append(outs)
        tr["Z"].append(Z)
        tr["attn"].append(al)
    logits, tin = ple_heads(spec, weights, Z.reshape(nc, -1), rnd, mm)
    tr["task_in"] = tin
    out = {"scores": sigmoid(logits).astype(np.float32), "logits": logits, "cand": cands, "ex": ex}
    if trace:
        out["trace"] = tr
    return out
