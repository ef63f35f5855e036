"""DLRM-style candidate scoring (oracle side), after the CTR article.

The CTR article ("广告 CTR 预估模型的 GPU 推理优化") scores every candidate
item of an ad request with one MLP of 3-5 layers x 1024 units over the
concatenated embeddings (section 三), batching all candidates through shared
weights (section 四).  Readings for what it leaves open:

* every Linear has a bias; ReLU follows every hidden Linear and none follows
  the final 1024 -> 1 Linear;
* the prediction is the logistic sigmoid of that last Linear, in fp32
  (section 三: the MLP's CTR output is FP32);
* fp16 holds the MLP's input activations and weights (section 三); see
  :mod:`oracle.lowp` for where rounding happens.
"""
import numpy as np

from .common import expand, candidate_inputs, sigmoid, requests_to_candidates, OracleInputError
from .lowp import rounder


def mlp_layers(spec):
    return len(spec["mlp_hidden"]) + 1


def dlrm_forward(spec, tables, weights, batch, requests=None, exact=False):
    """Steps A0-A4 for all candidates (or those of the listed requests).

    Returns a dict with ``scores`` (fp32), ``logits`` (fp64), ``inputs`` (the
    fp64 MLP input rows), ``hidden`` (the last hidden layer's activations),
    ``pooled`` (fp32 per feature), ``cand`` (global candidate indices scored)
    and the expansion ``ex``.
    """
    if spec["model"] != "dlrm":
        raise OracleInputError("not a DLRM spec")
    rnd = rounder(spec["lowp"], exact)
    ex = expand(spec, batch)
    cands = requests_to_candidates(ex, requests)
    x, pooled = candidate_inputs(spec, tables, ex, cands, rnd)
    h = x
    hidden = None
    L = mlp_layers(spec)
    for i in range(L):
        W = rnd(np.asarray(weights[f"mlp.{i}.weight"], dtype=np.float32).astype(np.float64))
        b = np.asarray(weights[f"mlp.{i}.bias"], dtype=np.float32).astype(np.float64)
        if W.shape[1] != h.shape[1]:
            raise OracleInputError(f"mlp.{i}.weight expects {W.shape[1]} inputs, got {h.shape[1]}")
        y = h @ W.T + b
        if i < L - 1:
            h = rnd(np.maximum(y, 0.0))
            hidden = h
        else:
            z = y[:, 0]
    scores = sigmoid(z).astype(np.float32)
    return {"scores": scores, "logits": z, "inputs": x, "hidden": hidden, "pooled": pooled,
            "cand": cands, "ex": ex}
