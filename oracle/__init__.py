"""CPU oracle for the candidate-scoring forward pass — TEST INFRASTRUCTURE ONLY.

A plain, slow, obviously-correct numpy implementation of what the two source
articles define:

* "广告 CTR 预估模型的 GPU 推理优化" (GPU inference optimisation for ad CTR
  models; cited below as *the CTR article*): mean-pooled fp32 embeddings,
  clamp to +-10, fp16 MLP of 3-5 x 1024 over the candidates, fp32 output.
* The iQIYI article on moving its ad CVR model to PyTorch + GPU inference
  (cited below as *the CVR article*): per-sequence SwiGLU encoding, Query
  Decoding with three temperature-scaled cross-attention queries, Query
  Boosting by a Split -> Mixing -> Reverting token mixer, PLE experts and
  two-layer heads, BF16 inference.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the GPU path:
its inputs come from the seeded generators (which hold none of the method's
arithmetic) and from hand-built test cases.

Precision.  The pages fix the precision of the deployed method: fp32
embeddings, fp16 (CTR article, section 三) or BF16 (CVR article, section
3.4.3) for the dense network, fp32 output.  The oracle therefore pools in fp32
exactly as defined, rounds to the low-precision type at the points where the
method hands a tensor to a dense operator (see :mod:`oracle.lowp`), and does
all other arithmetic in fp64.  ``exact=True`` removes the low-precision
rounding (fp64 throughout after pooling) to show what the reduced precision
costs.

Every function here has at least one pin in ``tests/test_oracle_*.py`` that
does not re-derive it from its own formula.
"""
from .common import expand, pool_bags, candidate_inputs, OracleInputError
from .dlrm import dlrm_forward
from .hyformer import hyformer_forward, token_mix, token_revert


def score(spec, tables, weights, batch, requests=None, exact=False, trace=False, accumulate="fp64"):
    """Score a batch (or a subset of its requests) with the model the spec names.
    ``accumulate`` (CVR model only): "fp64" (default) or "fp32" sums in every Linear."""
    if spec["model"] == "dlrm":
        return dlrm_forward(spec, tables, weights, batch, requests=requests, exact=exact)
    if spec["model"] == "hyformer":
        return hyformer_forward(spec, tables, weights, batch, requests=requests, exact=exact, trace=trace,
                                accumulate=accumulate)
    raise OracleInputError(f"unknown model {spec['model']!r}")


__all__ = ["score", "expand", "pool_bags", "candidate_inputs", "dlrm_forward", "hyformer_forward",
           "token_mix", "token_revert", "OracleInputError"]
