"""How far the precision plan may sit from exact arithmetic: the bound the oracle's own pins and
the GPU parity tests share.

Each rounding site perturbs its tensor by a relative error of at most u (u = 2^-8 for bf16,
2^-11 for fp16: half the spacing of the format's 8 or 11 significant bits, relative to the low
end of a binade), roughly uniform and independent between sites.  A Linear over such inputs and
weights moves its output by about u * sqrt(2/3) * rms of the output per rounded pair, and
well-conditioned layers (Glorot weights, ReLU) carry earlier perturbations forward at about the
same relative size, so a logit's error behaves like a sum of independent terms over the rounding
sites on its path: std ~ 0.82 u sqrt(sites) rms(z).  The maximum over a batch of a few hundred
such errors stays within ~3.5 std.  Bound: 4 u kappa sqrt(sites) rms(z).

kappa is the condition of the attention (1 where there is none).  Its output o = sum_t a_t H_t
with a = softmax(s) moves by do = sum_t a_t (H_t - o) ds_t + sum_t a_t dH_t, so a relative
perturbation of the scores s_t = H_t.q / tau reaches o multiplied by about the weight-averaged
spread of the scores, sigma_a(s) = sqrt(sum_t a_t (s_t - sum a s)^2).  kappa = 1 + the largest
sigma_a(s) over the batch's attentions, read off the exact oracle's weights (log a_t = s_t minus a
constant).  Sharp attention (the stress data's gain-3 encoders and queries) has kappa near 3-4.

It does not cover a softmax that has become one-hot: there sigma_a(s) is near zero, yet a rounding
can move the argmax between nearly tied positions and change the output by the difference of two
whole rows.  The clamp data set (tables U(-50, 50), every embedding at the +-10 clamp) drives the
CVR model's attention there, so the CVR model is held to this bound on its other data sets only.
"""
import math

import numpy as np


def unit_roundoff(spec):
    return 2.0 ** -11 if spec["lowp"] == "fp16" else 2.0 ** -8


def rounding_sites(spec):
    """Rounded tensors on the path to a logit: weights and inputs of every Linear, plus the
    stored sequence states (CVR)."""
    if spec["model"] == "dlrm":
        return 2 * (len(spec["mlp_hidden"]) + 1)
    # inputs + tokenizer weight; sequence row + gate|up weights + SwiGLU product + down weights +
    # states; per layer: query input + weights, mixed tokens + fc1, hidden + fc2; then z + expert
    # and gate weights, task input + fc1, head hidden + fc2
    return 2 + 5 + 6 * spec["n_layers"] + 7


def attention_condition(spec, trace):
    """kappa from the attention weights of an oracle trace (1 for the DLRM model)."""
    if spec["model"] == "dlrm" or trace is None:
        return 1.0
    worst = 0.0
    for layer in trace["attn"]:
        for per_seq in layer:
            for a in per_seq:
                if np.size(a) < 2:
                    continue
                ls = np.log(np.maximum(a, 1e-300))
                mu = float(np.sum(a * ls))
                worst = max(worst, float(np.sqrt(np.sum(a * (ls - mu) ** 2))))
    return 1.0 + worst


def exact_bound(spec, z_exact, trace=None):
    """Bound on |z - z_exact| for the rounding plan; ``trace``: the exact oracle's trace (CVR)."""
    rms = float(np.sqrt(np.mean(np.square(z_exact)))) if np.size(z_exact) else 0.0
    kappa = attention_condition(spec, trace)
    return 4.0 * unit_roundoff(spec) * kappa * math.sqrt(rounding_sites(spec)) * rms
