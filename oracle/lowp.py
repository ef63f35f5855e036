"""Rounding to the dense network's low-precision types (oracle side).

The CTR article (section 三, mixed precision) casts the looked-up embeddings
to FP16 after the +-10 clamp and runs the MLP with FP16 input activations and
FP16 weights, returning an FP32 prediction.  The CVR article (section 3.4.3)
runs the dense network in BF16.  Neither page states a rounding mode; the
reading taken is round-to-nearest-even, the IEEE default.

Reading of where rounding happens: every Linear weight matrix and every
Linear input is in the low-precision type.  In the DLRM-style model that is
every hidden activation (the CTR article names the MLP's input activations as
FP16).  In the CVR model the encoded sequence states, which are stored and
read back by the attention, are also low precision; the other per-candidate
tensors that are not Linear inputs stay at full precision (see
:mod:`oracle.hyformer`).  Arithmetic inside an operator (dot-product
accumulation, bias, activation function, softmax, pooling sums, residual add)
is at least fp32 — here fp64.  Biases stay fp32.  The embedding pooling
before the cast and the final probabilities are fp32.

Values are returned as fp64 arrays holding exactly representable
low-precision numbers, so the rest of the oracle can keep computing in fp64.
"""
import numpy as np


def round_fp16(x):
    """Round to the nearest IEEE binary16 value, ties to even (numpy's direct fp64->fp16 cast)."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).astype(np.float64)


def round_bf16(x):
    """Round to the nearest bfloat16 value, ties to even.

    bfloat16 keeps 8 significant bits and fp32's exponent range.  A normal
    value ``m * 2**e`` (``0.5 <= |m| < 1``) is rounded by scaling ``m`` to
    ``[128, 256)``, rounding to an integer (``np.rint`` rounds half to even)
    and scaling back.  Below fp32's smallest normal the spacing is the fixed
    subnormal quantum ``2**-133``.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    normal = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = np.rint(np.ldexp(x, 133)) * 2.0 ** -133
    return np.where(np.abs(x) < 2.0 ** -126, sub, normal)


def rounder(lowp: str, exact: bool = False):
    """The rounding function for a spec's ``lowp`` field (identity when ``exact``)."""
    if exact:
        return lambda x: np.asarray(x, dtype=np.float64)
    if lowp == "fp16":
        return round_fp16
    if lowp == "bf16":
        return round_bf16
    raise ValueError(f"unknown low-precision type {lowp!r}")
