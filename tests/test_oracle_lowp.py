"""Pins for the oracle's low-precision rounding (round to nearest, ties to even)."""
import numpy as np
import torch

from oracle.lowp import round_bf16, round_fp16, rounder


def _bf16_bits_rne(x32):
    """fp32 -> bf16 by integer rounding on the bit pattern (a different route to the same definition)."""
    u = np.asarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return (r << np.uint64(16)).astype(np.uint32).view(np.float32).astype(np.float64)


def test_bf16_known_values():
    e = 2.0 ** -7  # bf16 spacing just above 1
    cases = {
        1.0: 1.0,
        1.0 + e / 2: 1.0,                   # tie, 1.0 has the even significand
        1.0 + 1.5 * e: 1.0 + 2 * e,          # tie, rounds up to the even neighbour
        1.0 + e / 2 + 2.0 ** -30: 1.0 + e,   # just above the tie
        -(1.0 + 1.5 * e): -(1.0 + 2 * e),
        0.0: 0.0,
        3.0: 3.0,
        255.5: 256.0,                        # 8 significant bits: 255 | 256 spacing 1 .. tie to even
        254.5: 254.0,
    }
    for x, want in cases.items():
        assert round_bf16(x) == want, (x, round_bf16(x), want)


def test_bf16_matches_bit_rounding_and_torch(rng):
    x = rng.standard_normal(200_000).astype(np.float32) * np.float32(3.0) ** rng.integers(-20, 20, 200_000).astype(np.float32)
    a = round_bf16(x.astype(np.float64))
    b = _bf16_bits_rne(x)
    c = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(a, b)
    assert np.array_equal(a, c)


def test_bf16_rounds_fp64_directly():
    # a value just above a bf16 tie whose fp32 rounding lands exactly on the tie
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert round_bf16(x) == 1.0 + 2.0 ** -7


def test_fp16_known_values():
    e = 2.0 ** -10
    assert round_fp16(1.0 + e / 2) == 1.0
    assert round_fp16(1.0 + 1.5 * e) == 1.0 + 2 * e
    assert round_fp16(1.0 + e / 2 + 2.0 ** -40) == 1.0 + e   # direct from fp64, not via fp32
    assert round_fp16(65504.0) == 65504.0
    assert round_fp16(10.0) == 10.0 and round_fp16(-10.0) == -10.0
    assert round_fp16(2.0 ** -24) == 2.0 ** -24              # smallest subnormal
    assert round_fp16(2.0 ** -26) == 0.0


def test_fp16_matches_torch_on_fp32_inputs(rng):
    # torch converts fp64 to fp16 through fp32 (double rounding), so compare on fp32 inputs only
    x = rng.uniform(-12, 12, 100_000).astype(np.float32)
    want = torch.from_numpy(x).to(torch.float16).to(torch.float64).numpy()
    assert np.array_equal(round_fp16(x.astype(np.float64)), want)


def test_rounder_exact_is_identity(rng):
    x = rng.standard_normal(100)
    assert np.array_equal(rounder("bf16", exact=True)(x), x)
    assert np.array_equal(rounder("fp16")(x), round_fp16(x))
