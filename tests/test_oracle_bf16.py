"""Pins for the oracle's bf16 rounding (round to nearest, ties to even).

float -> bf16 is checked against torch's own conversion over random and edge bit patterns.
double -> bf16 (one rounding) is checked against exact rational arithmetic: the two bf16
neighbours of x are found exactly and the nearer one (the even one on a tie) is expected.
"""
from fractions import Fraction
import math
import struct

import numpy as np
import torch


def _torch_bf16_bits(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_matches_torch(oracle):
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2**32, size=400_000, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=50_000, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    near = np.concatenate([ties - 1, ties + 1])
    special = np.array([0, 0x80000000, 0x7F7FFFFF, 0x7F7F8000, 0x7F7F7FFF, 0x00000001, 0x00008000,
                        0x00018000, 0x007FFFFF, 0x7F800000, 0xFF800000], dtype=np.uint32)
    allbits = np.concatenate([bits, ties, near, special]).astype(np.uint32)
    x = allbits.view(np.float32)
    finite = np.isfinite(x) | np.isinf(x)
    got = oracle.f32_to_bf16(x[finite])
    ref = _torch_bf16_bits(x[finite].copy())
    np.testing.assert_array_equal(got, ref)
    nan = oracle.f32_to_bf16(np.array([np.nan], np.float32))[0]
    assert (nan & 0x7F80) == 0x7F80 and (nan & 0x7F) != 0


def _bf16_value(h: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", (h & 0xFFFF) << 16))[0])


def _exact_rne_bf16(x: float) -> int:
    """Nearest bf16 to the double x by exhaustive comparison of its two neighbours."""
    fx = Fraction(x)
    # candidate from truncation of the float nearest below (in magnitude) and its successor
    f = np.float32(x)
    h = int(np.array([f], np.float32).view(np.uint32)[0] >> 16)
    cands = {h, (h + 1) & 0xFFFF, (h - 1) & 0xFFFF}
    best = None
    for c in cands:
        if (c & 0x7F80) == 0x7F80:
            continue
        v = _bf16_value(c)
        if (v < 0) != (fx < 0) and v != 0:
            continue
        err = abs(v - fx)
        key = (err, c & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return best[1]


def test_f64_to_bf16_single_rounding(oracle):
    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000)))
    # exact ties and near-ties in double that a double-then-float rounding would get wrong
    for _ in range(500):
        h = int(rng.integers(0x0080, 0x7F00))
        lo, hi = _bf16_value(h), _bf16_value(h + 1)
        mid = (lo + hi) / 2
        vals += [float(mid), float(mid) * (1 + 2**-40), float(mid) * (1 - 2**-40)]
        vals += [-float(mid)]
    for v in vals:
        assert oracle.f64_to_bf16(v) == _exact_rne_bf16(v), v


def test_f64_to_bf16_specials(oracle):
    assert oracle.f64_to_bf16(0.0) == 0
    assert oracle.f64_to_bf16(-0.0) == 0x8000
    assert oracle.f64_to_bf16(math.inf) == 0x7F80
    assert oracle.f64_to_bf16(1e300) == 0x7F80
    assert oracle.f64_to_bf16(-1e300) == 0xFF80
    assert oracle.f64_to_bf16(1.0) == 0x3F80
    # the largest finite bf16 and a value just past its rounding boundary
    assert oracle.f64_to_bf16(float(_bf16_value(0x7F7F))) == 0x7F7F
    assert oracle.f64_to_bf16(float(_bf16_value(0x7F7F)) * (1 + 2**-8)) == 0x7F80
