"""Pins for the oracle's NVFP4 key codec (CPU only).

The oracle computes e4m3_rn_satfinite(e2m1(nib) * e4m3(scale)) (page
"vllm.models.minimax_m3.amd.indexer_nvfp4", module docstring).  It is pinned
here against things other than itself: torch's own float8_e4m3fn decoder and
round-to-nearest-even cast, an exact rational (fractions.Fraction) rounding
written from the format definition as a bracket search, the OCP E2M1 value
table, and hand-worked values in tests/golden/nvfp4_spot_values.txt.
"""
import math
import os
from fractions import Fraction

import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_spot_values.txt")

# OCP MX v1.0 E2M1 magnitudes for codes 0..7
E2M1_TABLE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_all_codes():
    for nib in range(16):
        v = oracle.e2m1_value(nib)
        mag = E2M1_TABLE[nib & 7]
        assert abs(v) == mag
        assert math.copysign(1.0, v) == (-1.0 if nib & 8 else 1.0)


def test_e4m3_decode_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().tolist()
    for c in range(256):
        v = oracle.e4m3_value(c)
        if c in (0x7F, 0xFF):
            assert math.isnan(v) and math.isnan(ref[c])
        else:
            assert v == ref[c], (hex(c), v, ref[c])
            assert math.copysign(1.0, v) == math.copysign(1.0, ref[c])


def _e4m3_grid():
    """(value, code) for the 127 non-negative finite E4M3 codes, from the
    format definition, exact."""
    out = []
    for e in range(16):
        for m in range(8):
            if e == 15 and m == 7:
                continue
            if e == 0:
                v = Fraction(m, 8) * Fraction(1, 64)
            else:
                v = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            out.append((v, e * 8 + m))
    return out


GRID = _e4m3_grid()


def _exact_rn_sat(x: Fraction) -> Fraction:
    a = abs(x)
    if a >= 448:
        r = Fraction(448)
    else:
        lo = max((g for g in GRID if g[0] <= a), key=lambda g: g[0])
        hi = min((g for g in GRID if g[0] >= a), key=lambda g: g[0])
        dl, dh = a - lo[0], hi[0] - a
        if dl < dh:
            r = lo[0]
        elif dh < dl:
            r = hi[0]
        else:
            r = lo[0] if lo[1] % 2 == 0 else hi[0]
    return -r if x < 0 else r


def test_nvfp4_exhaustive_vs_exact_rationals():
    """All 16 nibbles x 254 non-NaN scale codes."""
    for s in range(256):
        if s in (0x7F, 0xFF):
            continue
        sv = Fraction(oracle.e4m3_value(s))
        for nib in range(16):
            prod = Fraction(E2M1_TABLE[nib & 7]) * sv * (-1 if nib & 8 else 1)
            want = _exact_rn_sat(prod)
            got = oracle.nvfp4_element(nib, s)
            assert Fraction(got) == want, (hex(nib), hex(s), float(prod), got, float(want))
            if got == 0:
                # sign of zero follows the sign of the product
                assert math.copysign(1.0, got) == (-1.0 if ((nib & 8) != 0) != ((s & 0x80) != 0) else 1.0)


def test_rounding_matches_torch_cast_in_range():
    """In range torch's fp32 -> float8_e4m3fn cast is round-to-nearest-even,
    so it must agree with the oracle's rounding."""
    g = torch.Generator().manual_seed(7)
    xs = torch.cat([
        torch.randn(20000, generator=g) * 10,
        torch.rand(5000, generator=g) * 0.02,  # subnormal range
        torch.tensor([(v + w) / 2 for (v, _), (w, _) in zip(GRID[:-1], GRID[1:])],
                     dtype=torch.float64).float(),  # exact midpoints
    ])
    xs = xs[xs.abs() < 440]
    ref = xs.to(torch.float8_e4m3fn).float().tolist()
    for x, r in zip(xs.tolist(), ref):
        assert oracle.e4m3_rn_satfinite(x) == r, (x, r)


def test_saturation_never_overflows():
    for x in [448.0, 449.0, 463.99, 464.0, 480.0, 1e6, float("1e300")]:
        assert oracle.e4m3_rn_satfinite(x) == 448.0
        assert oracle.e4m3_rn_satfinite(-x) == -448.0


def test_golden_spot_values():
    n = 0
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            nib, sc, prod, want = line.split()
            nib, sc = int(nib, 16), int(sc, 16)
            assert oracle.e2m1_value(nib) * oracle.e4m3_value(sc) == float(prod)
            got = oracle.nvfp4_element(nib, sc)
            assert got == float(want), (hex(nib), hex(sc), got, want)
            assert math.copysign(1.0, got) == math.copysign(1.0, float(want))
            n += 1
    assert n >= 15
