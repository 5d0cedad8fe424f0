"""Pins of the oracle's number formats (decode tables and BF16 rounding).

Each check compares the oracle with something other than itself: the spec
values stored under tests/golden/ (with their citations), torch's own
float8_e4m3fn / float8_e8m0fnu / bfloat16 conversions, and brute-force
searches over the whole code space.
"""
import math
import os

import numpy as np
import pytest
import torch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def _same(a, b):
    if math.isnan(a) or math.isnan(b):
        return math.isnan(a) and math.isnan(b)
    return a == b and math.copysign(1.0, a) == math.copysign(1.0, b)


def test_e2m1_all_16_codes_match_spec_table(oracle):
    rows = _read("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        assert _same(oracle.e2m1_value(int(code)), float(val)), code


def test_e4m3_spec_points(oracle):
    for code, val in _read("e4m3_points.txt"):
        assert _same(oracle.e4m3_value(int(code, 16)), float(val)), code


def test_e4m3_all_256_codes_match_torch(oracle):
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e4m3_value(c), float(ref[c])), c


def test_e8m0_spec_points_and_all_codes_match_torch(oracle):
    for code, val in _read("e8m0_points.txt"):
        assert _same(oracle.e8m0_value(int(code)), float(val)), code
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    for c in range(256):
        assert _same(oracle.e8m0_value(c), float(ref[c])), c


def test_bf16_decode_matches_torch_on_all_patterns(oracle):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b in range(0, 65536, 7):  # a stride keeps the ctypes loop short
        assert _same(oracle.bf16_value(int(b)), float(ref[b])), b


def _bf16_nearest_bruteforce(x):
    """Nearest BF16 by scanning the two BF16 neighbours of x (ties to even)."""
    f = np.float64(x)
    # all finite positive bf16 values, increasing with the bit pattern
    vals = _ALL_BF16_POS
    i = np.searchsorted(vals, abs(f))
    cands = []
    for j in (i - 1, i):
        if 0 <= j < len(vals):
            cands.append((abs(vals[j] - abs(f)), j))
    cands.sort(key=lambda c: (c[0], c[1] % 2))
    d, j = cands[0]
    if abs(f) > vals[-1]:
        # beyond the largest finite value: IEEE rounds to inf once past the
        # midpoint between max and 2^128
        mid = (vals[-1] + 2.0 ** 128) / 2
        if abs(f) >= mid:
            return 0x7F80 | (0x8000 if f < 0 else 0)
        j = len(vals) - 1
    return int(j) | (0x8000 if math.copysign(1.0, f) < 0 else 0)


_ALL_BF16_POS = (np.arange(0, 0x7F80, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)


def test_bf16_rounding_matches_bruteforce_and_torch(oracle):
    rng = np.random.default_rng(11)
    xs = list(rng.standard_normal(3000) * 10.0 ** rng.integers(-40, 39, 3000))
    # exact ties: midpoints between consecutive BF16 values
    for b in rng.integers(1, 0x7F7F, 500):
        lo = _ALL_BF16_POS[b]
        hi = _ALL_BF16_POS[b + 1]
        xs.append((lo + hi) / 2)
        xs.append(-(lo + hi) / 2)
    xs += [0.0, -0.0, 1e-45, 3.0e38, 3.4e38, 3.5e38, -3.5e38, 2.0 ** -133, 2.0 ** -134, 2.0 ** -135]
    for x in xs:
        assert oracle.bf16_rne(x) == _bf16_nearest_bruteforce(x), x
    # torch rounds float32 -> bfloat16 to nearest even; compare on float32 inputs
    f32 = rng.standard_normal(4000).astype(np.float32) * np.float32(37.0)
    ref = torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().astype(np.uint16)
    for x, r in zip(f32, ref):
        assert oracle.bf16_rne(float(x)) == int(r)
