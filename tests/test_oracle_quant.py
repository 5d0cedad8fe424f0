"""Pins of the oracle's per-1x32 FP8 quantiser (E8M0 scale + E4M3 elements).

The element encoding is checked against a brute-force nearest search over
the finite E4M3 values as torch decodes them (ties to the even code), and
against torch's own float8_e4m3fn cast where that cast does not overflow;
the scale exponent against frexp.  Every finite BF16 value is exercised
both as the block maximum and as an ordinary element.
"""
import numpy as np
import pytest
import torch

from mixture_experts_fp8_amd.workloads import bf16_to_f32

# finite non-negative E4M3 values as torch decodes codes 0x00 .. 0x7E
E4M3_POS = torch.arange(127, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def nearest_code_bruteforce(a):
    """Nearest finite E4M3 code (0..126) to each |a|, ties to the even code."""
    a = np.abs(np.asarray(a, np.float64))
    d = np.abs(E4M3_POS[None, :] - a[:, None])
    best = d.min(axis=1, keepdims=True)
    cand = d == best
    # among equally near codes take the even one (at most two candidates)
    codes = np.where(cand, np.arange(127)[None, :], 1 << 20)
    even = np.where(cand & (np.arange(127)[None, :] % 2 == 0), np.arange(127)[None, :], 1 << 20)
    c_even = even.min(axis=1)
    c_any = codes.min(axis=1)
    return np.where(c_even < (1 << 20), c_even, c_any)


def encode_bruteforce(v):
    v = np.asarray(v, np.float64)
    c = nearest_code_bruteforce(v)
    return (c | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def finite_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    return bits[exp != 0xFF]


def test_every_bf16_as_block_max(oracle):
    """Block = [x, x/2, -x/4, ...]: scale from floor(log2|x|) - 8, codes by brute force."""
    pats = finite_bf16_patterns()
    x = bf16_to_f32(pats).astype(np.float64)
    nz = x != 0
    pats, x = pats[nz], x[nz]
    M = len(pats)
    blocks = np.zeros((M, 32), np.uint16)
    rng = np.random.default_rng(5)
    blocks[:, 0] = pats
    # other elements: bf16 values no larger in magnitude than x
    for i in range(1, 32):
        frac = rng.uniform(-1, 1, M)
        blocks[:, i] = np.frombuffer(
            ((x * frac).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16).tobytes(), np.uint16)
    q, s = oracle.quant_act(blocks)
    vals = bf16_to_f32(blocks).astype(np.float64)
    amax = np.abs(vals).max(axis=1)
    m, e = np.frexp(amax)
    E = np.clip(e - 1 - 8, -127, 127)
    assert np.array_equal(s[:, 0].astype(np.int64), E + 127)
    scaled = vals * np.exp2(-E.astype(np.float64))[:, None]
    # the scaled block maximum lies in [256, 512) unless the exponent clamped
    ok = E > -127
    smax = np.abs(scaled).max(axis=1)
    assert np.all((smax[ok] >= 256) & (smax[ok] < 512))
    ref = np.zeros_like(q)
    for lo in range(0, M, 4096):
        ref[lo:lo + 4096] = encode_bruteforce(scaled[lo:lo + 4096].ravel()).reshape(-1, 32)
    assert np.array_equal(q, ref)


@pytest.mark.parametrize("amax_bits", [0x3F80, 0x4380, 0x0080, 0x7F7F, 0x3C01])
def test_every_bf16_as_ordinary_element(oracle, amax_bits):
    """All finite BF16 values no larger than a fixed block maximum, as elements."""
    pats = finite_bf16_patterns()
    amax = float(bf16_to_f32(np.array([amax_bits], np.uint16))[0])
    v = bf16_to_f32(pats).astype(np.float64)
    keep = np.abs(v) <= amax
    pats = pats[keep]
    n = len(pats)
    nb = (n + 30) // 31
    blocks = np.zeros((nb, 32), np.uint16)
    blocks[:, 0] = amax_bits
    flat = np.zeros(nb * 31, np.uint16)
    flat[:n] = pats
    blocks[:, 1:] = flat.reshape(nb, 31)
    q, s = oracle.quant_act(blocks)
    _, e = np.frexp(amax)
    E = max(min(e - 1 - 8, 127), -127)
    assert np.all(s == E + 127)
    vals = bf16_to_f32(blocks).astype(np.float64) * 2.0 ** (-E)
    ref = encode_bruteforce(vals.ravel()).reshape(nb, 32)
    assert np.array_equal(q, ref)


def test_encode_matches_torch_cast_in_range(oracle):
    """torch's float8_e4m3fn cast rounds to nearest even and overflows past 464;
    below that it must agree with the oracle's encoder code for code."""
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.uniform(-463.9, 463.9, 20000),
                        rng.uniform(-1, 1, 20000) * 2.0 ** -6,
                        (np.arange(-3700, 3700) / 8.0)])  # many exact ties
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(x)) for x in v], np.uint8)
    assert np.array_equal(got, ref)


def test_saturation_and_zero(oracle):
    assert oracle.e4m3_encode(448.0) == 0x7E
    assert oracle.e4m3_encode(463.99) == 0x7E
    assert oracle.e4m3_encode(1e30) == 0x7E
    assert oracle.e4m3_encode(-1e30) == 0xFE
    assert oracle.e4m3_encode(0.0) == 0x00
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(2.0 ** -11) == 0x00   # below half the least subnormal
    assert oracle.e4m3_encode(2.0 ** -10) == 0x00   # exact tie with 0 -> even code 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10) == 0x02  # tie between 1 and 2 -> 2
    q, s = oracle.quant_block(np.zeros(32))
    assert s == 0 and np.all(q == 0)
    q, s = oracle.quant_block(-np.zeros(32))
    assert s == 0 and np.all(q == 0x80)


def test_block_exponent_closed_form(oracle):
    for a, E in [(1.0, -8), (1.5, -8), (2.0, -7), (511.0, 0), (512.0, 1), (0.0, -127),
                 (2.0 ** -130, -127), (2.0 ** 200, 127), (2.0 ** 134, 126)]:
        assert oracle.block_exponent(a) == E, a
