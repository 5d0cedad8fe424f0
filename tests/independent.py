"""Independent statements of the layer's pieces, for pinning the oracle.

Nothing here calls the oracle or the HIP library.  Number formats come from
torch's own float8 decoders; the quantiser is a brute-force nearest search;
dot products are exact integer arithmetic.  These are slow and only meant for
small shapes.
"""
from fractions import Fraction
import math

import numpy as np
import torch

# decoded values of every E4M3 code (torch's float8_e4m3fn) and E8M0 code
E4M3_ALL = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
E4M3_POS = E4M3_ALL[:127]
E8M0_ALL = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
# E2M1 magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6 as listed by the OCP MX spec
E2M1_ALL = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0,
                     -0.0, -0.5, -1.0, -1.5, -2.0, -3.0, -4.0, -6.0])


def bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def unpack_e2m1(codes):
    """[..., n/2] bytes -> [..., n] codes, element 2i from the low nibble of byte i."""
    codes = np.asarray(codes, np.uint8)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = codes & 15
    out[..., 1::2] = codes >> 4
    return out


def dequant_mxfp4(codes, scales):
    """MXFP4 matrix -> float64 values."""
    v = E2M1_ALL[unpack_e2m1(codes)]
    s = E8M0_ALL[np.asarray(scales, np.uint8)]
    return v * np.repeat(s, 32, axis=-1)


def dequant_fp8(codes, scales):
    v = E4M3_ALL[np.asarray(codes, np.uint8)]
    s = E8M0_ALL[np.asarray(scales, np.uint8)]
    return v * np.repeat(s, 32, axis=-1)


def encode_e4m3_bruteforce(v):
    """Nearest finite E4M3 code to each value (ties to the even code), sign kept."""
    v = np.asarray(v, np.float64).ravel()
    a = np.abs(v)
    d = np.abs(E4M3_POS[None, :] - a[:, None])
    best = d.min(axis=1, keepdims=True)
    idx = np.arange(127)[None, :]
    cand = d == best
    even = np.where(cand & (idx % 2 == 0), idx, 1 << 20).min(axis=1)
    anyc = np.where(cand, idx, 1 << 20).min(axis=1)
    c = np.where(even < (1 << 20), even, anyc)
    return (c | np.where(np.signbit(v), 0x80, 0)).astype(np.uint8)


def quantize_rows_bruteforce(x):
    """[..., n] float64 -> (codes [..., n], scale codes [..., n/32]) by the per-1x32 rule:
    scale exponent floor(log2 amax) - 8 clamped to [-127, 127], elements nearest."""
    x = np.asarray(x, np.float64)
    shp = x.shape
    blocks = x.reshape(-1, 32)
    amax = np.abs(blocks).max(axis=1)
    _, e = np.frexp(amax)
    E = np.where(amax > 0, e - 1 - 8, -127)
    E = np.clip(E, -127, 127)
    scaled = blocks * np.exp2(-E.astype(np.float64))[:, None]
    q = encode_e4m3_bruteforce(scaled).reshape(shp)
    s = (E + 127).astype(np.uint8).reshape(shp[:-1] + (shp[-1] // 32,))
    return q, s


# ---------------------------------------------------------------- exact dots

def _int_parts_fp8(codes, scales):
    """value = n * 2^p exactly: n integer (code value * 512), p = scale - 127 - 9 per element."""
    n = np.rint(E4M3_ALL[codes] * 512).astype(np.int64)
    p = np.repeat(scales.astype(np.int64) - 127 - 9, 32, axis=-1)
    return n, p


def _int_parts_fp4(codes_packed, scales):
    c = unpack_e2m1(codes_packed)
    n = np.rint(E2M1_ALL[c] * 2).astype(np.int64)
    p = np.repeat(scales.astype(np.int64) - 127 - 1, 32, axis=-1)
    return n, p


def exact_dot(na, pa, nb, pb):
    """Exact sum of (na*2^pa) * (nb*2^pb) as a Fraction."""
    prod = na * nb
    ex = pa + pb
    lo = int(ex.min())
    total = 0
    for v, x in zip(prod.tolist(), (ex - lo).tolist()):
        if v:
            total += v << x
    return Fraction(total) * (Fraction(2) ** lo)


def bruteforce_forward(hidden_bits, topk_ids, topk_weights, w13, w13_s, w2, w2_s, expert_offset=0):
    """The layer, route by route, with exact dot products.

    Returns (o exact Fractions as float64 [M, H], intermediates {f: (iq, is)}).
    """
    M, H = hidden_bits.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    k = topk_ids.shape[1]
    a_q, a_s = quantize_rows_bruteforce(bf16_to_f64(hidden_bits))
    out = np.zeros((M, H), np.float64)
    inter = {}
    for t in range(M):
        na, pa = _int_parts_fp8(a_q[t], a_s[t])
        o = [Fraction(0)] * H
        for s in range(k):
            e = int(topk_ids[t, s]) - expert_offset
            if e < 0 or e >= E:
                continue
            h = np.zeros(I)
            for j in range(I):
                ng, pg = _int_parts_fp4(w13[e, 2 * j], w13_s[e, 2 * j])
                nu, pu = _int_parts_fp4(w13[e, 2 * j + 1], w13_s[e, 2 * j + 1])
                g = float(exact_dot(na, pa, ng, pg))
                u = float(exact_dot(na, pa, nu, pu))
                h[j] = g / (1.0 + math.exp(-g)) * u
            iq, is_ = quantize_rows_bruteforce(h)
            inter[t * k + s] = (iq, is_)
            ni, pi = _int_parts_fp8(iq, is_)
            wk = Fraction(float(topk_weights[t, s]))
            for hh in range(H):
                n2, p2 = _int_parts_fp4(w2[e, hh], w2_s[e, hh])
                o[hh] += wk * exact_dot(ni, pi, n2, p2)
        out[t] = [float(v) for v in o]
    return out, inter


def bf16_round_bruteforce(x):
    """float64 -> BF16 bits by choosing the nearer of the two neighbouring BF16
    values (ties to the even pattern); finite inputs within BF16 range."""
    x = np.asarray(x, np.float64).ravel()
    f32 = x.astype(np.float32)  # nearest float32; exact if x came from a short sum
    b = (f32.view(np.uint32) >> 16).astype(np.int64) & 0x7FFF
    res = np.empty(x.shape, np.uint16)
    for i, (xv, bv) in enumerate(zip(x.tolist(), b.tolist())):
        a = abs(xv)
        best = None
        for cand in (bv - 1, bv, bv + 1):
            if cand < 0 or cand >= 0x7F80:
                continue
            val = float(bf16_to_f64(np.array([cand], np.uint16))[0])
            key = (abs(val - a), cand % 2)
            if best is None or key < best[0]:
                best = (key, cand)
        res[i] = best[1] | (0x8000 if math.copysign(1.0, xv) < 0 else 0)
    return res


def _int_parts_bf16(bits):
    """BF16 bits -> (n, p) with value = n * 2^p exactly (finite values)."""
    b = np.asarray(bits, np.uint16).astype(np.int64)
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    n = np.where(e == 0, m, m + 128)
    p = np.where(e == 0, -133, e - 134)
    return np.where(b & 0x8000, -n, n), p


def bruteforce_a16_forward(hidden_bits, topk_ids, topk_weights, w13, w13_s, w2, w2_s, expert_offset=0):
    """The A16W4 variant route by route: exact dot products of the BF16
    activations with the MXFP4 rows, SiLU(g) * u rounded to BF16 by the
    brute-force neighbour search, exact stage-two dot products, exact sum of
    the weighted routes.  Returns (o as float64 [M, H], {f: BF16 bits [I]})."""
    M, H = hidden_bits.shape
    E = w13.shape[0]
    I = w13.shape[1] // 2
    k = topk_ids.shape[1]
    out = np.zeros((M, H), np.float64)
    inter = {}
    for t in range(M):
        na, pa = _int_parts_bf16(hidden_bits[t])
        o = [Fraction(0)] * H
        for s in range(k):
            e = int(topk_ids[t, s]) - expert_offset
            if e < 0 or e >= E:
                continue
            h = np.zeros(I)
            for j in range(I):
                ng, pg = _int_parts_fp4(w13[e, 2 * j], w13_s[e, 2 * j])
                nu, pu = _int_parts_fp4(w13[e, 2 * j + 1], w13_s[e, 2 * j + 1])
                g = float(exact_dot(na, pa, ng, pg))
                u = float(exact_dot(na, pa, nu, pu))
                h[j] = g / (1.0 + math.exp(-g)) * u
            hb = bf16_round_bruteforce(h)
            inter[t * k + s] = hb
            nh, ph = _int_parts_bf16(hb)
            wk = Fraction(float(topk_weights[t, s]))
            for hh in range(H):
                n2, p2 = _int_parts_fp4(w2[e, hh], w2_s[e, hh])
                o[hh] += wk * exact_dot(nh, ph, n2, p2)
        out[t] = [float(v) for v in o]
    return out, inter
