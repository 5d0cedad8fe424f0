"""CPU oracle for the A8W4 fused-MoE layer (test infrastructure only).

Only the tests, the smoke check and the CPU-baseline leg of the benchmark
may import this package.  The HIP library never does, and this package
imports nothing from it: the two share no code.  The arithmetic lives in
``moe_oracle.c`` (plain C, FP64, OpenMP); this module only builds that file
with gcc, loads it, and marshals numpy arrays to it.

Sources of what is computed (page titles and sections):
  * aiter PR 5609 "Add DeepSeek V4.1 Flash TP4 gfx950 MoE tuning",
    Configuration: the number formats (8-bit float activations, 4-bit MX
    weights, one shared scale per run of 32), the gate and up rows stored
    alternately, a SiLU gate, and a result in bfloat16 with the routing
    probabilities entering only after the down projection.
  * aiter PR 5904 "Add tuned a8w4 fused-MoE configs for DeepSeek V4.1-Flash
    (TP4 + EP, gfx950)", "Fused-MoE kernel, expert-parallel benchmark": what
    one timed call spans -- grouping routes by expert, the two GEMMs, and the
    re-quantisation between them.
  * OCP Microscaling Formats v1.0 (E2M1, E8M0) and OCP 8-bit Floating Point
    v1.0 (E4M3) for the number formats those pages name.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB = os.path.join(_HERE, "libmoe_oracle.so")

_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (-O3, OpenMP) next to its source.  ISO C99
    mode keeps floating-point contraction off, so the result does not depend
    on the optimisation level."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O3", "-std=c99", "-fopenmp", "-fPIC", "-shared",
             "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build(force=False)
    lib = ctypes.CDLL(_LIB)
    c_i64, c_int, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    lib.oracle_e2m1_value.argtypes = [c_int]
    lib.oracle_e2m1_value.restype = ctypes.c_double
    lib.oracle_e8m0_value.argtypes = [c_int]
    lib.oracle_e8m0_value.restype = ctypes.c_double
    lib.oracle_e4m3_value.argtypes = [c_int]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_bf16_value.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_value.restype = ctypes.c_double
    lib.oracle_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = c_int
    lib.oracle_block_exponent.argtypes = [ctypes.c_double]
    lib.oracle_block_exponent.restype = c_int
    lib.oracle_quant_block.argtypes = [vp, c_int, vp, vp]
    lib.oracle_quant_block.restype = None
    lib.oracle_quant_act.argtypes = [c_i64, c_i64, vp, vp, vp]
    lib.oracle_quant_act.restype = None
    lib.oracle_sort.argtypes = [c_i64, c_int, c_int, c_int, c_int, vp, vp, vp, c_i64]
    lib.oracle_sort.restype = c_i64
    lib.oracle_route.argtypes = [c_i64, c_i64] + [vp] * 10
    lib.oracle_route.restype = None
    lib.oracle_forward.argtypes = ([c_i64, c_i64, c_i64, c_int, c_int, c_int] + [vp] * 7
                                   + [vp, c_i64, vp, vp])
    lib.oracle_forward.restype = None
    lib.oracle_intermediate.argtypes = ([c_i64, c_i64, c_i64, c_int, c_int, c_int] + [vp] * 4
                                        + [vp, c_i64, vp, vp, vp, vp, vp])
    lib.oracle_intermediate.restype = None
    lib.oracle_forward_given_intermediate.argtypes = ([c_i64, c_i64, c_i64, c_int, c_int, c_int]
                                                      + [vp] * 4 + [vp, c_i64, vp, vp, vp, vp, vp])
    lib.oracle_forward_given_intermediate.restype = None
    lib.oracle_a16_stage1.argtypes = [c_i64, c_i64, vp, vp, vp, vp, vp, vp]
    lib.oracle_a16_stage1.restype = None
    lib.oracle_a16_forward.argtypes = ([c_i64, c_i64, c_i64, c_int, c_int, c_int] + [vp] * 7
                                       + [vp, c_i64, vp, vp, vp])
    lib.oracle_a16_forward.restype = None
    lib.oracle_a16_intermediate.argtypes = ([c_i64, c_i64, c_i64, c_int, c_int, c_int] + [vp] * 4
                                            + [vp, c_i64, vp, vp, vp])
    lib.oracle_a16_intermediate.restype = None
    lib.oracle_a16_forward_given_intermediate.argtypes = ([c_i64, c_i64, c_i64, c_int, c_int, c_int]
                                                          + [vp] * 4 + [vp, c_i64, vp, vp, vp])
    lib.oracle_a16_forward_given_intermediate.restype = None
    lib.oracle_softmax_topk.argtypes = [c_i64, c_int, c_int, c_int, vp, vp, vp]
    lib.oracle_softmax_topk.restype = None
    lib.oracle_num_threads.argtypes = []
    lib.oracle_num_threads.restype = c_int
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# ------------------------------------------------------------------ formats

def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e8m0_value(code: int) -> float:
    return _load().oracle_e8m0_value(int(code))


def e4m3_value(code: int) -> float:
    return _load().oracle_e4m3_value(int(code))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def bf16_rne(x: float) -> int:
    return _load().oracle_bf16_rne(float(x))


def e4m3_encode(x: float) -> int:
    return _load().oracle_e4m3_encode(float(x))


def block_exponent(amax: float) -> int:
    return _load().oracle_block_exponent(float(amax))


def quant_block(v) -> tuple[np.ndarray, int]:
    """One block of values -> (E4M3 codes, E8M0 scale code)."""
    v = _c(v, np.float64)
    q = np.zeros(v.shape[0], np.uint8)
    s = np.zeros(1, np.uint8)
    _load().oracle_quant_block(_p(v), v.shape[0], _p(q), _p(s))
    return q, int(s[0])


# ----------------------------------------------------------------- the path

def quant_act(hidden_bf16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """hidden as uint16 BF16 bits [M, H] -> (codes u8 [M, H], scales u8 [M, H/32])."""
    x = _c(hidden_bf16, np.uint16)
    M, H = x.shape
    q = np.zeros((M, H), np.uint8)
    s = np.zeros((M, H // 32), np.uint8)
    _load().oracle_quant_act(M, H, _p(x), _p(q), _p(s))
    return q, s


def sort(topk_ids: np.ndarray, num_experts: int, expert_offset: int, block_m: int):
    """-> (sorted_ids i32 [P], block_expert i32 [P/bm]) for the local routes."""
    ids = _c(topk_ids, np.int32)
    M, k = ids.shape
    R = M * k
    cap = R + min(num_experts, R) * (block_m - 1) + 1
    sorted_ids = np.zeros(max(cap, 1), np.int32)
    block_expert = np.zeros(max(cap // block_m + 1, 1), np.int32)
    P = _load().oracle_sort(M, k, num_experts, expert_offset, block_m, _p(ids),
                            _p(sorted_ids), _p(block_expert), cap)
    if P < 0:
        raise RuntimeError("oracle sort: capacity exceeded")
    return sorted_ids[:P].copy(), block_expert[:P // block_m].copy()


def route(a_q, a_s, w13_e, w13_s_e, w2_e, w2_s_e):
    """One route through one expert: returns (h f64 [I], iq u8 [I], is u8 [I/32], y f64 [H])."""
    a_q = _c(a_q, np.uint8)
    a_s = _c(a_s, np.uint8)
    w13_e = _c(w13_e, np.uint8)
    w13_s_e = _c(w13_s_e, np.uint8)
    w2_e = _c(w2_e, np.uint8)
    w2_s_e = _c(w2_s_e, np.uint8)
    H = a_q.shape[0]
    I = w13_e.shape[0] // 2
    h = np.zeros(I, np.float64)
    iq = np.zeros(I, np.uint8)
    is_ = np.zeros(I // 32, np.uint8)
    y = np.zeros(H, np.float64)
    _load().oracle_route(H, I, _p(a_q), _p(a_s), _p(w13_e), _p(w13_s_e), _p(w2_e), _p(w2_s_e),
                         _p(h), _p(iq), _p(is_), _p(y))
    return h, iq, is_, y


def forward(hidden_bf16, topk_ids, topk_weights, w13, w13_s, w2, w2_s,
            expert_offset: int = 0, tokens=None, want_f64: bool = False):
    """The layer's BF16 output (uint16 bits) for all tokens or a list of tokens.

    Returns out_bf16 [ntok, H] (and the FP64 combine [ntok, H] if want_f64).
    """
    x = _c(hidden_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    w13 = _c(w13, np.uint8)
    w13_s = _c(w13_s, np.uint8)
    w2 = _c(w2, np.uint8)
    w2_s = _c(w2_s, np.uint8)
    M, H = x.shape
    k = ids.shape[1]
    E = w13.shape[0]
    I = w13.shape[1] // 2
    if tokens is None:
        tok = None
        ntok = M
    else:
        tok = _c(tokens, np.int64)
        ntok = tok.shape[0]
    out = np.zeros((ntok, H), np.uint16)
    o64 = np.zeros((ntok, H), np.float64) if want_f64 else None
    _load().oracle_forward(M, H, I, E, expert_offset, k, _p(x), _p(ids), _p(wts),
                           _p(w13), _p(w13_s), _p(w2), _p(w2_s),
                           _p(tok), ntok, _p(o64), _p(out))
    return (out, o64) if want_f64 else out


def a16_stage1(x_bf16_row, w13_e, w13_s_e):
    """A16W4 stage one for one route -> (h FP64 [I], BF16 bits [I])."""
    x = _c(x_bf16_row, np.uint16)
    w13_e = _c(w13_e, np.uint8)
    w13_s_e = _c(w13_s_e, np.uint8)
    H = x.shape[0]
    I = w13_e.shape[0] // 2
    h = np.zeros(I, np.float64)
    hb = np.zeros(I, np.uint16)
    _load().oracle_a16_stage1(H, I, _p(x), _p(w13_e), _p(w13_s_e), None, _p(h), _p(hb))
    return h, hb


def a16_intermediate(hidden_bf16, topk_ids, w13, w13_s, routes, expert_offset: int = 0):
    """A16W4 stage one for flat route indices -> (BF16 bits [n, I], SiLU(g) * u
    FP64 [n, I], gate/up FP64 [n, 2I] with gate j at 2j and up j at 2j + 1)."""
    x = _c(hidden_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    w13 = _c(w13, np.uint8)
    w13_s = _c(w13_s, np.uint8)
    r = _c(routes, np.int64)
    M, H = x.shape
    k = ids.shape[1]
    E = w13.shape[0]
    I = w13.shape[1] // 2
    n = r.shape[0]
    hb = np.zeros((n, I), np.uint16)
    h = np.zeros((n, I), np.float64)
    gu = np.zeros((n, 2 * I), np.float64)
    _load().oracle_a16_intermediate(M, H, I, E, expert_offset, k, _p(x), _p(ids), _p(w13), _p(w13_s),
                                    _p(r), n, _p(gu), _p(h), _p(hb))
    return hb, h, gu


def a16_forward_given_intermediate(topk_ids, topk_weights, w2, w2_s, inter_bf16, expert_offset: int = 0,
                                   tokens=None, want_f64: bool = False):
    """A16W4 stage two and the combine applied to a given BF16 intermediate
    [ntok, topk, I] (bits; non-local slots ignored) -> out_bf16 [ntok, H]
    (and the FP64 combine if want_f64)."""
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    w2 = _c(w2, np.uint8)
    w2_s = _c(w2_s, np.uint8)
    inter = _c(inter_bf16, np.uint16)
    M, k = ids.shape
    E, H = w2.shape[0], w2.shape[1]
    I = w2.shape[2] * 2
    tok = None if tokens is None else _c(tokens, np.int64)
    ntok = M if tokens is None else tok.shape[0]
    assert inter.shape == (ntok, k, I)
    out = np.zeros((ntok, H), np.uint16)
    o64 = np.zeros((ntok, H), np.float64) if want_f64 else None
    _load().oracle_a16_forward_given_intermediate(M, H, I, E, expert_offset, k, _p(ids), _p(wts), _p(w2),
                                                  _p(w2_s), _p(tok), ntok, _p(inter), _p(o64), _p(out))
    return (out, o64) if want_f64 else out


def a16_forward(hidden_bf16, topk_ids, topk_weights, w13, w13_s, w2, w2_s,
                expert_offset: int = 0, tokens=None, want_f64: bool = False,
                want_inter: bool = False):
    """The A16W4 layer's BF16 output (uint16 bits) for all tokens or a list of
    tokens; optionally the FP64 combine and the BF16 intermediate
    [ntok, topk, I] (zero for non-local slots)."""
    x = _c(hidden_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    w13, w13_s, w2, w2_s = (_c(a, np.uint8) for a in (w13, w13_s, w2, w2_s))
    M, H = x.shape
    k = ids.shape[1]
    E = w13.shape[0]
    I = w13.shape[1] // 2
    tok = None if tokens is None else _c(tokens, np.int64)
    ntok = M if tokens is None else tok.shape[0]
    out = np.zeros((ntok, H), np.uint16)
    o64 = np.zeros((ntok, H), np.float64) if want_f64 else None
    inter = np.zeros((ntok, k, I), np.uint16) if want_inter else None
    _load().oracle_a16_forward(M, H, I, E, expert_offset, k, _p(x), _p(ids), _p(wts),
                               _p(w13), _p(w13_s), _p(w2), _p(w2_s), _p(tok), ntok,
                               _p(inter), _p(o64), _p(out))
    res = (out,)
    if want_f64:
        res += (o64,)
    if want_inter:
        res += (inter,)
    return res if len(res) > 1 else out


def intermediate(hidden_bf16, topk_ids, w13, w13_s, routes, expert_offset: int = 0,
                 want_f64: bool = False, want_gu: bool = False):
    """Requantised intermediate for flat route indices -> (iq u8 [n, I], is u8 [n, I/32]),
    then h = SiLU(gate) * up FP64 [n, I] if want_f64, then the FP64 gate/up sums
    [n, 2I] (gate j at 2j, up j at 2j + 1) and the sums of |a_k w_k| of the
    same dot products [n, 2I] if want_gu."""
    x = _c(hidden_bf16, np.uint16)
    ids = _c(topk_ids, np.int32)
    w13 = _c(w13, np.uint8)
    w13_s = _c(w13_s, np.uint8)
    r = _c(routes, np.int64)
    M, H = x.shape
    k = ids.shape[1]
    E = w13.shape[0]
    I = w13.shape[1] // 2
    n = r.shape[0]
    iq = np.zeros((n, I), np.uint8)
    is_ = np.zeros((n, I // 32), np.uint8)
    h = np.zeros((n, I), np.float64) if want_f64 else None
    gu = np.zeros((n, 2 * I), np.float64) if want_gu else None
    gu_abs = np.zeros((n, 2 * I), np.float64) if want_gu else None
    _load().oracle_intermediate(M, H, I, E, expert_offset, k, _p(x), _p(ids), _p(w13), _p(w13_s),
                                _p(r), n, _p(gu), _p(gu_abs), _p(h), _p(iq), _p(is_))
    res = (iq, is_)
    if want_f64:
        res += (h,)
    if want_gu:
        res += (gu, gu_abs)
    return res


def forward_given_intermediate(topk_ids, topk_weights, w2, w2_s, inter_q, inter_s,
                               expert_offset: int = 0, tokens=None, want_f64: bool = False,
                               want_abs: bool = False):
    """Stage two and the combine applied to a given intermediate.

    inter_q [ntok, topk, I] / inter_s [ntok, topk, I/32] hold the requantised
    intermediate of each listed token's slots (non-local slots are ignored).
    Returns out_bf16 [ntok, H], then the FP64 combine if want_f64, then if
    want_abs the sum over local slots of |weight| * sum_j |inter_j w2[h, j]|.
    """
    ids = _c(topk_ids, np.int32)
    wts = _c(topk_weights, np.float32)
    w2 = _c(w2, np.uint8)
    w2_s = _c(w2_s, np.uint8)
    iq = _c(inter_q, np.uint8)
    is_ = _c(inter_s, np.uint8)
    M, k = ids.shape
    E, H = w2.shape[0], w2.shape[1]
    I = w2.shape[2] * 2
    if tokens is None:
        tok, ntok = None, M
    else:
        tok = _c(tokens, np.int64)
        ntok = tok.shape[0]
    assert iq.shape == (ntok, k, I) and is_.shape == (ntok, k, I // 32)
    out = np.zeros((ntok, H), np.uint16)
    o64 = np.zeros((ntok, H), np.float64) if want_f64 else None
    oab = np.zeros((ntok, H), np.float64) if want_abs else None
    _load().oracle_forward_given_intermediate(M, H, I, E, expert_offset, k, _p(ids), _p(wts),
                                              _p(w2), _p(w2_s), _p(tok), ntok, _p(iq), _p(is_),
                                              _p(o64), _p(out), _p(oab))
    res = (out,)
    if want_f64:
        res += (o64,)
    if want_abs:
        res += (oab,)
    return res if len(res) > 1 else out


def softmax_topk(logits, k_routed: int, shared_id: int = -1):
    """Router: (ids int32 [M, k], weights float64 [M, k]) for logits float32
    [M, E_routed]: the k_routed largest logits (lower id on ties) in
    descending order, weighted by the softmax of the chosen logits; with
    shared_id >= 0 a last slot holding that expert with weight 1."""
    lg = _c(logits, np.float32)
    M, Er = lg.shape
    assert 1 <= k_routed <= Er
    k = k_routed + (1 if shared_id >= 0 else 0)
    ids = np.zeros((M, k), np.int32)
    wts = np.zeros((M, k), np.float64)
    _load().oracle_softmax_topk(M, Er, k_routed, shared_id, _p(lg), _p(ids), _p(wts))
    return ids, wts


def num_threads() -> int:
    return _load().oracle_num_threads()
