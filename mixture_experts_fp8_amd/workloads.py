"""Seeded synthetic inputs for the A8W4 fused-MoE layer.

This module serves both the CPU oracle and the HIP path and therefore holds
none of the layer's arithmetic: it only draws random weight codes, scale
codes, BF16 activations and routings, with the shapes and distributions of
the workloads the pages measure:

  * aiter PR 5609 "Add DeepSeek V4.1 Flash TP4 gfx950 MoE tuning",
    Configuration: hidden 5120, TP-local intermediate 576 padded to 640;
    backbone 384 experts top-6 with decode rows M = 6 ... 768, draft 128
    experts top-3 with M = 5 ... 640; Validation: boundary token counts
    31/32/33/255/256/257 and a concentrated-routing case.
  * aiter PR 5904 "Add tuned a8w4 fused-MoE configs for DeepSeek V4.1-Flash
    (TP4 + EP, gfx950)": hidden 5120, intermediate 2304, 96 local experts,
    top-6, token counts 1 ... 16384, random routing.
  * aiter PR 6286 "Retune gfx942 a16w4 DSv4.1 tiles for Triton 3.8", the
    isolated-kernel tables: 385 experts top-7 with a fused shared expert, and
    round-robin top-k routing; its A16W4 sizes (w1 N 1536 K 5120, w2 N 5120
    K 768, 384 top-6 and 385 top-7, M = 12 ... 16384).

Distributions (no trained weights exist here, so all are synthetic):
  weights  E2M1 codes uniform over the 16 codes, E8M0 scale codes uniform over
           {119, 120, 121, 122} (block exponents -8 ... -5); intermediate
           columns past the valid width hold code 0.  (The numerical stress
           geometry "wide-scale" draws codes 100 ... 140 instead.)
  hidden   BF16 of N(0, 1) draws (in "wide-scale" each block of 32 scaled by
           a power of two between 2^-20 and 2^20).
  routing  softmax of N(0, 1) logits, top-k, renormalised to sum 1 (float32);
           concentrated: 80 % of a token's slots go to 4 hot experts;
           round-robin: ids (t*k + s) mod E with weights 1/k;
           shared: one extra slot naming the shared expert with weight 1.
"""
from __future__ import annotations

import dataclasses
from functools import lru_cache

import numpy as np

# E8M0 scale codes used for the weights: exponents -8 .. -5
WEIGHT_SCALE_CODES = (119, 120, 121, 122)

ROUTINGS = ("softmax", "concentrated", "roundrobin")


@dataclasses.dataclass(frozen=True)
class Workload:
    """One geometry of the layer as one GPU holds it."""
    name: str
    hidden: int          # H
    inter: int           # I as stored (padded)
    inter_valid: int     # I before zero padding
    num_experts: int     # E held in the weight tensors
    routed_experts: int  # experts the router chooses among (excluding a shared one)
    topk: int            # slots per token, including a shared slot
    shared: bool         # last slot is the shared expert (id routed_experts), weight 1
    expert_offset: int   # global id of weight row 0
    tokens: tuple        # token counts (M) of the workload
    routings: tuple      # routing modes exercised
    config_id: int
    scale_codes: tuple = None   # E8M0 weight scale codes drawn (None: WEIGHT_SCALE_CODES)
    act_exp_spread: int = 0     # hidden blocks of 32 scaled by 2^u, u uniform in [-spread, spread]


WORKLOADS = {
    "draft-decode": Workload("draft-decode", 5120, 640, 576, 128, 128, 3, False, 0,
                             (5,), ("softmax",), 1),
    "backbone-decode": Workload("backbone-decode", 5120, 640, 576, 384, 384, 6, False, 0,
                                (6, 12, 24, 48, 96, 192, 384, 768, 31, 32, 33, 255, 256, 257),
                                ("softmax",), 2),
    "draft-sweep": Workload("draft-sweep", 5120, 640, 576, 128, 128, 3, False, 0,
                            (5, 10, 20, 40, 80, 160, 320, 640), ("softmax", "concentrated"), 3),
    "local-slice": Workload("local-slice", 5120, 2304, 2304, 96, 384, 6, False, 0,
                            (1, 4, 16, 64, 256, 1024, 4096, 16384), ("softmax",), 4),
    "prefill-shared": Workload("prefill-shared", 5120, 640, 576, 385, 384, 7, True, 0,
                               (4096, 16384), ("roundrobin", "softmax"), 5),
    # the A16W4 variant (BF16 activations): w1 N = 1536, K = 5120; w2 N = 5120, K = 768
    "a16w4-backbone": Workload("a16w4-backbone", 5120, 768, 768, 384, 384, 6, False, 0,
                               (12, 256, 1024, 1536, 4096, 16384), ("roundrobin",), 6),
    "a16w4-shared": Workload("a16w4-shared", 5120, 768, 768, 385, 384, 7, True, 0,
                             (12, 256, 1024, 1536, 4096, 16384), ("roundrobin",), 7),
    # a numerical stress geometry, not a measured one: weight scales over 41
    # binades (codes 100 ... 140) and hidden blocks scaled by 2^-20 ... 2^20,
    # so the MFMA scale operands and the requantisation exponents span a wide
    # range (the measured workloads keep them within a few binades)
    "wide-scale": Workload("wide-scale", 5120, 640, 576, 32, 32, 4, False, 0,
                           (40, 300, 1100), ("softmax",), 8, scale_codes=(100, 140), act_exp_spread=20),
}

# the decode buckets of the backbone geometry (the boundary counts are parity cases)
BACKBONE_DECODE_BUCKETS = (6, 12, 24, 48, 96, 192, 384, 768)


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields changed (small test geometries)."""
    return dataclasses.replace(w, **changes)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> BF16 bit patterns (uint16), nearest with ties to even."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_weights(w: Workload, seed=None):
    """(w13 [E,2I,H/2], w13_s [E,2I,H/32], w2 [E,H,I/2], w2_s [E,H,I/32]) as uint8."""
    rng = np.random.default_rng([w.config_id, 1] if seed is None else seed)
    E, H, I, Iv = w.num_experts, w.hidden, w.inter, w.inter_valid
    sc = WEIGHT_SCALE_CODES if w.scale_codes is None else w.scale_codes
    lo, hi = sc[0], sc[-1] + 1

    def codes(shape):  # uniform random bytes = two independent uniform E2M1 codes
        n = int(np.prod(shape))
        raw = rng.bit_generator.random_raw((n + 7) // 8).view(np.uint8)
        return raw[:n].reshape(shape)

    w13 = codes((E, 2 * I, H // 2))
    w13_s = rng.integers(lo, hi, size=(E, 2 * I, H // 32), dtype=np.uint8)
    w2 = codes((E, H, I // 2))
    w2_s = rng.integers(lo, hi, size=(E, H, I // 32), dtype=np.uint8)
    if Iv < I:
        w13[:, 2 * Iv:, :] = 0          # gate/up rows of the padded columns
        w2[:, :, Iv // 2:] = 0          # down-projection columns past the valid width
    return w13, w13_s, w2, w2_s


@lru_cache(maxsize=2)
def cached_weights(w: Workload):
    return make_weights(w)


def make_hidden(rng, M: int, H: int, exp_spread: int = 0) -> np.ndarray:
    x = rng.standard_normal((M, H), dtype=np.float32)
    if exp_spread:
        # one power of two per block of 32: exact in BF16, no overflow
        e = rng.integers(-exp_spread, exp_spread + 1, size=(M, H // 32))
        x = x * np.repeat(np.exp2(e).astype(np.float32), 32, axis=1)
    return bf16_bits(x)


def _softmax_topk(logits: np.ndarray, k: int):
    """float32 softmax over the last axis, top-k by value (lower id on ties),
    weights renormalised to sum 1 in float32."""
    z = logits - logits.max(axis=1, keepdims=True)
    p = np.exp(z, dtype=np.float32)
    p = p / p.sum(axis=1, keepdims=True, dtype=np.float32)
    order = np.argsort(-p, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(p, order, axis=1)
    top = top / top.sum(axis=1, keepdims=True, dtype=np.float32)
    return order.astype(np.int32), top.astype(np.float32)


def make_routing(rng, w: Workload, M: int, mode: str):
    """(topk_ids int32 [M, topk] global ids, topk_weights float32 [M, topk])."""
    kr = w.topk - (1 if w.shared else 0)
    Er = w.routed_experts
    if mode == "softmax":
        logits = rng.standard_normal((M, Er), dtype=np.float32)
        ids, wts = _softmax_topk(logits, kr)
    elif mode == "roundrobin":
        t = np.arange(M, dtype=np.int64)[:, None]
        s = np.arange(kr, dtype=np.int64)[None, :]
        ids = ((t * kr + s) % Er).astype(np.int32)
        wts = np.full((M, kr), 1.0 / kr, np.float32)
    elif mode == "concentrated":
        hot = 4
        ids = np.zeros((M, kr), np.int32)
        for t in range(M):
            chosen = []
            for _ in range(kr):
                free_hot = [e for e in range(hot) if e not in chosen]
                if free_hot and rng.random() < 0.8:
                    chosen.append(int(free_hot[rng.integers(len(free_hot))]))
                else:
                    while True:
                        e = int(rng.integers(hot, Er))
                        if e not in chosen:
                            break
                    chosen.append(e)
            ids[t] = chosen
        logits = rng.standard_normal((M, kr), dtype=np.float32)
        z = logits - logits.max(axis=1, keepdims=True)
        p = np.exp(z, dtype=np.float32)
        wts = (p / p.sum(axis=1, keepdims=True, dtype=np.float32)).astype(np.float32)
    else:
        raise ValueError("unknown routing mode %r" % mode)
    if w.shared:
        ids = np.concatenate([ids, np.full((M, 1), Er, np.int32)], axis=1)
        wts = np.concatenate([wts, np.ones((M, 1), np.float32)], axis=1)
    return np.ascontiguousarray(ids), np.ascontiguousarray(wts)


def make_inputs(w: Workload, M: int, mode: str = "softmax", seed=None):
    """(hidden BF16 bits [M,H], topk_ids [M,k], topk_weights [M,k]) for one call."""
    rng = np.random.default_rng([w.config_id, 2, M, ROUTINGS.index(mode)] if seed is None else seed)
    hidden = make_hidden(rng, M, w.hidden, w.act_exp_spread)
    ids, wts = make_routing(rng, w, M, mode)
    return hidden, ids, wts


def local_routes(w: Workload, topk_ids: np.ndarray) -> int:
    le = topk_ids.astype(np.int64) - w.expert_offset
    return int(((le >= 0) & (le < w.num_experts)).sum())
