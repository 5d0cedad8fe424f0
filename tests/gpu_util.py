"""Helpers for the GPU parity tests: device copies, one layer's weights, and
the comparison gate.  Everything here only moves data; the arithmetic under
test runs in the HIP library, the expected values come from the oracle."""
import numpy as np
import torch

from mixture_experts_fp8_amd import abi, workloads as wl

DEV = torch.device("cuda:0")

# fixed per-rank gate of the pages' validation: |gpu - ref| <= 0.02 + 0.02 |ref|
ATOL = 0.02
RTOL = 0.02


def note(msg):
    print(msg, flush=True)


def dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(a).to(DEV)


def host_bf16_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class Layer:
    """One geometry with its weights on the host (for the oracle) and packed on the GPU."""

    def __init__(self, w: wl.Workload, weights=None):
        self.w = w
        self.host = weights if weights is not None else wl.make_weights(w)
        d = abi.make_dims(1, w.hidden, w.inter, w.num_experts, w.topk, w.expert_offset, w.routed_experts)
        raw = [dev(x) for x in self.host]
        self.packed = abi.moe_a8w4_pack_weights(d, *raw)
        torch.cuda.synchronize()
        del raw

    def dims(self, M):
        w = self.w
        return abi.make_dims(M, w.hidden, w.inter, w.num_experts, w.topk, w.expert_offset,
                             w.routed_experts)

    def forward(self, hidden, ids, wts, out=None, workspace=None):
        M = hidden.shape[0]
        x = hidden if torch.is_tensor(hidden) else dev(hidden)
        i = ids if torch.is_tensor(ids) else dev(ids)
        g = wts if torch.is_tensor(wts) else dev(wts)
        return abi.moe_a8w4_forward(self.dims(M), x, i, g, *self.packed, out=out, workspace=workspace)


def gate_failures(got, ref):
    """Boolean mask of elements outside the gate (non-finite counts as failing)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return ~(np.abs(got - ref) <= ATOL + RTOL * np.abs(ref)) | ~np.isfinite(got)


def assert_gate(got, ref, what=""):
    bad = gate_failures(got, ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError("%s: %d of %d outside atol=rtol=2e-2, e.g. %s got %s ref %s" % (
            what, bad.sum(), bad.size, idx.tolist(), np.asarray(got)[tuple(idx.T)],
            np.asarray(ref)[tuple(idx.T)]))


# --------------------------------------------------------- layer parity
#
# The requantised intermediate has more than one correct value: GPU stage one
# accumulates in FP32 (inside the MFMA) where the oracle uses FP64, so an
# element lying within that accumulation error of an FP8 rounding boundary may
# round to the neighbouring code, and a block maximum that close to a power of
# two may pick the neighbouring scale.  The checks therefore split the layer:
#   (a) the GPU intermediate must be a faithful rounding of the oracle's exact
#       FP64 SiLU(gate) * up, within a local error budget: the GPU's gate and
#       up sums carry an accumulation error bounded by
#           2^-12 * (K / 128) * max|a| * max|w_row|
#       (per 128-long MFMA step, a measured single-instruction error of
#       2^-14.7 of the largest product, times 4 for margin), propagated
#       through SiLU(g) * u; every element must lie within that budget plus
#       one FP8 step of the exact value, block scales must be equal or one
#       apart only where the exact block maximum is within the budget of a
#       power of two, and at most 2 % of codes may differ from the correctly
#       rounded ones;
#   (b) given the GPU's intermediate, the output is unique: the oracle's stage
#       two and combine applied to it must match the GPU output at the gate;
#   (c) against the oracle end to end, at most 1 % of elements may fall
#       outside the gate (a flipped intermediate code moves small outputs by
#       about 0.03).

import oracle  # noqa: E402


def gpu_intermediate(layer, xd, idd, M):
    """(sorted_ids, inter_q, inter_s) of the GPU steps, rows 0 .. num_padded."""
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    q, s = abi.moe_a8w4_quant_act(xd)
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, idd)
    iq, is_ = abi.moe_a8w4_stage1(d, bm, q, s, srt, bexp, npad, layer.packed[0], layer.packed[1])
    torch.cuda.synchronize()
    P = int(npad.item())
    return srt[:P].cpu().numpy(), iq[:P].cpu().numpy(), is_[:P].cpu().numpy()


def route_positions(sorted_ids, M, topk, routes):
    real = np.nonzero(sorted_ids != M)[0]
    f = (sorted_ids[real] & 0xFFFFFF).astype(np.int64) * topk + (sorted_ids[real] >> 24)
    lookup = np.full(M * topk, -1, np.int64)
    lookup[f] = real
    return lookup[routes]


_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _dequant(q, s):
    return _E4M3[q] * np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=-1)


def stage1_budget(layer, hidden, ids, routes):
    """Per-element bound on |h_gpu - h_exact| from the FP32 accumulation of
    gate and up (see (a) above), for the listed flat routes."""
    w = layer.w
    h13, h13s = layer.host[:2]
    k = ids.shape[1]
    tok = routes // k
    aq, as_ = oracle.quant_act(hidden[tok])
    A = _dequant(aq, as_)
    le = ids.ravel()[routes].astype(np.int64) - w.expert_offset
    KS = w.hidden // 128
    out = np.zeros((len(routes), w.inter))
    e2m1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])
    for e in np.unique(le):
        rs = np.nonzero(le == e)[0]
        codes = np.empty((2 * w.inter, w.hidden), np.uint8)
        codes[:, 0::2] = h13[e] & 15
        codes[:, 1::2] = h13[e] >> 4
        W = e2m1[codes] * np.repeat(np.exp2(h13s[e].astype(np.float64) - 127), 32, axis=1)
        wmax = np.abs(W).max(axis=1)
        gu = A[rs] @ W.T                                   # [n, 2I]
        g, u = gu[:, 0::2], gu[:, 1::2]
        amax = np.abs(A[rs]).max(axis=1, keepdims=True)
        dg = 2.0 ** -12 * KS * amax * wmax[None, 0::2]
        du = 2.0 ** -12 * KS * amax * wmax[None, 1::2]
        with np.errstate(over="ignore"):
            sig = 1.0 / (1.0 + np.exp(-g))
        silu = g * sig
        dsilu = sig * (1.0 + g * (1.0 - sig))
        out[rs] = np.abs(dsilu * u) * dg + np.abs(silu) * du + dg * du + 2.0 ** -20 * np.abs(silu * u)
    return out


def check_intermediate(layer, hidden, ids, routes, giq, gis):
    h13, h13s = layer.host[:2]
    riq, ris, h = oracle.intermediate(hidden, ids, h13, h13s, routes,
                                      expert_offset=layer.w.expert_offset, want_f64=True)
    budget = stage1_budget(layer, hidden, ids, routes)
    sd = gis.astype(np.int64) - ris.astype(np.int64)
    assert np.abs(sd).max(initial=0) <= 1, "block scales differ by more than one"
    if (sd != 0).any():
        hb = (np.abs(h) + budget).reshape(h.shape[0], -1, 32).max(axis=2)
        lo = np.maximum(np.abs(h) - budget, 0).reshape(h.shape[0], -1, 32).max(axis=2)
        # a power of two must lie within [lo, hb] of the exact block maximum
        crosses = np.floor(np.log2(np.maximum(lo, 1e-300))) != np.floor(np.log2(np.maximum(hb, 1e-300)))
        assert np.all(crosses[sd != 0]), "a block scale differs away from a power-of-two boundary"
    gv = _dequant(giq, gis)
    unit = np.repeat(np.exp2(gis.astype(np.float64) - 127), 32, axis=-1)
    reach = (np.abs(h) + budget) / unit
    step = np.where(reach < 2.0 ** -6, 2.0 ** -9,
                    np.exp2(np.floor(np.log2(np.maximum(reach, 2.0 ** -6))) - 3))
    allowed = budget + np.maximum(step, reach - 448.0 + 32.0) * unit
    err = np.abs(gv - h)
    bad = err > allowed * (1 + 1e-9)
    if bad.any():
        rows, cols = np.nonzero(bad)
        lines = []
        for r, c in list(zip(rows, cols))[:8]:
            lines.append("route %d j %d: exact %.6g gpu %.6g (code %#x scale %d) oracle code %#x "
                         "scale %d budget %.3g" % (routes[r], c, h[r, c], gv[r, c], giq[r, c],
                                                   gis[r, c // 32], riq[r, c], ris[r, c // 32],
                                                   budget[r, c]))
        raise AssertionError("%d intermediate elements outside budget + one FP8 step:\n  %s" % (
            bad.sum(), "\n  ".join(lines)))
    mism = float((giq != riq).mean())
    assert mism <= 0.02, "%.3f of intermediate codes differ from the correctly rounded ones" % mism
    return mism


def check_forward(layer, hidden, ids, wts, out_bits, xd, idd, tokens=None):
    """(a), (b) and (c) above for the listed tokens (all if None)."""
    w = layer.w
    M, k = ids.shape
    tok = np.arange(M, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    sorted_ids, giq, gis = gpu_intermediate(layer, xd, idd, M)
    routes = (tok[:, None] * k + np.arange(k)[None, :]).ravel()
    le = ids.ravel()[routes].astype(np.int64) - w.expert_offset
    local = (le >= 0) & (le < w.num_experts)
    pos = route_positions(sorted_ids, M, k, routes)
    assert np.all(pos[local] >= 0), "a local route is missing from the sort"
    # (a)
    mism = check_intermediate(layer, hidden, ids, routes[local], giq[pos[local]], gis[pos[local]]) \
        if local.any() else 0.0
    # (b)
    iq_t = np.zeros((len(routes), w.inter), np.uint8)
    is_t = np.full((len(routes), w.inter // 32), 127, np.uint8)
    iq_t[local] = giq[pos[local]]
    is_t[local] = gis[pos[local]]
    got = wl.bf16_to_f32(out_bits[tok])
    ref_b = oracle.forward_given_intermediate(ids, wts, layer.host[2], layer.host[3],
                                              iq_t.reshape(len(tok), k, -1), is_t.reshape(len(tok), k, -1),
                                              expert_offset=w.expert_offset, tokens=tok)
    assert_gate(got, wl.bf16_to_f32(ref_b), "output given the GPU intermediate")
    # (c)
    h13, h13s, h2, h2s = layer.host
    ref = oracle.forward(hidden, ids, wts, h13, h13s, h2, h2s, expert_offset=w.expert_offset, tokens=tok)
    frac = float(gate_failures(got, wl.bf16_to_f32(ref)).mean())
    note("  parity: %d tokens, intermediate code mismatch %.2e, end-to-end outside gate %.2e" % (
        len(tok), mism, frac))
    assert frac <= 0.01
