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
# accumulates in the MFMA (below FP32 precision) where the oracle uses FP64,
# so an element lying within that accumulation error of an FP8 rounding
# boundary may round to the neighbouring code, and a block maximum that close
# to a power of two may pick the neighbouring scale.  The checks therefore
# split the layer, on every listed token:
#   (a) the GPU intermediate must be a faithful rounding of the oracle's exact
#       FP64 SiLU(gate) * up, within a local error budget: the GPU's gate and
#       up sums carry an accumulation error of at most
#           (7 * 2^-13 + KS * 2^-20) * sum_k |a_k w_k|
#       -- the scaled MFMA sums each run of 8 products in a window 13
#       binades deep under the run's largest product, truncating the rest
#       (test_gpu_mfma.py measures this on the hardware), and the FP32
#       accumulation over the KS steps adds the second term --, propagated
#       through SiLU(g) * u (SiLU is 1.1-Lipschitz); every element must lie
#       within that budget plus one FP8 step of the exact value, block scales
#       must be equal or one apart only where the exact block maximum is
#       within the budget of a power of two, and at most MAX_CODE_FLIPS of
#       the codes may differ from the correctly rounded ones;
#   (b) given the GPU's intermediate, the output is unique: the oracle's stage
#       two and combine applied to it must match the GPU output at the gate,
#       on every element (for the numerical stress geometry: at the gate or
#       within stage two's own accumulation budget, whichever is larger);
#   (c) against the oracle end to end, every element outside the gate (for
#       the stress geometry: outside the gate and the budget) must belong to
#       a token one of whose routes has an intermediate code that differs
#       from the oracle's (a flipped code moves small outputs by about 0.03),
#       and at most MAX_E2E_MISS of the elements may be outside.

import json  # noqa: E402
import os  # noqa: E402

import oracle  # noqa: E402

MAX_CODE_FLIPS = 1e-3    # fraction of intermediate codes (measured 4e-4; at least 4 flips allowed)
MAX_E2E_MISS = 1e-2      # fraction of output elements (measured up to 5e-3, 4e-4 .. 9e-4 at full size)
ROUTES_PER_CHUNK = 8192  # oracle work per chunk of tokens (bounds host memory)
MFMA_RUN_ERR = 7 * 2.0 ** -13   # per run of 8 products, relative to the sum of |products|

_E4M3 = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _dequant(q, s):
    return _E4M3[q] * np.repeat(np.exp2(s.astype(np.float64) - 127), 32, axis=-1)


def log_rates(kind, rates):
    """Append the measured rates to $MOE_PARITY_LOG (JSON lines), if set."""
    path = os.environ.get("MOE_PARITY_LOG")
    if path:
        rec = dict(kind=kind, test=os.environ.get("PYTEST_CURRENT_TEST", ""), **rates)
        with open(path, "a") as f:
            f.write(json.dumps(rec) + "\n")


def stage1_budget(K, gu, gu_abs):
    """Per-element bound on |h_gpu - h_exact| (see (a) above) from the exact
    gate/up sums gu [n, 2I] and the sums of |a_k w_k| gu_abs [n, 2I]."""
    c = MFMA_RUN_ERR + (K // 128) * 2.0 ** -20
    g, u = gu[:, 0::2], gu[:, 1::2]
    dg, du = c * gu_abs[:, 0::2], c * gu_abs[:, 1::2]
    with np.errstate(over="ignore"):
        silu = g / (1.0 + np.exp(-g))
    return 1.1 * dg * (np.abs(u) + du) + np.abs(silu) * du + 2.0 ** -20 * np.abs(silu * u)


def stage2_budget(K, topk, out_abs, ref):
    """Bound on |out_gpu - out_exact| given the intermediate, from stage two's
    accumulation (as stage one's), the route-row encoding (2^-14 of a
    32-output block's largest magnitude per route), the FP32 sum over the
    slots and the final BF16 rounding.  out_abs: the oracle's sum over slots
    of |weight| * sum_j |inter_j w2[h, j]|."""
    c = MFMA_RUN_ERR + (K // 128) * 2.0 ** -20 + topk * 2.0 ** -24
    blk = np.repeat(out_abs.reshape(out_abs.shape[0], -1, 32).max(axis=2), 32, axis=1)
    return c * out_abs + topk * 2.0 ** -14 * blk + 2.0 ** -8 * np.abs(ref)


def check_intermediate(h, budget, riq, ris, giq, gis, routes):
    """(a) for n routes: exact h [n, I], budget [n, I], oracle codes riq/ris and
    GPU codes giq/gis.  Returns the number of codes differing from the oracle's."""
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
    return int((giq != riq).sum())


def check_routes_intermediate(layer, hidden, ids, routes, giq, gis, max_code_flips=MAX_CODE_FLIPS):
    """(a) for a list of local flat routes with the GPU's codes giq [n, I] and
    scales gis [n, I/32].  Returns the fraction of codes differing from the
    oracle's."""
    w = layer.w
    riq, ris, h, gu, gu_abs = oracle.intermediate(hidden, ids, layer.host[0], layer.host[1], routes,
                                                 expert_offset=w.expert_offset, want_f64=True, want_gu=True)
    flips = check_intermediate(h, stage1_budget(w.hidden, gu, gu_abs), riq, ris, giq, gis, routes)
    assert flips <= max(4, max_code_flips * giq.size), (flips, giq.size)
    return flips / max(giq.size, 1)


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


def check_forward(layer, hidden, ids, wts, out_bits, xd, idd, tokens=None, inter=None,
                  max_code_flips=MAX_CODE_FLIPS, max_e2e_miss=MAX_E2E_MISS, stage2_within_budget=False):
    """(a), (b) and (c) above for the listed tokens (all if None).  inter:
    the GPU's (sorted_ids, inter_q, inter_s) if already at hand, else it is
    recomputed through the step entry points.  stage2_within_budget: (b)
    accepts an element within stage two's accumulation budget when that is
    larger than the gate (the numerical stress geometry only).  Returns a
    dict of the rates."""
    w = layer.w
    M, k = ids.shape
    tok_all = np.arange(M, dtype=np.int64) if tokens is None else np.asarray(tokens, np.int64)
    sorted_ids, giq_all, gis_all = inter if inter is not None else gpu_intermediate(layer, xd, idd, M)
    h13, h13s, h2, h2s = layer.host
    got_all = wl.bf16_to_f32(out_bits)
    flips = codes = miss = elems = 0
    per_chunk = max(1, ROUTES_PER_CHUNK // k)
    for c0 in range(0, len(tok_all), per_chunk):
        tok = tok_all[c0:c0 + per_chunk]
        routes = (tok[:, None] * k + np.arange(k)[None, :]).ravel()
        le = ids.ravel()[routes].astype(np.int64) - w.expert_offset
        local = (le >= 0) & (le < w.num_experts)
        pos = route_positions(sorted_ids, M, k, routes)
        assert np.all(pos[local] >= 0), "a local route is missing from the sort"
        lr = routes[local]
        riq, ris, h, gu, gu_abs = oracle.intermediate(hidden, ids, h13, h13s, lr, expert_offset=w.expert_offset,
                                                     want_f64=True, want_gu=True)
        giq, gis = giq_all[pos[local]], gis_all[pos[local]]
        # (a)
        if len(lr):
            flips += check_intermediate(h, stage1_budget(w.hidden, gu, gu_abs), riq, ris, giq, gis, lr)
            codes += giq.size
        # (b)
        def per_slot(q_local, s_local):
            iq_t = np.zeros((len(routes), w.inter), np.uint8)
            is_t = np.full((len(routes), w.inter // 32), 127, np.uint8)
            iq_t[local] = q_local
            is_t[local] = s_local
            return iq_t.reshape(len(tok), k, -1), is_t.reshape(len(tok), k, -1)
        got = got_all[tok]
        if stage2_within_budget:
            ref_b, ref_b64, oab = oracle.forward_given_intermediate(
                ids, wts, h2, h2s, *per_slot(giq, gis), expert_offset=w.expert_offset, tokens=tok,
                want_f64=True, want_abs=True)
            outside = gate_failures(got, wl.bf16_to_f32(ref_b)) & ~(
                np.abs(got - ref_b64) <= stage2_budget(w.inter, k, oab, ref_b64))
            assert not outside.any(), "output given the GPU intermediate: %d of %d outside the gate " \
                "and stage two's budget" % (outside.sum(), outside.size)
        else:
            ref_b = oracle.forward_given_intermediate(ids, wts, h2, h2s, *per_slot(giq, gis),
                                                      expert_offset=w.expert_offset, tokens=tok)
            assert_gate(got, wl.bf16_to_f32(ref_b), "output given the GPU intermediate")
        # (c): the oracle's own output is its stage two and combine on its own
        # intermediate (the same as oracle.forward, pinned in the CPU tests)
        if stage2_within_budget:
            ref, ref64, oab = oracle.forward_given_intermediate(
                ids, wts, h2, h2s, *per_slot(riq, ris), expert_offset=w.expert_offset, tokens=tok,
                want_f64=True, want_abs=True)
            bad = gate_failures(got, wl.bf16_to_f32(ref)) & ~(
                np.abs(got - ref64) <= stage2_budget(w.inter, k, oab, ref64))
        else:
            ref = oracle.forward_given_intermediate(ids, wts, h2, h2s, *per_slot(riq, ris),
                                                    expert_offset=w.expert_offset, tokens=tok)
            bad = gate_failures(got, wl.bf16_to_f32(ref))
        if bad.any():
            differs = np.zeros(len(routes), bool)
            differs[local] = (giq != riq).any(axis=1) | (gis != ris).any(axis=1)
            unexplained = bad.any(axis=1) & ~differs.reshape(len(tok), k).any(axis=1)
            assert not unexplained.any(), (
                "tokens %s miss the gate end to end with the oracle's own intermediate" %
                tok[unexplained][:8].tolist())
        miss += int(bad.sum())
        elems += bad.size
    rates = dict(tokens=len(tok_all), code_flips=flips / max(codes, 1), flips=flips,
                 e2e_miss=miss / max(elems, 1))
    note("  parity: %d tokens, intermediate code flips %.2e, end-to-end outside gate %.2e" % (
        rates["tokens"], rates["code_flips"], rates["e2e_miss"]))
    log_rates("a8w4", rates)
    assert flips <= max(4, max_code_flips * codes), rates
    assert rates["e2e_miss"] <= max_e2e_miss, rates
    return rates
