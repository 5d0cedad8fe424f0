"""The GPU parity checker (gpu_util.check_forward) exercised on the CPU: fed
the oracle's own sort, intermediate and output in place of the GPU's, it must
pass with no code flips and no misses; fed results with a planted mistake (a
shifted intermediate code, a wrong output element, a missing route, a block
scale off by one away from a power-of-two boundary) it must fail.  No GPU is
involved: the "device" results here come from the oracle."""
import numpy as np
import pytest

import oracle
from mixture_experts_fp8_amd import workloads as wl
import gpu_util


class HostLayer:
    """The parts of gpu_util.Layer the checker reads: the workload and the
    host weights."""

    def __init__(self, w):
        self.w = w
        self.host = wl.make_weights(w)


def oracle_results(layer, M, mode="softmax"):
    w = layer.w
    hidden, ids, wts = wl.make_inputs(w, M, mode)
    bm = 16
    sorted_ids, _ = oracle.sort(ids, w.num_experts, w.expert_offset, bm)
    real = np.nonzero(sorted_ids != M)[0]
    routes = (sorted_ids[real] & 0xFFFFFF).astype(np.int64) * w.topk + (sorted_ids[real] >> 24)
    riq, ris = oracle.intermediate(hidden, ids, *layer.host[:2], routes, expert_offset=w.expert_offset)
    iq = np.zeros((len(sorted_ids), w.inter), np.uint8)
    is_ = np.zeros((len(sorted_ids), w.inter // 32), np.uint8)
    iq[real], is_[real] = riq, ris
    out = oracle.forward(hidden, ids, wts, *layer.host, expert_offset=w.expert_offset)
    return hidden, ids, wts, out, (sorted_ids, iq, is_)


@pytest.fixture(scope="module")
def case():
    w = wl.scaled(wl.WORKLOADS["draft-sweep"], hidden=512, inter=128, inter_valid=96, num_experts=6,
                  routed_experts=6, config_id=880)
    layer = HostLayer(w)
    return layer, oracle_results(layer, 24)


def run(layer, res, **kw):
    hidden, ids, wts, out, inter = res
    return gpu_util.check_forward(layer, hidden, ids, wts, out, None, None, inter=inter, **kw)


def test_oracle_results_pass(case):
    layer, res = case
    rates = run(layer, res)
    assert rates["code_flips"] == 0 and rates["e2e_miss"] == 0 and rates["tokens"] == 24


def test_chunking_does_not_change_the_outcome(case, monkeypatch):
    layer, res = case
    monkeypatch.setattr(gpu_util, "ROUTES_PER_CHUNK", 7)
    assert run(layer, res)["tokens"] == 24


def test_shifted_intermediate_code_fails(case):
    layer, (hidden, ids, wts, out, (srt, iq, is_)) = case
    iq2 = iq.copy()
    p = int(np.nonzero(srt != ids.shape[0])[0][3])
    j = int(np.argmax(np.abs(iq2[p].astype(np.int16) & 0x7F)))   # a large code, far from any tie
    iq2[p, j] = (iq2[p, j] & 0x80) | ((iq2[p, j] & 0x7F) - 4)
    with pytest.raises(AssertionError, match="outside budget"):
        run(layer, (hidden, ids, wts, out, (srt, iq2, is_)))


def test_scale_off_by_one_fails(case):
    layer, (hidden, ids, wts, out, (srt, iq, is_)) = case
    is2 = is_.copy()
    p = int(np.nonzero(srt != ids.shape[0])[0][0])
    is2[p, 0] += 1
    with pytest.raises(AssertionError):
        run(layer, (hidden, ids, wts, out, (srt, iq, is2)))


def test_wrong_output_element_fails(case):
    layer, (hidden, ids, wts, out, inter) = case
    out2 = out.copy()
    v = wl.bf16_to_f32(out2[5, 100:101])
    out2[5, 100] = wl.bf16_bits(v * 1.1 + 0.1)[0]
    with pytest.raises(AssertionError, match="given the GPU intermediate"):
        run(layer, (hidden, ids, wts, out2, inter))


def test_missing_route_fails(case):
    layer, (hidden, ids, wts, out, (srt, iq, is_)) = case
    srt2 = srt.copy()
    srt2[int(np.nonzero(srt != ids.shape[0])[0][2])] = ids.shape[0]
    with pytest.raises(AssertionError, match="missing from the sort"):
        run(layer, (hidden, ids, wts, out, (srt2, iq, is_)))


def test_budget_pinned_by_a_closed_form():
    """The stage-one budget for gate g and up u with accumulation errors
    dg = c sum|a w|_g, du = c sum|a w|_u (c = 7 * 2^-13 + (K/128) 2^-20):
    1.1 dg (|u| + du) + |SiLU(g)| du + 2^-20 |SiLU(g) u|.  At g = 0, SiLU(0) = 0,
    so it is 1.1 dg (|u| + du); at large g, SiLU(g) = g."""
    K = 1024
    c = 7 * 2.0 ** -13 + 8 * 2.0 ** -20
    gu = np.array([[0.0, 3.0, 50.0, -2.0]])          # (g, u) = (0, 3) and (50, -2)
    gu_abs = np.array([[10.0, 20.0, 100.0, 40.0]])
    b = gpu_util.stage1_budget(K, gu, gu_abs)
    want0 = 1.1 * c * 10 * (3 + c * 20)
    want1 = 1.1 * c * 100 * (2 + c * 40) + 50 * c * 40 + 2.0 ** -20 * 100
    np.testing.assert_allclose(b, [[want0, want1]], rtol=1e-12)


def test_stage2_budget_closed_form():
    """Stage two's budget: c * out_abs + topk * 2^-14 * (the 32-block maximum of
    out_abs) + 2^-8 |ref|, c = 7 * 2^-13 + (K/128) 2^-20 + topk 2^-24."""
    out_abs = np.zeros((1, 64))
    out_abs[0, 5] = 8.0
    out_abs[0, 40] = 2.0
    ref = np.full((1, 64), 4.0)
    b = gpu_util.stage2_budget(640, 3, out_abs, ref)
    c = 7 * 2.0 ** -13 + 5 * 2.0 ** -20 + 3 * 2.0 ** -24
    assert b[0, 0] == 3 * 2.0 ** -14 * 8 + 2.0 ** -8 * 4
    np.testing.assert_allclose(b[0, 5], c * 8 + 3 * 2.0 ** -14 * 8 + 2.0 ** -8 * 4, rtol=1e-15)
    np.testing.assert_allclose(b[0, 33], 3 * 2.0 ** -14 * 2 + 2.0 ** -8 * 4, rtol=1e-15)
