"""GPU checks of the fused decode launch moe_a8w4_stages_fused (stage one,
stage two and the top-k combine in one kernel, blocks of 16 or 32 routes),
an export beside moe_a8w4_forward (which runs separate launches).  It runs
the same tile arithmetic as the separate stage launches, so its
intermediate, its route rows and its output must equal theirs bit for bit;
its output is also checked against the oracle on every token (the gate of
the pages' validation, with the two-part check of gpu_util.check_forward on
the fused launch's own intermediate).  Its cross-workgroup counters are left
zero and its status word 0 after every call, so back-to-back calls on one
counters buffer stay correct."""
import numpy as np
import pytest
import torch

from mixture_experts_fp8_amd import abi, workloads as wl
from gpu_util import DEV, Layer, check_forward, dev, host_bf16_bits, note

pytestmark = pytest.mark.gpu

# (workload, experts held, experts routed over, tokens, routing); block_m is
# the library's choice: 16 or 32 in every case (the last column of the note)
CASES = [
    ("draft-decode", 8, 8, 5, "softmax"),
    ("backbone-decode", 24, 24, 31, "softmax"),
    ("backbone-decode", 24, 24, 60, "softmax"),
    ("draft-sweep", 16, 16, 40, "concentrated"),
    ("local-slice", 8, 32, 16, "softmax"),      # K = 2304: stage two split over the waves
    ("local-slice", 8, 32, 64, "softmax"),      # block_m 32 at K = 2304
    ("prefill-shared", 9, 8, 12, "roundrobin"),
]


def step_path(layer, d, bm, xd, idd, wd):
    """The separate launches: quantise + sort, stage one, stage two, combine."""
    q, s, srt, bexp, npad = abi.moe_a8w4_quant_sort(d, bm, xd, idd)
    iq, is_ = abi.moe_a8w4_stage1(d, bm, q, s, srt, bexp, npad, layer.packed[0], layer.packed[1])
    y = torch.zeros(abi.route_rows_bytes(d), dtype=torch.uint8, device=DEV)
    abi.moe_a8w4_stage2(d, bm, iq, is_, srt, bexp, npad, wd, layer.packed[2], layer.packed[3], y)
    out = abi.moe_a8w4_combine(d, idd, y)
    return q, s, srt, bexp, npad, iq, is_, y, out


def compare(d, bm, ref, got_iq, got_is, got_y, got_out, ids, E, offset):
    q, s, srt, bexp, npad, iq, is_, y, out = ref
    P = int(npad.item())
    sid = srt[:P].cpu().numpy()
    real = np.nonzero(sid != d.tokens)[0]
    assert np.array_equal(got_iq[:P].cpu().numpy()[real], iq[:P].cpu().numpy()[real])
    assert np.array_equal(got_is[:P].cpu().numpy()[real], is_[:P].cpu().numpy()[real])
    M, k, H = d.tokens, d.topk, d.hidden
    local = ((ids - offset >= 0) & (ids - offset < E)).ravel()
    yr, yg = y.cpu().numpy(), got_y.cpu().numpy()
    codes_r, codes_g = yr[:M * k * H * 2].reshape(M * k, -1), yg[:M * k * H * 2].reshape(M * k, -1)
    exps_r, exps_g = yr[M * k * H * 2:].reshape(M * k, -1), yg[M * k * H * 2:].reshape(M * k, -1)
    assert np.array_equal(codes_r[local], codes_g[local])
    assert np.array_equal(exps_r[local], exps_g[local])
    assert torch.equal(out.view(torch.int16), got_out.view(torch.int16))


@pytest.mark.parametrize("name,E,routed,M,mode", CASES)
def test_fused_equals_separate_launches(name, E, routed, M, mode):
    base = wl.WORKLOADS[name]
    w = wl.scaled(base, num_experts=E, routed_experts=routed, config_id=300 + M)
    layer = Layer(w)
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    note("fused vs separate %s E=%d routed=%d M=%d %s bm=%d" % (name, E, routed, M, mode, bm))
    assert bm in (16, 32)
    n = abi.moe_a8w4_fused_counters(d, bm)
    counters = torch.zeros(n, dtype=torch.int32, device=DEV)
    # three calls in a row on one counters buffer, each on new inputs
    for rep in range(3):
        hidden, ids, wts = wl.make_inputs(w, M, mode, seed=[rep])
        xd, idd, wd = dev(hidden), dev(ids), dev(wts)
        ref = step_path(layer, d, bm, xd, idd, wd)
        q, s, srt, bexp, npad = ref[:5]
        y = torch.zeros(abi.route_rows_bytes(d), dtype=torch.uint8, device=DEV)
        out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
        iq, is_, y, out = abi.moe_a8w4_stages_fused(d, bm, q, s, srt, bexp, npad, idd, wd, *layer.packed,
                                                    counters, y_routes=y, out=out)
        torch.cuda.synchronize()
        assert not counters.any(), "rep %d: counters not cleared: status %d, %d nonzero" % (
            rep, int(counters[0]), int((counters != 0).sum()))
        compare(d, bm, ref, iq, is_, y, out, ids, w.num_experts, w.expert_offset)
        # the whole layer through moe_a8w4_forward: the same output
        fwd = layer.forward(xd, idd, wd)
        torch.cuda.synchronize()
        assert torch.equal(fwd.view(torch.int16), out.view(torch.int16))
        # and the fused launch's output against the oracle, every token
        P = int(npad.item())
        inter = (srt[:P].cpu().numpy(), iq[:P].cpu().numpy(), is_[:P].cpu().numpy())
        check_forward(layer, hidden, ids, wts, host_bf16_bits(out), xd, idd, inter=inter)


FULL = [("backbone-decode", 6), ("backbone-decode", 768), ("local-slice", 1), ("local-slice", 256)]


@pytest.fixture(scope="module")
def full_layers():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[name] = Layer(wl.WORKLOADS[name])
        return cache[name]

    yield get
    cache.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name,M", FULL)
def test_fused_full_size(name, M, full_layers):
    """The real geometries (384 experts at I 640; 96 local experts at I 2304):
    the fused launch against the separate launches, bit for bit, and against
    the oracle on every token."""
    w = wl.WORKLOADS[name]
    layer = full_layers(name)
    hidden, ids, wts = wl.make_inputs(w, M, w.routings[0])
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    note("fused full size %s M=%d bm=%d" % (name, M, bm))
    xd, idd, wd = dev(hidden), dev(ids), dev(wts)
    ref = step_path(layer, d, bm, xd, idd, wd)
    q, s, srt, bexp, npad = ref[:5]
    counters = torch.zeros(abi.moe_a8w4_fused_counters(d, bm), dtype=torch.int32, device=DEV)
    iq, is_, y, out = abi.moe_a8w4_stages_fused(d, bm, q, s, srt, bexp, npad, idd, wd, *layer.packed,
                                                counters)
    torch.cuda.synchronize()
    assert not counters.any()
    compare(d, bm, ref, iq, is_, y, out, ids, w.num_experts, w.expert_offset)
    P = int(npad.item())
    inter = (srt[:P].cpu().numpy(), iq[:P].cpu().numpy(), is_[:P].cpu().numpy())
    check_forward(layer, hidden, ids, wts, host_bf16_bits(out), xd, idd, inter=inter)
