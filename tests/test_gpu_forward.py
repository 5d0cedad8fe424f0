"""GPU parity of the whole layer through the C ABI against the oracle, at the
gate of the pages' validation (atol = rtol = 2e-2, all outputs finite), on
every token: small geometries, every point of the five workloads at full size
(with the pages' boundary token counts), a numerical stress geometry, edge
cases, input preservation, the step entry points, and replays of a captured
graph on changed inputs."""
import numpy as np
import pytest
import torch

from mixture_experts_fp8_amd import abi, workloads as wl
import oracle
from gpu_util import DEV, Layer, assert_gate, check_forward, dev, host_bf16_bits, note

pytestmark = pytest.mark.gpu


SMALL = [
    ("draft-decode", 8, 5, "softmax"),
    ("draft-decode", 8, 1, "softmax"),
    ("draft-sweep", 12, 40, "concentrated"),
    ("backbone-decode", 24, 31, "softmax"),
    ("backbone-decode", 24, 33, "softmax"),
    ("backbone-decode", 24, 200, "softmax"),
    ("backbone-decode", 24, 257, "softmax"),
    ("local-slice", 8, 16, "softmax"),
    ("prefill-shared", 9, 70, "roundrobin"),
]


@pytest.mark.parametrize("name,E,M,mode", SMALL)
def test_forward_small_all_tokens(name, E, M, mode):
    base = wl.WORKLOADS[name]
    routed = E - 1 if base.shared else E
    w = wl.scaled(base, num_experts=E, routed_experts=routed, config_id=100 + E)
    if name == "local-slice":
        w = wl.scaled(w, routed_experts=4 * E)   # a quarter of the routes are local
    layer = Layer(w)
    hidden, ids, wts = wl.make_inputs(w, M, mode)
    note("forward %s E=%d M=%d %s bm=%d" % (name, E, M, mode, abi.moe_a8w4_block_m(layer.dims(M))))
    out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    xd, idd = dev(hidden), dev(ids)
    layer.forward(xd, idd, wts, out=out)
    torch.cuda.synchronize()
    check_forward(layer, hidden, ids, wts, host_bf16_bits(out), xd, idd)


# Every point of the five workloads, each token checked against the oracle:
# the draft decode call; the backbone decode buckets and the boundary token
# counts of the pages' validation (aiter PR 5609, "Validation and limits":
# M 31/32/33/255/256/257 in each geometry); the draft sweep under both
# routings plus the boundary counts; the local-slice token counts of the
# pages' benchmark table (aiter PR 5904, "Fused-MoE kernel, expert-parallel
# benchmark") plus the boundary counts; the prefill geometry with the shared
# expert under both routings; and the numerical stress geometry.
BOUNDARY = (31, 32, 33, 255, 256, 257)
FULL = ([("draft-decode", 5, "softmax")]
        + [("backbone-decode", M, "softmax") for M in wl.BACKBONE_DECODE_BUCKETS + BOUNDARY]
        + [("draft-sweep", M, mode) for mode in ("softmax", "concentrated")
           for M in wl.WORKLOADS["draft-sweep"].tokens]
        + [("draft-sweep", M, "softmax") for M in BOUNDARY]
        + [("local-slice", M, "softmax") for M in wl.WORKLOADS["local-slice"].tokens + BOUNDARY]
        + [("prefill-shared", M, mode) for M in (4096, 16384) for mode in ("roundrobin", "softmax")]
        + [("wide-scale", M, "softmax") for M in wl.WORKLOADS["wide-scale"].tokens])


@pytest.fixture(scope="module")
def layers():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            cache[name] = Layer(wl.WORKLOADS[name])
        return cache[name]

    yield get
    cache.clear()


@pytest.mark.parametrize("name,M,mode", FULL)
def test_forward_full_size_every_token(layers, name, M, mode):
    layer = layers(name)
    w = layer.w
    hidden, ids, wts = wl.make_inputs(w, M, mode)
    note("forward full %s M=%d %s bm=%d" % (name, M, mode, abi.moe_a8w4_block_m(layer.dims(M))))
    out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    xd, idd, wd = dev(hidden), dev(ids), dev(wts)
    layer.forward(xd, idd, wd, out=out)
    torch.cuda.synchronize()
    bits = host_bf16_bits(out)
    vals = wl.bf16_to_f32(bits)
    assert np.isfinite(vals).all()
    # tokens with no local route are exact zeros
    le = ids.astype(np.int64) - w.expert_offset
    none_local = ~((le >= 0) & (le < w.num_experts)).any(axis=1)
    assert np.all(vals[none_local] == 0)
    # the sort at full size, bit for bit
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, idd)
    torch.cuda.synchronize()
    ref_sorted, ref_bexp = oracle.sort(ids, w.num_experts, w.expert_offset, bm)
    P = int(npad.item())
    assert P == len(ref_sorted)
    assert np.array_equal(srt[:P].cpu().numpy(), ref_sorted)
    assert np.array_equal(bexp[:P // bm].cpu().numpy(), ref_bexp)
    # every token against the oracle (the stress geometry's outputs reach
    # 2^90 with heavy cancellation: stage two is held to its own budget there)
    check_forward(layer, hidden, ids, wts, bits, xd, idd, stage2_within_budget=(name == "wide-scale"))
    # inputs unchanged
    assert np.array_equal(host_bf16_bits(xd), hidden)
    assert np.array_equal(idd.cpu().numpy(), ids)
    assert np.array_equal(wd.cpu().numpy(), wts)


TILE_SHAPES = [  # (hidden, inter, experts, topk, tokens): block_m 64/128 with short and odd K
    (512, 128, 4, 2, 300),    # stage two has a single K step
    (1024, 384, 3, 1, 200),   # stage two has three K steps (ring of three)
    (512, 256, 8, 2, 150),    # block_m 64, two K steps in stage two
    (8704, 256, 2, 1, 300),   # block_m 128, long K (68 steps in stage one)
    (16896, 128, 4, 1, 150),  # block_m 64, token scales too many to preload (K > 16384)
    # token-resident kernel (the block's tokens stay in LDS, 4 or 5 weight slices per workgroup)
    (1024, 640, 4, 2, 150),   # block_m 128, stage two resident at the size limit (128 x 640)
    (1024, 512, 4, 2, 70),    # block_m 64, both stages resident, 4 slices
    (512, 640, 4, 2, 150),    # block_m 128, stage one resident with 5 slices (N = 1280)
]


@pytest.mark.parametrize("H,I,E,k,M", TILE_SHAPES)
def test_tile_kernel_short_and_odd_k(H, I, E, k, M):
    base = wl.WORKLOADS["draft-decode"]
    w = wl.scaled(base, hidden=H, inter=I, inter_valid=I, num_experts=E, routed_experts=E, topk=k,
                  config_id=200 + H + I + E)
    layer = Layer(w)
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    bm = abi.moe_a8w4_block_m(layer.dims(M))
    assert bm >= 64
    note("tile kernel H=%d I=%d E=%d k=%d M=%d bm=%d" % (H, I, E, k, M, bm))
    out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    xd, idd = dev(hidden), dev(ids)
    layer.forward(xd, idd, wts, out=out)
    torch.cuda.synchronize()
    check_forward(layer, hidden, ids, wts, host_bf16_bits(out), xd, idd)


@pytest.mark.parametrize("M", [40, 2100, 4000])
def test_forward_most_experts_and_slots(M):
    """The largest expert count (512) and top-k (8) the library takes, at
    blocks of 16, 64 and 128 routes (mean routes per expert 0.6, 33, 63),
    every token against the oracle."""
    base = wl.WORKLOADS["backbone-decode"]
    w = wl.scaled(base, hidden=512, inter=128, inter_valid=128, num_experts=512, routed_experts=512, topk=8,
                  config_id=500)
    layer = Layer(w)
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    note("most experts and slots M=%d bm=%d" % (M, bm))
    out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    xd, idd = dev(hidden), dev(ids)
    layer.forward(xd, idd, wts, out=out)
    torch.cuda.synchronize()
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, idd)
    torch.cuda.synchronize()
    ref_sorted, ref_bexp = oracle.sort(ids, w.num_experts, w.expert_offset, bm)
    P = int(npad.item())
    assert P == len(ref_sorted)
    assert np.array_equal(srt[:P].cpu().numpy(), ref_sorted)
    assert np.array_equal(bexp[:P // bm].cpu().numpy(), ref_bexp)
    check_forward(layer, hidden, ids, wts, host_bf16_bits(out), xd, idd)


def test_edge_cases():
    w = wl.scaled(wl.WORKLOADS["backbone-decode"], num_experts=12, routed_experts=12, config_id=120)
    layer = Layer(w)
    M = 9
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    # a token whose routes are all non-local, negative and too-large ids, a duplicate
    ids = ids.copy()
    ids[0, :] = -1
    ids[1, 2] = 500
    ids[2, 1] = ids[2, 0]
    note("edge cases M=%d" % M)
    xd, idd = dev(hidden), dev(ids)
    out = layer.forward(xd, idd, wts)
    torch.cuda.synchronize()
    bits = host_bf16_bits(out)
    assert np.all(bits[0] == 0)
    check_forward(layer, hidden, ids, wts, bits, xd, idd)
    # expert_offset: the same experts addressed as a slice at 192
    w2 = wl.scaled(w, expert_offset=192)
    layer2 = Layer(w2, weights=layer.host)
    out2 = layer2.forward(hidden, np.where(ids >= 0, ids + 192, ids).astype(np.int32), wts)
    torch.cuda.synchronize()
    assert_gate(wl.bf16_to_f32(host_bf16_bits(out2)), wl.bf16_to_f32(bits), "offset")
    # M = 0 is a no-op
    d0 = layer.dims(0)
    assert abi.load().moe_a8w4_forward(d0, *([None] * 9), 0, None) == abi.MOE_OK


@pytest.mark.parametrize("E,M,want_bm", [(16, 80, 32), (16, 200, 64), (8, 400, 128)])
def test_steps_compose_to_forward(E, M, want_bm):
    """The step entry points (stage two writing route rows, then the separate
    combine) give the forward's output bit for bit, at blocks of 32, 64 and
    128 routes."""
    w = wl.scaled(wl.WORKLOADS["draft-sweep"], num_experts=E, routed_experts=E, config_id=121)
    layer = Layer(w)
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    assert bm == want_bm
    note("steps M=%d bm=%d" % (M, bm))
    xd, idd, wd = dev(hidden), dev(ids), dev(wts)
    q, s = abi.moe_a8w4_quant_act(xd)
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, idd)
    iq, is_ = abi.moe_a8w4_stage1(d, bm, q, s, srt, bexp, npad, layer.packed[0], layer.packed[1])
    y = abi.moe_a8w4_stage2(d, bm, iq, is_, srt, bexp, npad, wd, layer.packed[2], layer.packed[3])
    out_steps = abi.moe_a8w4_combine(d, idd, y)
    out_fwd = layer.forward(xd, idd, wd)
    out_again = layer.forward(xd, idd, wd)
    q2, s2, srt2, bexp2, npad2 = abi.moe_a8w4_quant_sort(d, bm, xd, idd)
    torch.cuda.synchronize()
    P = int(npad.item())
    assert int(npad2.item()) == P
    assert torch.equal(q2, q) and torch.equal(s2, s)
    assert torch.equal(srt2[:P], srt[:P]) and torch.equal(bexp2[:P // bm], bexp[:P // bm])
    # same kernels in the same order, no atomics: bitwise equal, and repeatable
    assert torch.equal(out_steps.view(torch.int16), out_fwd.view(torch.int16))
    assert torch.equal(out_again.view(torch.int16), out_fwd.view(torch.int16))
    check_forward(layer, hidden, ids, wts, host_bf16_bits(out_fwd), xd, idd)


def shared_layer():
    """A small layer with the prefill configuration's fused shared expert:
    8 routed experts top-2 plus the shared one (local expert 8) in the last
    slot, I = 640."""
    w = wl.scaled(wl.WORKLOADS["prefill-shared"], hidden=1024, num_experts=9, routed_experts=8, topk=3,
                  config_id=901)
    return w, Layer(w)


def edit_shared_routes(w, ids, duplicates):
    """Tokens that break the shared-expert pattern: no shared slot, the
    shared expert twice, the shared expert first, only the shared slot local,
    no local slot, an out-of-range routed id; `duplicates` more tokens with
    the shared expert in two slots."""
    x = w.routed_experts
    ids = ids.copy()
    ids[0, 2] = (ids[0, 0] + 1) % x if (ids[0, 0] + 1) % x != ids[0, 1] else (ids[0, 0] + 2) % x
    ids[1, 0] = x
    ids[2, [0, 2]] = ids[2, [2, 0]]
    ids[3, :2] = -1
    ids[4, :] = -1
    ids[5, 1] = 500
    ids[6:6 + duplicates, 1] = x
    return ids


@pytest.mark.parametrize("M,duplicates", [(20, 0), (40, 0), (100, 0), (400, 0), (400, 150), (40, 30), (20, 12)])
def test_shared_expert_routes(M, duplicates):
    """The prefill configuration's fused shared expert, with tokens that
    break its pattern (no shared slot, the shared expert twice or first, only
    the shared slot local, none local, an out-of-range id) and with many
    tokens holding it twice (its sorted run then longer than M): at every
    block size moe_a8w4_forward gives the step entry points' output bit for
    bit, repeatably, zeros for the token with no local slot, and the
    oracle's gate on every token."""
    w, layer = shared_layer()
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    ids = edit_shared_routes(w, ids, duplicates)
    d = layer.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    note("shared-expert routes M=%d bm=%d duplicates=%d" % (M, bm, duplicates))
    xd, idd, wd = dev(hidden), dev(ids), dev(wts)
    q, s = abi.moe_a8w4_quant_act(xd)
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, idd)
    iq, is_ = abi.moe_a8w4_stage1(d, bm, q, s, srt, bexp, npad, layer.packed[0], layer.packed[1])
    y = abi.moe_a8w4_stage2(d, bm, iq, is_, srt, bexp, npad, wd, layer.packed[2], layer.packed[3])
    out_steps = abi.moe_a8w4_combine(d, idd, y)
    out_fwd = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    layer.forward(xd, idd, wd, out=out_fwd)
    out_again = layer.forward(xd, idd, wd)
    torch.cuda.synchronize()
    assert torch.equal(out_steps.view(torch.int16), out_fwd.view(torch.int16))
    assert torch.equal(out_again.view(torch.int16), out_fwd.view(torch.int16))
    bits = host_bf16_bits(out_fwd)
    assert np.all(bits[4] == 0)
    check_forward(layer, hidden, ids, wts, bits, xd, idd)


def test_shared_expert_block_sizes_covered():
    """The token counts of test_shared_expert_routes reach every block size."""
    w, _ = shared_layer()
    bms = {abi.moe_a8w4_block_m(abi.make_dims(M, w.hidden, w.inter, w.num_experts, w.topk, w.expert_offset,
                                               w.routed_experts)) for M in (20, 40, 100, 400)}
    assert bms == {16, 32, 64, 128}


def test_graph_replay_on_changed_inputs():
    """Capture one call; replay it on original, changed, concentrated and
    restored inputs written into the captured buffers; each replay matches
    the eager call on the same inputs and the oracle."""
    w = wl.scaled(wl.WORKLOADS["draft-sweep"], num_experts=16, routed_experts=16, config_id=122)
    layer = Layer(w)
    M = 40
    cases = {
        "original": wl.make_inputs(w, M, "softmax", seed=[1]),
        "changed": wl.make_inputs(w, M, "softmax", seed=[2]),
        "concentrated": wl.make_inputs(w, M, "concentrated", seed=[3]),
    }
    cases["restored"] = cases["original"]
    d = layer.dims(M)
    ws = torch.empty(abi.moe_a8w4_workspace_bytes(d), dtype=torch.uint8, device=DEV)
    xd, idd, wd = dev(cases["original"][0]), dev(cases["original"][1]), dev(cases["original"][2])
    out = torch.empty((M, w.hidden), dtype=torch.bfloat16, device=DEV)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer.forward(xd, idd, wd, out=out, workspace=ws)      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.forward(xd, idd, wd, out=out, workspace=ws)
    torch.cuda.synchronize()
    for name, (h, i, wt) in cases.items():
        note("graph replay %s" % name)
        xd.copy_(dev(h))
        idd.copy_(dev(i))
        wd.copy_(dev(wt))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        eager = layer.forward(dev(h), dev(i), dev(wt)).float().cpu().numpy()
        torch.cuda.synchronize()
        assert np.array_equal(got, eager), name     # the call is deterministic
        check_forward(layer, h, i, wt, host_bf16_bits(out), xd, idd)
