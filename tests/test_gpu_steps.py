"""GPU parity of the single steps through the C ABI: activation quantisation
and the sort bit-exact against the oracle, the weight packing against its
stated permutation, and the stage-one intermediate within one FP8 quantum."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_fp8_amd import abi, workloads as wl
from gpu_util import DEV, MFMA_RUN_ERR, Layer, _E4M3, check_routes_intermediate, dev, note

pytestmark = pytest.mark.gpu


def finite_bf16_blocks(cols, seed=0):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(seed)
    bits = rng.permutation(bits)
    n = (len(bits) + cols - 1) // cols * cols
    out = np.zeros(n, np.uint16)
    out[: len(bits)] = bits
    return out.reshape(-1, cols)


@pytest.mark.parametrize("case", ["exhaustive-bf16", "normal-257x5120", "ones-3x512"])
def test_quant_act_bit_exact(case):
    if case == "exhaustive-bf16":
        x = finite_bf16_blocks(1024)
    elif case == "normal-257x5120":
        x = wl.make_hidden(np.random.default_rng(3), 257, 5120)
    else:
        x = wl.bf16_bits(np.ones((3, 512), np.float32))
    note("quant_act %s %s" % (case, x.shape))
    xd = dev(x)
    q, s = abi.moe_a8w4_quant_act(xd)
    torch.cuda.synchronize()
    rq, rs = oracle.quant_act(x)
    assert np.array_equal(q.cpu().numpy(), rq)
    assert np.array_equal(s.cpu().numpy(), rs)


SORT_CASES = []
for name, Ms in [("backbone-decode", (1, 6, 31, 32, 33, 255, 256, 257, 768)),
                 ("draft-sweep", (5, 640)), ("local-slice", (16, 4096, 16384)),
                 ("prefill-shared", (4096, 16384))]:
    for M in Ms:
        for bm in (16, 32, 64, 128):
            SORT_CASES.append((name, M, bm))


@pytest.mark.parametrize("name,M,bm", SORT_CASES)
def test_sort_bit_exact(name, M, bm):
    w = wl.WORKLOADS[name]
    mode = w.routings[-1]
    _, ids, _ = wl.make_inputs(wl.scaled(w, hidden=32), M, mode)
    note("sort %s M=%d bm=%d mode=%s" % (name, M, bm, mode))
    d = abi.make_dims(M, 5120, 640, w.num_experts, w.topk, w.expert_offset)
    s, b, n = abi.moe_a8w4_sort(d, bm, dev(ids))
    torch.cuda.synchronize()
    rs, rb = oracle.sort(ids, w.num_experts, w.expert_offset, bm)
    P = int(n.item())
    assert P == len(rs)
    assert np.array_equal(s[:P].cpu().numpy(), rs)
    assert np.array_equal(b[: P // bm].cpu().numpy(), rb)


def test_sort_nonlocal_duplicates_offset_and_repeatability():
    rng = np.random.default_rng(8)
    M, k, E, off, bm = 300, 6, 96, 192, 32
    ids = rng.integers(-10, 500, size=(M, k)).astype(np.int32)
    ids[5, 1] = ids[5, 0]
    ids[7, :] = 1000                       # a token with no local route
    d = abi.make_dims(M, 5120, 640, E, k, off)
    rs, rb = oracle.sort(ids, E, off, bm)
    idd = dev(ids)
    first = None
    for rep in range(20):
        s, b, n = abi.moe_a8w4_sort(d, bm, idd)
        torch.cuda.synchronize()
        P = int(n.item())
        got = (s[:P].cpu().numpy(), b[: P // bm].cpu().numpy())
        assert np.array_equal(got[0], rs) and np.array_equal(got[1], rb)
        if first is None:
            first = got
    # no local route at all
    s, b, n = abi.moe_a8w4_sort(d, bm, dev(np.full((M, k), 5, np.int32)))
    torch.cuda.synchronize()
    assert int(n.item()) == 0


@pytest.mark.parametrize("bm", [16, 128])
def test_sort_skewed_across_chunks(bm):
    """Routes are split into chunks sorted by separate workgroups: one expert
    holding most routes spans all chunks, others are empty or tiny, and some
    routes are not local."""
    rng = np.random.default_rng(11)
    M, k, E, off = 20000, 6, 40, 8
    ids = rng.integers(0, 64, size=(M, k)).astype(np.int32)
    hot = rng.random((M, k)) < 0.7
    ids[hot] = off + 3
    ids[:, 0] = np.where(rng.random(M) < 0.01, off + E - 1, ids[:, 0])
    note("sort skewed M=%d bm=%d" % (M, bm))
    d = abi.make_dims(M, 5120, 640, E, k, off)
    s, b, n = abi.moe_a8w4_sort(d, bm, dev(ids))
    torch.cuda.synchronize()
    rs, rb = oracle.sort(ids, E, off, bm)
    P = int(n.item())
    assert P == len(rs)
    assert np.array_equal(s[:P].cpu().numpy(), rs)
    assert np.array_equal(b[: P // bm].cpu().numpy(), rb)


def test_pack_layout():
    """Packed codes/scales equal the documented permutation of the inputs."""
    E, H, I = 2, 512, 256
    w = wl.Workload("pack", H, I, I, E, E, 2, False, 0, (), ("softmax",), 55)
    w13, w13_s, w2, w2_s = wl.make_weights(w)
    d = abi.make_dims(1, H, I, E, 2)
    p13, p13s, p2, p2s = [t.cpu().numpy() for t in abi.moe_a8w4_pack_weights(
        d, dev(w13), dev(w13_s), dev(w2), dev(w2_s))]

    def expect(codes, scales, N, K):
        KS, NG = K // 128, N // 64
        ec = np.zeros(codes.size, np.uint8)
        es = np.zeros(scales.size, np.uint8)
        for e in range(E):
            for g in range(NG):
                for s in range(KS):
                    for t in range(4):
                        for lane in range(64):
                            m, q = lane % 16, lane // 16
                            n = g * 64 + 16 * (m // 4) + 4 * t + (m % 4)
                            dst = ((((e * NG + g) * KS + s) * 4 + t) * 64 + lane) * 16
                            ec[dst:dst + 16] = codes[e, n, 64 * s + 16 * q: 64 * s + 16 * q + 16]
                            es[(((e * NG + g) * KS + s) * 64 + lane) * 4 + t] = scales[e, n, 4 * s + q]
        return ec, es

    ec, es = expect(w13, w13_s, 2 * I, H)
    assert np.array_equal(p13.ravel(), ec) and np.array_equal(p13s.ravel(), es)
    ec, es = expect(w2, w2_s, H, I)
    assert np.array_equal(p2.ravel(), ec) and np.array_equal(p2s.ravel(), es)


@pytest.mark.parametrize("name,M,E", [("draft-decode", 33, 8), ("local-slice", 40, 6),
                                      ("backbone-decode", 257, 16)])
def test_stage1_intermediate(name, M, E):
    """Stage one against the oracle's requantised intermediate, route by route.

    The GPU intermediate must be a faithful rounding of the oracle's exact
    value (see gpu_util.check_routes_intermediate), and rows holding a route must be
    fully written: the buffers start as 0xFF, which no code or scale takes.
    """
    w = wl.scaled(wl.WORKLOADS[name], num_experts=E, routed_experts=E, config_id=60 + E)
    L = Layer(w)
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    note("stage1 %s M=%d E=%d" % (name, M, E))
    d = L.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    q, s = abi.moe_a8w4_quant_act(dev(hidden))
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, dev(ids))
    cap = abi.moe_a8w4_sort_capacity(d, bm)
    iq = torch.full((cap, w.inter), 0xFF, dtype=torch.uint8, device=DEV)
    is_ = torch.full((cap, w.inter // 32), 0xFF, dtype=torch.uint8, device=DEV)
    abi.moe_a8w4_stage1(d, bm, q, s, srt, bexp, npad, L.packed[0], L.packed[1], iq, is_)
    torch.cuda.synchronize()
    P = int(npad.item())
    sorted_ids = srt[:P].cpu().numpy()
    real = np.nonzero(sorted_ids != M)[0]
    routes = (sorted_ids[real] & 0xFFFFFF).astype(np.int64) * w.topk + (sorted_ids[real] >> 24)
    giq = iq.cpu().numpy()[real]
    gis = is_.cpu().numpy()[real]
    assert not (gis == 0xFF).any(), "unwritten scales in routed rows"
    assert not (giq == 0xFF).any(), "unwritten codes in routed rows"
    check_routes_intermediate(L, hidden, ids, routes, giq, gis)
    if w.inter_valid < w.inter:
        assert np.all((giq[:, w.inter_valid:] & 0x7F) == 0)


# ------------------------------------------------------------ route rows

_E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def decode_route_rows(buf, M, topk, H):
    """The stage-two route rows of a uint8 buffer: (codes [M*topk, H] int16,
    exponents [M*topk, H/32], values [M*topk, H] float64 = code * 2^(S-140))."""
    nb = M * topk * H * 2
    codes = buf[:nb].view(np.int16).reshape(M * topk, H)
    exps = buf[nb:nb + M * topk * H // 32].reshape(M * topk, H // 32)
    vals = codes.astype(np.float64) * np.repeat(np.exp2(exps.astype(np.float64) - 140), 32, axis=1)
    return codes, exps, vals


def test_combine_route_rows_bit_exact():
    """Combine of host-written route rows: each output must be the BF16
    rounding (nearest, ties to even) of the float32 sum, in ascending k, of
    the exactly decoded values of the token's local slots; zero without one."""
    w = wl.scaled(wl.WORKLOADS["draft-decode"], num_experts=8, routed_experts=16, expert_offset=4,
                  config_id=71)
    M, k, H = 37, 6, 512
    rng = np.random.default_rng(71)
    ids = rng.integers(0, 16, size=(M, k)).astype(np.int32)
    ids[3] = 15                                     # a token with no local slot
    codes = rng.integers(-16384, 16385, size=(M * k, H)).astype(np.int16)
    exps = rng.integers(30, 161, size=(M * k, H // 32)).astype(np.uint8)
    codes[5, :64] = 16384
    codes[6, :64] = -16384
    buf = np.concatenate([codes.view(np.uint8).ravel(), exps.ravel()])
    d = abi.make_dims(M, H, w.inter, w.num_experts, k, w.expert_offset, w.routed_experts)
    note("combine route rows M=%d k=%d H=%d" % (M, k, H))
    out = abi.moe_a8w4_combine(d, dev(ids), dev(buf))
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    vals = (codes.astype(np.float64) * np.repeat(np.exp2(exps.astype(np.float64) - 140), 32, axis=1))
    vals = vals.astype(np.float32).reshape(M, k, H)   # exact: 15-bit integers times powers of two
    local = (ids - w.expert_offset >= 0) & (ids - w.expert_offset < w.num_experts)
    acc = np.zeros((M, H), np.float32)
    for kk in range(k):
        acc = np.where(local[:, kk:kk + 1], (acc + vals[:, kk]).astype(np.float32), acc)
    want = np.array([oracle.bf16_rne(float(x)) for x in acc.ravel()], np.uint16).reshape(M, H)
    assert np.array_equal(got, want)
    assert not got[3].any()


@pytest.mark.parametrize("name,M,E", [("draft-decode", 33, 8), ("local-slice", 8, 6),
                                      ("local-slice", 12, 6), ("local-slice", 40, 6),
                                      ("local-slice", 80, 6)])
def test_stage2_route_rows(name, M, E):
    """Stage two given the GPU's own intermediate, route by route: decoded rows
    within the accumulation budget (the scaled MFMA's run truncation, see
    test_gpu_mfma.py, plus FP32 accumulation) plus half an encoding step of
    topk_weight * (w2[e] h) in FP64; exponents as the format defines them
    (max |code| of a block in [2^13, 2^14] unless the block is tiny); rows of
    non-local slots untouched."""
    w = wl.scaled(wl.WORKLOADS[name], num_experts=E, routed_experts=E + 2, config_id=80 + M)
    L = Layer(w)
    hidden, ids, wts = wl.make_inputs(w, M, "softmax")
    d = L.dims(M)
    bm = abi.moe_a8w4_block_m(d)
    note("stage2 route rows %s M=%d E=%d bm=%d" % (name, M, E, bm))
    xd, idd, wd = dev(hidden), dev(ids), dev(wts)
    q, s = abi.moe_a8w4_quant_act(xd)
    srt, bexp, npad = abi.moe_a8w4_sort(d, bm, idd)
    iq, is_ = abi.moe_a8w4_stage1(d, bm, q, s, srt, bexp, npad, L.packed[0], L.packed[1])
    y = torch.full((abi.route_rows_bytes(d),), 0x5A, dtype=torch.uint8, device=DEV)
    abi.moe_a8w4_stage2(d, bm, iq, is_, srt, bexp, npad, wd, L.packed[2], L.packed[3], y)
    torch.cuda.synchronize()
    H, I, k = w.hidden, w.inter, w.topk
    codes, exps, got = decode_route_rows(y.cpu().numpy(), M, k, H)
    P = int(npad.item())
    sorted_ids = srt[:P].cpu().numpy()
    giq, gis = iq[:P].cpu().numpy(), is_[:P].cpu().numpy()
    real = np.nonzero(sorted_ids != M)[0]
    slots = (sorted_ids[real] & 0xFFFFFF).astype(np.int64) * k + (sorted_ids[real] >> 24)
    le = ids.ravel()[slots].astype(np.int64) - w.expert_offset
    h = _E4M3[giq[real]] * np.repeat(np.exp2(gis[real].astype(np.float64) - 127), 32, axis=1)
    h2, h2s = L.host[2], L.host[3]
    for e in np.unique(le):
        rs = np.nonzero(le == e)[0]
        c = np.empty((H, I), np.uint8)
        c[:, 0::2] = h2[e] & 15
        c[:, 1::2] = h2[e] >> 4
        W = _E2M1[c] * np.repeat(np.exp2(h2s[e].astype(np.float64) - 127), 32, axis=1)
        wt = wts.ravel()[slots[rs]].astype(np.float64)[:, None]
        exact = wt * (h[rs] @ W.T)
        # the scaled MFMA's run truncation (at most 7 * 2^-13 of a run's largest
        # product, so of sum |h w|) plus FP32 accumulation over the K steps
        acc_err = (MFMA_RUN_ERR + (I // 128) * 2.0 ** -20) * np.abs(wt) * (np.abs(h[rs]) @ np.abs(W).T)
        half_step = np.repeat(np.exp2(exps[slots[rs]].astype(np.float64) - 141), 32, axis=1)
        err = np.abs(got[slots[rs]] - exact)
        assert np.all(err <= acc_err + half_step), "expert %d: route values off by up to %.3g" % (
            e, (err - acc_err - half_step).max())
    blk = np.abs(codes[slots].astype(np.int64)).reshape(len(slots), -1, 32).max(axis=2)
    ex = exps[slots].astype(np.int64)
    assert np.all(blk <= 16384) and np.all(ex >= 14) and np.all(ex <= 254)
    assert np.all(blk[ex > 14] >= 8192), "a block exponent larger than its values need"
    untouched = np.ones(M * k, bool)
    untouched[slots] = False
    raw = y.cpu().numpy()
    assert np.all(raw[:M * k * H * 2].reshape(M * k, -1)[untouched] == 0x5A)
    assert np.all(raw[M * k * H * 2:].reshape(M * k, -1)[untouched] == 0x5A)
