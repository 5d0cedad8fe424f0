"""Pins of the oracle's whole layer: dense-MLP equivalence, exact brute force
on tiny shapes, and invariants the method fixes.

Shapes are small so that the CPU suite stays within minutes.
"""
import numpy as np
import pytest

from mixture_experts_fp8_amd import workloads as wl
import independent as ind


def small(H=256, I=64, Iv=None, E=8, routed=None, topk=3, shared=False, offset=0, cid=90):
    return wl.Workload("small", H, I, I if Iv is None else Iv, E, E if routed is None else routed,
                       topk, shared, offset, (), ("softmax",), cid)


def silu_mlp_dense(hidden_bits, w13e, w13se, w2e, w2se, want_gu=False):
    """Dense SiLU-gated MLP on dequantised operands (numpy FP64 matmuls), with
    the per-1x32 quantisation of the activations and of the intermediate done
    by the brute-force quantiser."""
    x = ind.bf16_to_f64(hidden_bits)
    aq, as_ = ind.quantize_rows_bruteforce(x)
    A = ind.dequant_fp8(aq, as_)
    W13 = ind.dequant_mxfp4(w13e, w13se)
    Wg, Wu = W13[0::2], W13[1::2]
    g = A @ Wg.T
    u = A @ Wu.T
    h = g / (1.0 + np.exp(-g)) * u
    iq, is_ = ind.quantize_rows_bruteforce(h)
    Hq = ind.dequant_fp8(iq, is_)
    W2 = ind.dequant_mxfp4(w2e, w2se)
    if want_gu:
        return Hq @ W2.T, iq, is_, g, u
    return Hq @ W2.T, iq, is_


@pytest.mark.parametrize("H,I,Iv,M", [(256, 64, 64, 7), (512, 128, 96, 5), (5120, 640, 576, 2)])
def test_single_expert_top1_equals_dense_mlp(oracle, H, I, Iv, M):
    w = small(H=H, I=I, Iv=Iv, E=1, topk=1, cid=91)
    w13, w13_s, w2, w2_s = wl.make_weights(w)
    rng = np.random.default_rng(7)
    hidden = wl.make_hidden(rng, M, H)
    ids = np.zeros((M, 1), np.int32)
    wts = np.ones((M, 1), np.float32)
    out, o64 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, want_f64=True)
    y, iq_ref, is_ref, g, u = silu_mlp_dense(hidden, w13[0], w13_s[0], w2[0], w2_s[0], want_gu=True)
    iq, is_, h, gu, gu_abs = oracle.intermediate(hidden, ids, w13, w13_s, np.arange(M), want_f64=True,
                                                 want_gu=True)
    assert np.array_equal(iq, iq_ref)
    assert np.array_equal(is_, is_ref)
    # the FP64 gate and up sums (gate j at 2j, up j at 2j + 1) and SiLU(gate) * up
    np.testing.assert_allclose(gu[:, 0::2], g, rtol=1e-12, atol=1e-12 * np.abs(g).max())
    np.testing.assert_allclose(gu[:, 1::2], u, rtol=1e-12, atol=1e-12 * np.abs(u).max())
    hd = g / (1.0 + np.exp(-g)) * u
    np.testing.assert_allclose(h, hd, rtol=1e-12, atol=1e-12 * np.abs(hd).max())
    # the sums of |a_k w_k| of the same dot products
    x = ind.bf16_to_f64(hidden)
    A = np.abs(ind.dequant_fp8(*ind.quantize_rows_bruteforce(x)))
    W13 = np.abs(ind.dequant_mxfp4(w13[0], w13_s[0]))
    np.testing.assert_allclose(gu_abs[:, 0::2], A @ W13[0::2].T, rtol=1e-12)
    np.testing.assert_allclose(gu_abs[:, 1::2], A @ W13[1::2].T, rtol=1e-12)
    # stage two's absolute sum, weighted by |w| over the slots
    _, o2, oab = oracle.forward_given_intermediate(ids, wts * -2, w2, w2_s, iq[:, None], is_[:, None],
                                                   want_f64=True, want_abs=True)
    Hq = np.abs(ind.dequant_fp8(iq, is_))
    np.testing.assert_allclose(oab, 2 * Hq @ np.abs(ind.dequant_mxfp4(w2[0], w2_s[0])).T, rtol=1e-12)
    np.testing.assert_allclose(o2, -2 * o64, rtol=1e-12, atol=1e-12 * np.abs(o64).max())
    np.testing.assert_allclose(o64, y, rtol=1e-12, atol=1e-12 * np.abs(y).max())
    # padded intermediate columns quantise to exact zeros
    assert np.all(iq[:, Iv:] == 0)
    # BF16 rounding of the FP64 result
    ref_bits = ind.bf16_round_bruteforce(y[: min(M, 2)].ravel()[:2000])
    assert np.array_equal(out[: min(M, 2)].ravel()[:2000], ref_bits)


@pytest.mark.parametrize("case", [
    dict(H=64, I=64, E=4, topk=2, M=9, mode="softmax"),
    dict(H=128, I=64, E=8, topk=3, M=5, mode="softmax"),
    dict(H=64, I=128, E=3, topk=3, M=4, mode="roundrobin"),
    dict(H=64, I=64, E=6, topk=3, M=33, mode="softmax"),
])
def test_oracle_equals_exact_bruteforce(oracle, case):
    w = small(H=case["H"], I=case["I"], E=case["E"], topk=case["topk"], cid=92)
    w13, w13_s, w2, w2_s = wl.make_weights(w)
    hidden, ids, wts = wl.make_inputs(w, case["M"], case["mode"], seed=[92, case["M"]])
    # make a few slots non-local to exercise the skip rule
    ids = ids.copy()
    ids[0, 0] = -1
    if case["M"] > 2:
        ids[2, -1] = case["E"] + 5
    out, o64 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, want_f64=True)
    ref, inter = ind.bruteforce_forward(hidden, ids, wts, w13, w13_s, w2, w2_s)
    np.testing.assert_allclose(o64, ref, rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    routes = np.array(sorted(inter.keys()), np.int64)
    iq, is_ = oracle.intermediate(hidden, ids, w13, w13_s, routes)
    for i, f in enumerate(routes):
        assert np.array_equal(iq[i], inter[int(f)][0])
        assert np.array_equal(is_[i], inter[int(f)][1])
    ref_bits = ind.bf16_round_bruteforce(ref.ravel())
    assert np.array_equal(out.ravel(), ref_bits)
    # the listed-token form gives the same rows
    sub = np.array([case["M"] - 1, 0, 1], np.int64)
    assert np.array_equal(oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, tokens=sub), out[sub])


@pytest.fixture(scope="module")
def inv_case():
    w = small(H=256, I=64, E=8, topk=3, cid=93)
    weights = wl.make_weights(w)
    hidden, ids, wts = wl.make_inputs(w, 6, "softmax", seed=[93])
    return w, weights, hidden, ids, wts


def test_weight_scaling_is_exact(oracle, inv_case):
    w, (w13, w13_s, w2, w2_s), hidden, ids, wts = inv_case
    _, o1 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, want_f64=True)
    _, o2 = oracle.forward(hidden, ids, wts * 2, w13, w13_s, w2, w2_s, want_f64=True)
    assert np.array_equal(o2, 2 * o1)


def test_slot_permutation(oracle, inv_case):
    w, (w13, w13_s, w2, w2_s), hidden, ids, wts = inv_case
    _, o1 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, want_f64=True)
    perm = [2, 0, 1]
    _, o2 = oracle.forward(hidden, ids[:, perm], wts[:, perm], w13, w13_s, w2, w2_s, want_f64=True)
    np.testing.assert_allclose(o2, o1, rtol=1e-13, atol=1e-13)


def test_expert_relabelling(oracle, inv_case):
    w, (w13, w13_s, w2, w2_s), hidden, ids, wts = inv_case
    out1 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s)
    perm = np.random.default_rng(1).permutation(w.num_experts)   # new id of old expert e
    inv = np.argsort(perm)
    out2 = oracle.forward(hidden, perm[ids].astype(np.int32), wts,
                          w13[inv], w13_s[inv], w2[inv], w2_s[inv])
    assert np.array_equal(out1, out2)


def test_nonlocal_ids_and_offset(oracle, inv_case):
    w, (w13, w13_s, w2, w2_s), hidden, ids, wts = inv_case
    out1 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s)
    # the same experts addressed as a slice at offset 192
    out2 = oracle.forward(hidden, ids + 192, wts, w13, w13_s, w2, w2_s, expert_offset=192)
    assert np.array_equal(out1, out2)
    # an extra slot that names a non-local expert changes nothing
    ids3 = np.concatenate([ids, np.full((ids.shape[0], 1), 1000, np.int32)], axis=1)
    wts3 = np.concatenate([wts, np.full((wts.shape[0], 1), 0.5, np.float32)], axis=1)
    assert np.array_equal(oracle.forward(hidden, ids3, wts3, w13, w13_s, w2, w2_s), out1)
    # a token with no local route gets a +0 row
    ids4 = ids.copy()
    ids4[1, :] = -3
    out4 = oracle.forward(hidden, ids4, wts, w13, w13_s, w2, w2_s)
    assert np.all(out4[1] == 0)
    assert np.array_equal(np.delete(out4, 1, 0), np.delete(out1, 1, 0))


def test_zero_padding_of_intermediate_is_exact(oracle):
    """I = 576 unpadded equals I = 640 with zero-coded padding."""
    w = small(H=512, I=640, Iv=576, E=3, topk=2, cid=94)
    w13, w13_s, w2, w2_s = wl.make_weights(w)
    hidden, ids, wts = wl.make_inputs(w, 3, "softmax", seed=[94])
    o_pad = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s)
    w13u = np.ascontiguousarray(w13[:, :2 * 576])
    w13su = np.ascontiguousarray(w13_s[:, :2 * 576])
    w2u = np.ascontiguousarray(w2[:, :, :288])
    w2su = np.ascontiguousarray(w2_s[:, :, :18])
    o_unp = oracle.forward(hidden, ids, wts, w13u, w13su, w2u, w2su)
    assert np.array_equal(o_pad, o_unp)


def test_shared_expert_decomposes(oracle):
    """top-6 routed + shared slot (weight 1) = routed result + the dense shared MLP."""
    w = small(H=256, I=64, E=9, routed=8, topk=4, shared=True, cid=95)
    w13, w13_s, w2, w2_s = wl.make_weights(w)
    hidden, ids, wts = wl.make_inputs(w, 5, "softmax", seed=[95])
    assert np.all(ids[:, -1] == 8) and np.all(wts[:, -1] == 1.0)
    _, o_all = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, want_f64=True)
    _, o_routed = oracle.forward(hidden, ids[:, :-1], wts[:, :-1], w13, w13_s, w2, w2_s, want_f64=True)
    y_shared, _, _ = silu_mlp_dense(hidden, w13[8], w13_s[8], w2[8], w2_s[8])
    np.testing.assert_allclose(o_all, o_routed + y_shared, rtol=1e-12, atol=1e-12)


def test_given_intermediate_reproduces_forward(oracle, inv_case):
    """Stage two + combine on the oracle's own intermediate is the forward."""
    w, (w13, w13_s, w2, w2_s), hidden, ids, wts = inv_case
    out, o64 = oracle.forward(hidden, ids, wts, w13, w13_s, w2, w2_s, want_f64=True)
    M, k = ids.shape
    routes = np.arange(M * k, dtype=np.int64)
    iq, is_ = oracle.intermediate(hidden, ids, w13, w13_s, routes)
    out2, o2 = oracle.forward_given_intermediate(ids, wts, w2, w2_s, iq.reshape(M, k, -1),
                                                 is_.reshape(M, k, -1), want_f64=True)
    assert np.array_equal(out, out2) and np.array_equal(o64, o2)
    # a changed intermediate element moves the output by exactly w * w2[:, j] * delta
    iq2 = iq.copy()
    iq2[0, 5] = (iq2[0, 5] + 1) % 0x7E
    _, o3 = oracle.forward_given_intermediate(ids, wts, w2, w2_s, iq2.reshape(M, k, -1),
                                              is_.reshape(M, k, -1), want_f64=True)
    W2 = ind.dequant_mxfp4(w2[ids[0, 0]], w2_s[ids[0, 0]])
    scale = ind.E8M0_ALL[is_[0, 0]]
    delta = (ind.E4M3_ALL[iq2[0, 5]] - ind.E4M3_ALL[iq[0, 5]]) * scale
    np.testing.assert_allclose(o3[0] - o64[0], float(wts[0, 0]) * W2[:, 5] * delta, rtol=1e-9, atol=1e-12)
