"""The seeded generators reproduce the statistics of the pages' workloads."""
import os

import numpy as np

from mixture_experts_fp8_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_local_slice_route_counts_match_printed_table():
    """96 local experts of 384 with top-6: local routes ~ 1.5 per token, as in the
    local-routes column of the expert-parallel benchmark table (golden file)."""
    w = wl.WORKLOADS["local-slice"]
    rows = [l.split() for l in open(os.path.join(GOLDEN, "local_routes_pr5904.txt"))
            if l.strip() and not l.startswith("#")]
    for tok, routes in rows:
        tok, routes = int(tok), int(routes)
        if tok < 256:
            continue  # small counts are dominated by sampling noise
        _, ids, _ = wl.make_inputs(wl.scaled(w, hidden=64), tok, "softmax")
        ours = wl.local_routes(w, ids)
        assert 0.85 < ours / routes < 1.15, (tok, ours, routes)


def test_routing_shapes_and_weights():
    for name, w in wl.WORKLOADS.items():
        for mode in w.routings:
            M = 37
            hidden, ids, wts = wl.make_inputs(wl.scaled(w, hidden=64), M, mode)
            assert hidden.shape == (M, 64) and hidden.dtype == np.uint16
            assert ids.shape == (M, w.topk) and wts.shape == (M, w.topk)
            kr = w.topk - (1 if w.shared else 0)
            assert np.allclose(wts[:, :kr].sum(axis=1), 1.0, atol=1e-6)
            assert np.all(ids[:, :kr] >= 0) and np.all(ids[:, :kr] < w.routed_experts)
            for row in ids[:, :kr]:
                assert len(set(row.tolist())) == kr
            if w.shared:
                assert np.all(ids[:, -1] == w.routed_experts) and np.all(wts[:, -1] == 1.0)


def test_concentrated_routing_is_concentrated():
    w = wl.WORKLOADS["draft-sweep"]
    _, ids, _ = wl.make_inputs(wl.scaled(w, hidden=64), 640, "concentrated")
    frac_hot = (ids < 4).mean()
    assert 0.6 < frac_hot < 0.9


def test_weight_generation_distribution():
    w = wl.scaled(wl.WORKLOADS["draft-decode"], num_experts=2, routed_experts=2, hidden=512)
    w13, w13_s, w2, w2_s = wl.make_weights(w)
    assert w13.shape == (2, 1280, 256) and w13_s.shape == (2, 1280, 16)
    assert w2.shape == (2, 512, 320) and w2_s.shape == (2, 512, 20)
    assert set(np.unique(w13_s).tolist()) == set(wl.WEIGHT_SCALE_CODES)
    assert np.all(w13[:, 1152:] == 0) and np.all(w2[:, :, 288:] == 0)
    lo = w13[:, :1152] & 15
    counts = np.bincount(lo.ravel(), minlength=16)
    assert counts.min() > 0.9 * counts.mean()
    assert np.array_equal(wl.make_weights(w)[0], w13)   # seeded
