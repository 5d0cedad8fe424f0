"""GPU parity of the router (softmax top-k, renormalised, optional shared slot)
against the oracle's, alone and inside the layer: ids bit-exact, weights
within float32 rounding, and the layer routed from its logits at the gate."""
import numpy as np
import pytest
import torch

import oracle
from mixture_experts_fp8_amd import abi, workloads as wl
from gpu_util import DEV, Layer, check_forward, dev, host_bf16_bits, note

pytestmark = pytest.mark.gpu

# float32 exp, sum of at most 8 terms and one division: a few ulp of 1
WEIGHT_ATOL = 2e-6


def check_route(logits, k_routed, shared, ids, wts):
    rid, rwt = oracle.softmax_topk(logits, k_routed, shared)
    assert np.array_equal(ids, rid)
    assert np.abs(wts.astype(np.float64) - rwt).max() <= WEIGHT_ATOL


@pytest.mark.parametrize("M,Er,kr,shared", [(64, 384, 6, -1), (33, 128, 3, -1), (40, 384, 6, 384),
                                           (17, 100, 8, -1), (5, 8, 1, 7), (3000, 384, 6, -1),
                                           (9, 512, 7, 512),
                                           (16384, 384, 6, 384)])   # the prefill geometry's full call
def test_route_matches_oracle(M, Er, kr, shared):
    rng = np.random.default_rng(M * 7 + Er)
    logits = rng.standard_normal((M, Er), dtype=np.float32)
    note("route M=%d E=%d k=%d shared=%d" % (M, Er, kr, shared))
    ids, wts = abi.moe_a8w4_route(dev(logits), kr, shared)
    torch.cuda.synchronize()
    check_route(logits, kr, shared, ids.cpu().numpy(), wts.cpu().numpy())


def test_route_ties_take_the_lower_id():
    rng = np.random.default_rng(11)
    logits = rng.integers(0, 3, size=(50, 96)).astype(np.float32)   # many equal values
    logits[0] = 1.0                                                  # all equal
    note("route ties")
    ids, wts = abi.moe_a8w4_route(dev(logits), 6)
    torch.cuda.synchronize()
    ids, wts = ids.cpu().numpy(), wts.cpu().numpy()
    check_route(logits, 6, -1, ids, wts)
    assert ids[0].tolist() == [0, 1, 2, 3, 4, 5]


@pytest.mark.parametrize("name,E,routed,topk,shared,M", [
    ("backbone-decode", 16, 16, 6, -1, 13),     # routing inside the sort launch
    ("backbone-decode", 16, 16, 6, -1, 33),     # routing in a launch of its own
    ("backbone-decode", 16, 16, 6, -1, 300),    # the same, several sort workgroups
    ("prefill-shared", 9, 8, 3, 8, 12),         # two routed slots and the shared expert, in the sort
    ("prefill-shared", 9, 8, 3, 8, 48),         # the same, routed first
])
def test_forward_routed(name, E, routed, topk, shared, M):
    w = wl.scaled(wl.WORKLOADS[name], num_experts=E, routed_experts=routed, topk=topk,
                  config_id=300 + E + M)
    layer = Layer(w)
    rng = np.random.default_rng(M)
    hidden = wl.make_hidden(rng, M, w.hidden)
    logits = rng.standard_normal((M, routed), dtype=np.float32)
    d = layer.dims(M)
    note("forward routed %s M=%d E=%d routed=%d topk=%d shared=%d" % (name, M, E, routed, topk, shared))
    xd = dev(hidden)
    out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    out, ids, wts = abi.moe_a8w4_forward_routed(d, xd, dev(logits), shared, *layer.packed, out=out)
    torch.cuda.synchronize()
    ids_h, wts_h = ids.cpu().numpy(), wts.cpu().numpy()
    check_route(logits, topk - (1 if shared >= 0 else 0), shared, ids_h, wts_h)
    # the layer on that routing, against the oracle
    check_forward(layer, hidden, ids_h, wts_h, host_bf16_bits(out), xd, ids)
