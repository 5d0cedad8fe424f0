"""moe_a8w4_forward_noalloc, the entry point for callers that cannot allocate
device memory, against moe_a8w4_forward through the C ABI: the same kernels
on the same inputs, so the outputs must be equal bit for bit, on two calls in
a row (the largest backbone decode bucket, then a smaller one: the static
scratch keeps the first call's contents), and a call whose workspace would
exceed the static scratch is rejected before anything is enqueued."""
import numpy as np
import pytest
import torch

from mixture_experts_fp8_amd import abi, workloads as wl
from gpu_util import DEV, Layer, dev, note

pytestmark = pytest.mark.gpu


def test_noalloc_equals_forward_on_two_calls_second_smaller():
    w = wl.WORKLOADS["backbone-decode"]
    layer = Layer(w)
    for M in (768, 48):
        d = layer.dims(M)
        assert abi.moe_a8w4_workspace_bytes(d) <= abi.NOALLOC_SCRATCH_BYTES
        hidden, ids, wts = wl.make_inputs(w, M, "softmax")
        xd, idd, wd = dev(hidden), dev(ids), dev(wts)
        note("noalloc vs forward M=%d bm=%d" % (M, abi.moe_a8w4_block_m(d)))
        ref = layer.forward(xd, idd, wd)
        out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
        abi.moe_a8w4_forward_noalloc(d, xd, idd, wd, *layer.packed, out=out)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16)), M
        # inputs untouched
        assert np.array_equal(idd.cpu().numpy(), ids)


def test_noalloc_rejects_calls_beyond_the_scratch():
    w = wl.WORKLOADS["prefill-shared"]
    M = 4096
    d = abi.make_dims(M, w.hidden, w.inter, w.num_experts, w.topk, w.expert_offset, w.routed_experts)
    assert abi.moe_a8w4_workspace_bytes(d) > abi.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, w.hidden), dtype=torch.bfloat16, device=DEV)
    ids = torch.zeros((M, w.topk), dtype=torch.int32, device=DEV)
    wts = torch.zeros((M, w.topk), dtype=torch.float32, device=DEV)
    wgt = torch.zeros(256, dtype=torch.uint8, device=DEV)
    out = torch.full((M, w.hidden), float("nan"), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(abi.MoeError) as err:
        abi.moe_a8w4_forward_noalloc(d, x, ids, wts, wgt, wgt, wgt, wgt, out=out)
    assert err.value.status == abi.MOE_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.isnan(out).all()     # nothing was enqueued
