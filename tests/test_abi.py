"""The C ABI library loads, exports every symbol its header declares, and
rejects invalid arguments on the host before any GPU work (no GPU needed)."""
import ctypes
import os
import re

import pytest

from mixture_experts_fp8_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_a8w4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_a(?:8|16)w4_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = abi.load()
    names = declared_functions()
    assert len(names) >= 11
    assert set(names) == set(abi.EXPORTS)
    for n in names:
        assert getattr(lib, n) is not None


def dims(**kw):
    d = dict(tokens=5, hidden=5120, inter=640, num_experts=128, topk=3, expert_offset=0)
    d.update(kw)
    return abi.make_dims(d["tokens"], d["hidden"], d["inter"], d["num_experts"], d["topk"],
                         d["expert_offset"])


@pytest.mark.parametrize("bad", [
    dict(tokens=-1), dict(tokens=1 << 24), dict(hidden=0), dict(hidden=5000), dict(hidden=256),
    dict(inter=0), dict(inter=576), dict(inter=64), dict(num_experts=0), dict(num_experts=513),
    dict(topk=0), dict(topk=9),
])
def test_invalid_dims_rejected(bad):
    lib = abi.load()
    d = dims(**bad)
    n = ctypes.c_size_t(0)
    assert lib.moe_a8w4_workspace_bytes(ctypes.byref(d), ctypes.byref(n)) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_block_m(ctypes.byref(d)) == abi.MOE_ERR_DIMS
    one = ctypes.c_void_p(256)
    st = lib.moe_a8w4_forward(ctypes.byref(d), *([one] * 9), 1 << 40, None)
    assert st == abi.MOE_ERR_DIMS


def test_null_dims_and_pointers():
    lib = abi.load()
    assert lib.moe_a8w4_block_m(None) == abi.MOE_ERR_NULL
    d = dims()
    one = ctypes.c_void_p(256)
    for i in range(9):
        ptrs = [one] * 9
        ptrs[i] = None
        assert lib.moe_a8w4_forward(ctypes.byref(d), *ptrs, 1 << 40, None) == abi.MOE_ERR_NULL


def test_misaligned_and_small_workspace():
    lib = abi.load()
    d = dims()
    ok = ctypes.c_void_p(4096)
    bad = ctypes.c_void_p(4096 + 8)
    need = abi.moe_a8w4_workspace_bytes(d)
    assert lib.moe_a8w4_forward(ctypes.byref(d), bad, *([ok] * 8), need, None) == abi.MOE_ERR_ALIGN
    ws_bad = ctypes.c_void_p(4096 + 16)   # 16-byte but not 256-byte aligned
    assert lib.moe_a8w4_forward(ctypes.byref(d), *([ok] * 8), ws_bad, need, None) == abi.MOE_ERR_ALIGN
    assert lib.moe_a8w4_forward(ctypes.byref(d), *([ok] * 9), need - 1, None) == abi.MOE_ERR_WORKSPACE


def test_zero_tokens_is_a_noop():
    lib = abi.load()
    d = dims(tokens=0)
    assert lib.moe_a8w4_forward(ctypes.byref(d), *([None] * 9), 0, None) == abi.MOE_OK


def test_block_m_capacity_and_workspace_sizes():
    assert abi.moe_a8w4_block_m(dims(tokens=5)) == 16
    assert abi.moe_a8w4_block_m(dims(tokens=768, num_experts=384, topk=6)) == 32
    assert abi.moe_a8w4_block_m(dims(tokens=16384, num_experts=96, topk=6, inter=2304)) == 128
    # a 96-expert slice of a 384-expert router: 1024 tokens give 16 routes per expert
    d = dims(tokens=1024, num_experts=96, topk=6, inter=2304)
    assert abi.moe_a8w4_block_m(d) == 128         # as if all 6 slots were local (64 per expert)
    assert abi.moe_a8w4_block_m(dims(tokens=640, num_experts=96, topk=6)) == 64    # 40 per expert
    assert abi.moe_a8w4_block_m(dims(tokens=656, num_experts=96, topk=6)) == 128   # 41
    d.routed_experts = 384
    assert abi.moe_a8w4_block_m(d) == 32
    assert abi.moe_a8w4_block_m(dims(tokens=320, num_experts=96, topk=6)) == 32    # 20 per expert
    assert abi.moe_a8w4_block_m(dims(tokens=336, num_experts=96, topk=6)) == 64    # 21
    d.routed_experts = -1
    assert abi.load().moe_a8w4_block_m(ctypes.byref(d)) == abi.MOE_ERR_DIMS
    # 385 experts of which the router chooses among 384: one shared expert in
    # one of the 7 slots, so the routed experts get M * 6 / 384 routes each
    d = dims(tokens=2560, num_experts=385, topk=7)
    d.routed_experts = 384
    assert abi.moe_a8w4_block_m(d) == 64          # 40 per routed expert (46.5 counting the shared slot)
    d = dims(tokens=4096, num_experts=385, topk=7, inter=768)
    d.routed_experts = 384
    assert abi.moe_a16w4_block_m(d) == 64         # 64 per routed expert (74.5 counting the shared slot)
    assert abi.moe_a8w4_block_m(d) == 128
    d = dims(tokens=33, num_experts=384, topk=6)
    R = 33 * 6
    for bm in (16, 32, 64, 128):
        cap = abi.moe_a8w4_sort_capacity(d, bm)
        assert cap % bm == 0 and cap >= R + min(384, R) * (bm - 1)
    with pytest.raises(abi.MoeError):
        abi.moe_a8w4_sort_capacity(d, 48)
    ws = abi.moe_a8w4_workspace_bytes(dims(tokens=16384, num_experts=385, topk=7))
    assert ws < 2 << 30     # dominated by the [M, topk, H] 16-bit route rows
    assert "block_m" in abi.status_str(abi.MOE_ERR_BLOCK_M)


def test_step_entry_points_validate():
    lib = abi.load()
    d = dims()
    p = ctypes.c_void_p(4096)
    assert lib.moe_a8w4_sort(ctypes.byref(d), 48, p, p, p, p, None) == abi.MOE_ERR_BLOCK_M
    assert lib.moe_a8w4_quant_sort(ctypes.byref(d), 16, p, p, p, p, p, p, None, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_stage1(ctypes.byref(d), 16, *([p] * 8), None, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_stage2(ctypes.byref(d), 16, *([p] * 8), None, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_quant_act(4, 48, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_combine(ctypes.byref(d), p, p, None, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_combine(ctypes.byref(d), p, ctypes.c_void_p(4100), p, None) == abi.MOE_ERR_ALIGN
    assert lib.moe_a8w4_pack_weights(ctypes.byref(d), *([p] * 7), None, None) == abi.MOE_ERR_NULL


def test_router_entry_points_validate():
    """Bad router dims, null or misaligned pointers: a status, nothing launched."""
    lib = abi.load()
    p, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4100)
    assert lib.moe_a8w4_route(4, 384, 0, -1, p, p, p, None) == abi.MOE_ERR_DIMS      # no routed slot
    assert lib.moe_a8w4_route(4, 5, 6, -1, p, p, p, None) == abi.MOE_ERR_DIMS        # k > experts
    assert lib.moe_a8w4_route(4, 384, 8, 384, p, p, p, None) == abi.MOE_ERR_DIMS     # 9 slots
    assert lib.moe_a8w4_route(4, 513, 6, -1, p, p, p, None) == abi.MOE_ERR_DIMS      # > 512 logits
    assert lib.moe_a8w4_route(-1, 384, 6, -1, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_route(0, 384, 6, -1, None, None, None, None) == abi.MOE_OK
    assert lib.moe_a8w4_route(4, 384, 6, -1, None, p, p, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_route(4, 384, 6, -1, odd, p, p, None) == abi.MOE_ERR_ALIGN
    d = dims(tokens=4, num_experts=16, topk=6)
    d.routed_experts = 16
    assert lib.moe_a8w4_forward_routed(ctypes.byref(d), p, None, -1, *([p] * 8), 1 << 30, None) \
        == abi.MOE_ERR_NULL
    d.routed_experts = 0                                                              # no logits width
    assert lib.moe_a8w4_forward_routed(ctypes.byref(d), p, p, -1, *([p] * 8), 1 << 30, None) \
        == abi.MOE_ERR_DIMS
    d.routed_experts = 16
    d.topk = 1                                                                        # shared slot only
    assert lib.moe_a8w4_forward_routed(ctypes.byref(d), p, p, 15, *([p] * 8), 1 << 30, None) \
        == abi.MOE_ERR_DIMS


def test_a16w4_entry_points_validate():
    """The A16W4 variant: bad dims, null or misaligned pointers, a small
    workspace, bad block_m; M = 0 succeeds without touching anything."""
    lib = abi.load()
    p, odd = ctypes.c_void_p(4096), ctypes.c_void_p(4096 + 8)
    d = dims(tokens=12, num_experts=384, topk=6, inter=768)
    need = abi.moe_a16w4_workspace_bytes(d)
    assert need > 0 and abi.moe_a16w4_block_m(d) == 16
    assert abi.moe_a16w4_block_m(dims(tokens=1536, num_experts=384, topk=6, inter=768)) == 32   # 24
    assert abi.moe_a16w4_block_m(dims(tokens=4096, num_experts=384, topk=6, inter=768)) == 64   # 64
    assert abi.moe_a16w4_block_m(dims(tokens=16384, num_experts=384, topk=6, inter=768)) == 128
    bad = dims(inter=576)
    n = ctypes.c_size_t(0)
    assert lib.moe_a16w4_workspace_bytes(ctypes.byref(bad), ctypes.byref(n)) == abi.MOE_ERR_DIMS
    assert lib.moe_a16w4_forward(ctypes.byref(bad), *([p] * 9), need, None) == abi.MOE_ERR_DIMS
    for i in range(9):
        ptrs = [p] * 9
        ptrs[i] = None
        assert lib.moe_a16w4_forward(ctypes.byref(d), *ptrs, need, None) == abi.MOE_ERR_NULL
    assert lib.moe_a16w4_forward(ctypes.byref(d), odd, *([p] * 8), need, None) == abi.MOE_ERR_ALIGN
    assert lib.moe_a16w4_forward(ctypes.byref(d), *([p] * 8), ctypes.c_void_p(4096 + 16), need, None) \
        == abi.MOE_ERR_ALIGN
    assert lib.moe_a16w4_forward(ctypes.byref(d), *([p] * 9), need - 1, None) == abi.MOE_ERR_WORKSPACE
    z = dims(tokens=0, inter=768)
    assert lib.moe_a16w4_forward(ctypes.byref(z), *([None] * 9), 0, None) == abi.MOE_OK
    assert lib.moe_a16w4_stage1(ctypes.byref(d), 48, *([p] * 7), None) == abi.MOE_ERR_BLOCK_M
    assert lib.moe_a16w4_stage1(ctypes.byref(d), 16, *([p] * 6), None, None) == abi.MOE_ERR_NULL


def test_fused_launch_entry_points_validate():
    """moe_a8w4_stages_fused: block_m 16 or 32 only, every pointer required,
    the counter count grows with the tokens."""
    lib = abi.load()
    p = ctypes.c_void_p(4096)
    d = dims(tokens=6, num_experts=384, topk=6)
    n6 = abi.moe_a8w4_fused_counters(d, 16)
    assert n6 > 0 and abi.moe_a8w4_fused_counters(dims(tokens=12, num_experts=384, topk=6), 16) > n6
    assert lib.moe_a8w4_fused_counters(ctypes.byref(d), 64) == abi.MOE_ERR_BLOCK_M
    assert lib.moe_a8w4_stages_fused(ctypes.byref(d), 64, *([p] * 16), None) == abi.MOE_ERR_BLOCK_M
    for i in range(16):
        ptrs = [p] * 16
        ptrs[i] = None
        assert lib.moe_a8w4_stages_fused(ctypes.byref(d), 16, *ptrs, None) == abi.MOE_ERR_NULL
    z = dims(tokens=0)
    assert lib.moe_a8w4_stages_fused(ctypes.byref(z), 16, *([None] * 16), None) == abi.MOE_OK


@pytest.mark.parametrize("which", range(16))
def test_step_entry_points_reject_each_misaligned_pointer(which):
    """Every pointer of the step entry points must be 16-byte aligned (the
    kernels read ids, codes and scales with 16-byte loads): one pointer at a
    4- or 24-byte offset gives MOE_ERR_ALIGN before any launch."""
    lib = abi.load()
    d = dims()
    ok = 1 << 20

    def ptrs(n):
        ps = [ctypes.c_void_p(ok + 4096 * i) for i in range(n)]
        if which < n:
            ps[which] = ctypes.c_void_p(ok + 4096 * which + (24 if which % 2 else 4))
        return ps

    calls = {
        "sort": lambda: lib.moe_a8w4_sort(ctypes.byref(d), 16, *ptrs(4), None),
        "quant_sort": lambda: lib.moe_a8w4_quant_sort(ctypes.byref(d), 16, *ptrs(7), None),
        "stage1": lambda: lib.moe_a8w4_stage1(ctypes.byref(d), 16, *ptrs(9), None),
        "stage2": lambda: lib.moe_a8w4_stage2(ctypes.byref(d), 16, *ptrs(9), None),
        "combine": lambda: lib.moe_a8w4_combine(ctypes.byref(d), *ptrs(3), None),
        "quant_act": lambda: lib.moe_a8w4_quant_act(4, 512, *ptrs(3), None),
        "stages_fused": lambda: lib.moe_a8w4_stages_fused(ctypes.byref(d), 16, *ptrs(16), None),
        "a16_stage1": lambda: lib.moe_a16w4_stage1(ctypes.byref(d), 16, *ptrs(7), None),
        "forward": lambda: lib.moe_a8w4_forward(ctypes.byref(d), *ptrs(9), 1 << 40, None),
    }
    nptr = {"sort": 4, "quant_sort": 7, "stage1": 9, "stage2": 9, "combine": 3, "quant_act": 3,
            "stages_fused": 16, "a16_stage1": 7, "forward": 9}
    for name, call in calls.items():
        if which < nptr[name]:
            assert call() == abi.MOE_ERR_ALIGN, (name, which)


def test_mfma_probe_validates():
    lib = abi.load()
    p = ctypes.c_void_p(1 << 20)
    assert lib.moe_a8w4_mfma_probe(0, 0, None, None, None, None, None, None) == abi.MOE_OK
    assert lib.moe_a8w4_mfma_probe(1, 4, p, p, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_mfma_probe(-1, 0, p, p, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_mfma_probe(1, 0, p, None, p, p, p, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_mfma_probe(1, 0, ctypes.c_void_p((1 << 20) + 8), p, p, p, p, None) == abi.MOE_ERR_ALIGN
    assert lib.moe_a8w4_stream_probe(0, 0, 512, None, None, None, None) == abi.MOE_OK
    assert lib.moe_a8w4_stream_probe(2, 64, 512, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_stream_probe(0, 65, 512, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_stream_probe(1, 64, 384, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a8w4_stream_probe(1, 64, 512, p, None, p, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_stream_probe(0, 64, 512, p, p, ctypes.c_void_p((1 << 20) + 4), None) == abi.MOE_ERR_ALIGN
    assert lib.moe_a16w4_mfma_probe(0, None, None, None, None) == abi.MOE_OK
    assert lib.moe_a16w4_mfma_probe(-1, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a16w4_mfma_probe((1 << 24) + 1, p, p, p, None) == abi.MOE_ERR_DIMS
    assert lib.moe_a16w4_mfma_probe(1, p, None, p, None) == abi.MOE_ERR_NULL
    assert lib.moe_a16w4_mfma_probe(1, p, p, ctypes.c_void_p((1 << 20) + 4), None) == abi.MOE_ERR_ALIGN


def test_noalloc_entry_point_validates_before_touching_the_gpu():
    """Oversized calls give MOE_ERR_SCRATCH, bad pointers their status, M = 0
    succeeds; all before any HIP call (no GPU here)."""
    lib = abi.load()
    p = ctypes.c_void_p(1 << 20)
    big = dims(tokens=16384, num_experts=385, topk=7)
    assert abi.moe_a8w4_workspace_bytes(big) > abi.NOALLOC_SCRATCH_BYTES
    assert lib.moe_a8w4_forward_noalloc(ctypes.byref(big), *([p] * 8), None) == abi.MOE_ERR_SCRATCH
    d = dims(tokens=768, num_experts=384, topk=6)
    assert abi.moe_a8w4_workspace_bytes(d) <= abi.NOALLOC_SCRATCH_BYTES
    assert lib.moe_a8w4_forward_noalloc(ctypes.byref(d), *([p] * 7), None, None) == abi.MOE_ERR_NULL
    assert lib.moe_a8w4_forward_noalloc(ctypes.byref(d), ctypes.c_void_p((1 << 20) + 4), *([p] * 7),
                                        None) == abi.MOE_ERR_ALIGN
    assert lib.moe_a8w4_forward_noalloc(ctypes.byref(dims(tokens=0)), *([None] * 8), None) == abi.MOE_OK
    assert "scratch" in abi.status_str(abi.MOE_ERR_SCRATCH)
