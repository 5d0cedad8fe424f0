"""Python binding of the C ABI in include/moe_a8w4.h (argument marshalling only).

Every function has the name of the C entry point it calls, takes torch
tensors that already live on the GPU, and launches on torch's current stream.
All compute runs in the HIP kernels of libmoe_a8w4.so; if that library is
missing, loading fails loudly.  There is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmoe_a8w4.so")

MOE_OK = 0
MOE_ERR_NULL = -1
MOE_ERR_DIMS = -2
MOE_ERR_ALIGN = -3
MOE_ERR_WORKSPACE = -4
MOE_ERR_BLOCK_M = -5
MOE_ERR_SCRATCH = -6
NOALLOC_SCRATCH_BYTES = 64 << 20

# every symbol include/moe_a8w4.h declares
EXPORTS = (
    "moe_a8w4_workspace_bytes", "moe_a8w4_block_m", "moe_a8w4_sort_capacity",
    "moe_a8w4_pack_weights", "moe_a8w4_forward", "moe_a8w4_quant_act", "moe_a8w4_sort",
    "moe_a8w4_quant_sort",
    "moe_a8w4_stage1", "moe_a8w4_stage2", "moe_a8w4_combine", "moe_a8w4_status_str",
    "moe_a8w4_route", "moe_a8w4_forward_routed", "moe_a8w4_stages_fused", "moe_a8w4_fused_counters",
    "moe_a16w4_forward", "moe_a16w4_workspace_bytes", "moe_a16w4_block_m", "moe_a16w4_stage1",
    "moe_a8w4_mfma_probe", "moe_a8w4_forward_noalloc", "moe_a16w4_mfma_probe", "moe_a8w4_stream_probe",
)


class moe_a8w4_dims(ctypes.Structure):
    _fields_ = [("tokens", ctypes.c_int32), ("hidden", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("num_experts", ctypes.c_int32), ("expert_offset", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("routed_experts", ctypes.c_int32)]


def make_dims(tokens, hidden, inter, num_experts, topk, expert_offset=0,
              routed_experts=0) -> moe_a8w4_dims:
    return moe_a8w4_dims(tokens, hidden, inter, num_experts, expert_offset, topk, routed_experts)


class MoeError(RuntimeError):
    def __init__(self, name, status):
        super().__init__("%s failed: status %d (%s)" % (name, status, status_str(status)))
        self.status = status


_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("HIP library %s is not built; run __graft_entry__.build()" % LIB_PATH)
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER(moe_a8w4_dims)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    sig = {
        "moe_a8w4_workspace_bytes": (ctypes.c_int, [P, ctypes.POINTER(sz)]),
        "moe_a8w4_block_m": (ctypes.c_int, [P]),
        "moe_a8w4_sort_capacity": (ctypes.c_int64, [P, i32]),
        "moe_a8w4_pack_weights": (ctypes.c_int, [P] + [vp] * 8 + [vp]),
        "moe_a8w4_forward": (ctypes.c_int, [P] + [vp] * 9 + [sz, vp]),
        "moe_a8w4_quant_act": (ctypes.c_int, [i32, i32, vp, vp, vp, vp]),
        "moe_a8w4_sort": (ctypes.c_int, [P, i32, vp, vp, vp, vp, vp]),
        "moe_a8w4_quant_sort": (ctypes.c_int, [P, i32] + [vp] * 7 + [vp]),
        "moe_a8w4_stage1": (ctypes.c_int, [P, i32] + [vp] * 9 + [vp]),
        "moe_a8w4_stage2": (ctypes.c_int, [P, i32] + [vp] * 9 + [vp]),
        "moe_a8w4_combine": (ctypes.c_int, [P, vp, vp, vp, vp]),
        "moe_a8w4_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "moe_a8w4_route": (ctypes.c_int, [i32, i32, i32, i32, vp, vp, vp, vp]),
        "moe_a8w4_forward_routed": (ctypes.c_int, [P, vp, vp, i32] + [vp] * 8 + [sz, vp]),
        "moe_a8w4_stages_fused": (ctypes.c_int, [P, i32] + [vp] * 16 + [vp]),
        "moe_a8w4_fused_counters": (ctypes.c_int64, [P, i32]),
        "moe_a16w4_forward": (ctypes.c_int, [P] + [vp] * 9 + [sz, vp]),
        "moe_a16w4_workspace_bytes": (ctypes.c_int, [P, ctypes.POINTER(sz)]),
        "moe_a16w4_block_m": (ctypes.c_int, [P]),
        "moe_a16w4_stage1": (ctypes.c_int, [P, i32] + [vp] * 7 + [vp]),
        "moe_a8w4_mfma_probe": (ctypes.c_int, [ctypes.c_int64, i32] + [vp] * 5 + [vp]),
        "moe_a8w4_forward_noalloc": (ctypes.c_int, [P] + [vp] * 8 + [vp]),
        "moe_a16w4_mfma_probe": (ctypes.c_int, [ctypes.c_int64, vp, vp, vp, vp]),
        "moe_a8w4_stream_probe": (ctypes.c_int, [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, vp, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().moe_a8w4_status_str(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(name, st):
    if st != MOE_OK:
        raise MoeError(name, st)


# ------------------------------------------------------------------ sizes

def moe_a8w4_workspace_bytes(dims: moe_a8w4_dims) -> int:
    n = ctypes.c_size_t(0)
    _check("moe_a8w4_workspace_bytes", load().moe_a8w4_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def moe_a8w4_block_m(dims: moe_a8w4_dims) -> int:
    bm = load().moe_a8w4_block_m(ctypes.byref(dims))
    if bm < 0:
        raise MoeError("moe_a8w4_block_m", bm)
    return bm


def moe_a8w4_sort_capacity(dims: moe_a8w4_dims, block_m: int) -> int:
    c = load().moe_a8w4_sort_capacity(ctypes.byref(dims), block_m)
    if c < 0:
        raise MoeError("moe_a8w4_sort_capacity", c)
    return c


# ---------------------------------------------------------------- weights

def moe_a8w4_pack_weights(dims, w13, w13_s, w2, w2_s, out=None, stream=None):
    """Packed copies (w13_p, w13_s_p, w2_p, w2_s_p) of uint8 device tensors."""
    if out is None:
        out = tuple(torch.empty_like(t) for t in (w13, w13_s, w2, w2_s))
    st = load().moe_a8w4_pack_weights(ctypes.byref(dims), _ptr(w13), _ptr(w13_s), _ptr(w2), _ptr(w2_s),
                                      *[_ptr(t) for t in out], _stream(stream))
    _check("moe_a8w4_pack_weights", st)
    return out


# -------------------------------------------------------------- the layer

def moe_a8w4_forward(dims, hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, w2_s_p,
                     out=None, workspace=None, stream=None):
    """BF16 output [M, H] of the layer (out and workspace are allocated if not given)."""
    if out is None:
        out = torch.empty((dims.tokens, dims.hidden), dtype=torch.bfloat16, device=hidden.device)
    if workspace is None:
        workspace = torch.empty(moe_a8w4_workspace_bytes(dims), dtype=torch.uint8, device=hidden.device)
    st = load().moe_a8w4_forward(ctypes.byref(dims), _ptr(hidden), _ptr(topk_ids), _ptr(topk_weights),
                                 _ptr(w13_p), _ptr(w13_s_p), _ptr(w2_p), _ptr(w2_s_p), _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream(stream))
    _check("moe_a8w4_forward", st)
    return out


def moe_a8w4_forward_noalloc(dims, hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, w2_s_p,
                             out=None, stream=None):
    """moe_a8w4_forward with the library's static device scratch as workspace
    (out is allocated here if not given; the C entry point allocates nothing)."""
    if out is None:
        out = torch.empty((dims.tokens, dims.hidden), dtype=torch.bfloat16, device=hidden.device)
    st = load().moe_a8w4_forward_noalloc(ctypes.byref(dims), _ptr(hidden), _ptr(topk_ids), _ptr(topk_weights),
                                         _ptr(w13_p), _ptr(w13_s_p), _ptr(w2_p), _ptr(w2_s_p), _ptr(out),
                                         _stream(stream))
    _check("moe_a8w4_forward_noalloc", st)
    return out


def moe_a8w4_route(logits, k_routed, shared_expert=-1, topk_ids=None, topk_weights=None, stream=None):
    """(topk_ids int32 [M, k], topk_weights float32 [M, k]) from router logits
    float32 [M, routed_experts]; k = k_routed + (shared_expert >= 0)."""
    M, Er = logits.shape
    k = k_routed + (1 if shared_expert >= 0 else 0)
    if topk_ids is None:
        topk_ids = torch.empty((M, k), dtype=torch.int32, device=logits.device)
    if topk_weights is None:
        topk_weights = torch.empty((M, k), dtype=torch.float32, device=logits.device)
    st = load().moe_a8w4_route(M, Er, k_routed, shared_expert, _ptr(logits), _ptr(topk_ids),
                               _ptr(topk_weights), _stream(stream))
    _check("moe_a8w4_route", st)
    return topk_ids, topk_weights


def moe_a8w4_forward_routed(dims, hidden, router_logits, shared_expert, w13_p, w13_s_p, w2_p, w2_s_p,
                            topk_ids=None, topk_weights=None, out=None, workspace=None, stream=None):
    """(out BF16 [M, H], topk_ids, topk_weights) of the layer routed from its
    logits [M, dims.routed_experts] (outputs allocated if not given)."""
    dev = hidden.device
    if topk_ids is None:
        topk_ids = torch.empty((dims.tokens, dims.topk), dtype=torch.int32, device=dev)
    if topk_weights is None:
        topk_weights = torch.empty((dims.tokens, dims.topk), dtype=torch.float32, device=dev)
    if out is None:
        out = torch.empty((dims.tokens, dims.hidden), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(moe_a8w4_workspace_bytes(dims), dtype=torch.uint8, device=dev)
    st = load().moe_a8w4_forward_routed(ctypes.byref(dims), _ptr(hidden), _ptr(router_logits), shared_expert,
                                        _ptr(topk_ids), _ptr(topk_weights), _ptr(w13_p), _ptr(w13_s_p),
                                        _ptr(w2_p), _ptr(w2_s_p), _ptr(out), _ptr(workspace),
                                        workspace.numel(), _stream(stream))
    _check("moe_a8w4_forward_routed", st)
    return out, topk_ids, topk_weights


# ------------------------------------------------------------- the steps

def moe_a8w4_quant_act(x, q=None, s=None, stream=None):
    M, H = x.shape
    if q is None:
        q = torch.empty((M, H), dtype=torch.uint8, device=x.device)
    if s is None:
        s = torch.empty((M, H // 32), dtype=torch.uint8, device=x.device)
    st = load().moe_a8w4_quant_act(M, H, _ptr(x), _ptr(q), _ptr(s), _stream(stream))
    _check("moe_a8w4_quant_act", st)
    return q, s


def moe_a8w4_sort(dims, block_m, topk_ids, sorted_ids=None, block_expert=None, num_padded=None,
                  stream=None):
    cap = moe_a8w4_sort_capacity(dims, block_m)
    dev = topk_ids.device
    if sorted_ids is None:
        sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    if block_expert is None:
        block_expert = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    if num_padded is None:
        num_padded = torch.empty(1, dtype=torch.int32, device=dev)
    st = load().moe_a8w4_sort(ctypes.byref(dims), block_m, _ptr(topk_ids), _ptr(sorted_ids),
                              _ptr(block_expert), _ptr(num_padded), _stream(stream))
    _check("moe_a8w4_sort", st)
    return sorted_ids, block_expert, num_padded


def moe_a8w4_quant_sort(dims, block_m, hidden, topk_ids, stream=None):
    """(a_q, a_s, sorted_ids, block_expert, num_padded) from one launch."""
    cap = moe_a8w4_sort_capacity(dims, block_m)
    dev = hidden.device
    M, H = dims.tokens, dims.hidden
    a_q = torch.empty((M, H), dtype=torch.uint8, device=dev)
    a_s = torch.empty((M, H // 32), dtype=torch.uint8, device=dev)
    sorted_ids = torch.empty(max(cap, 1), dtype=torch.int32, device=dev)
    block_expert = torch.empty(max(cap // block_m, 1), dtype=torch.int32, device=dev)
    num_padded = torch.empty(1, dtype=torch.int32, device=dev)
    st = load().moe_a8w4_quant_sort(ctypes.byref(dims), block_m, _ptr(hidden), _ptr(topk_ids), _ptr(a_q),
                                    _ptr(a_s), _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
                                    _stream(stream))
    _check("moe_a8w4_quant_sort", st)
    return a_q, a_s, sorted_ids, block_expert, num_padded


def moe_a8w4_stage1(dims, block_m, a_q, a_s, sorted_ids, block_expert, num_padded, w13_p, w13_s_p,
                    inter_q=None, inter_s=None, stream=None):
    cap = moe_a8w4_sort_capacity(dims, block_m)
    dev = a_q.device
    if inter_q is None:
        inter_q = torch.empty((cap, dims.inter), dtype=torch.uint8, device=dev)
    if inter_s is None:
        inter_s = torch.empty((cap, dims.inter // 32), dtype=torch.uint8, device=dev)
    st = load().moe_a8w4_stage1(ctypes.byref(dims), block_m, _ptr(a_q), _ptr(a_s), _ptr(sorted_ids),
                                _ptr(block_expert), _ptr(num_padded), _ptr(w13_p), _ptr(w13_s_p),
                                _ptr(inter_q), _ptr(inter_s), _stream(stream))
    _check("moe_a8w4_stage1", st)
    return inter_q, inter_s


def route_rows_bytes(dims):
    """Bytes of the stage-two route rows: [M, topk, H] int16 codes, then
    [M, topk, H/32] exponent bytes."""
    return dims.tokens * dims.topk * (2 * dims.hidden + dims.hidden // 32)


def moe_a8w4_stage2(dims, block_m, inter_q, inter_s, sorted_ids, block_expert, num_padded,
                    topk_weights, w2_p, w2_s_p, y_routes=None, stream=None):
    if y_routes is None:
        y_routes = torch.empty(route_rows_bytes(dims), dtype=torch.uint8, device=inter_q.device)
    st = load().moe_a8w4_stage2(ctypes.byref(dims), block_m, _ptr(inter_q), _ptr(inter_s),
                                _ptr(sorted_ids), _ptr(block_expert), _ptr(num_padded),
                                _ptr(topk_weights), _ptr(w2_p), _ptr(w2_s_p), _ptr(y_routes),
                                _stream(stream))
    _check("moe_a8w4_stage2", st)
    return y_routes


def moe_a8w4_fused_counters(dims, block_m) -> int:
    n = load().moe_a8w4_fused_counters(ctypes.byref(dims), block_m)
    if n < 0:
        raise MoeError("moe_a8w4_fused_counters", n)
    return n


def moe_a8w4_stages_fused(dims, block_m, a_q, a_s, sorted_ids, block_expert, num_padded, topk_ids,
                          topk_weights, w13_p, w13_s_p, w2_p, w2_s_p, counters, inter_q=None,
                          inter_s=None, y_routes=None, out=None, stream=None):
    """Stage one, stage two and the combine in one launch; counters (int32,
    moe_a8w4_fused_counters entries) must be zero and are left zero.
    Returns (inter_q, inter_s, y_routes, out)."""
    dev = a_q.device
    cap = moe_a8w4_sort_capacity(dims, block_m)
    if inter_q is None:
        inter_q = torch.empty((cap, dims.inter), dtype=torch.uint8, device=dev)
    if inter_s is None:
        inter_s = torch.empty((cap, dims.inter // 32), dtype=torch.uint8, device=dev)
    if y_routes is None:
        y_routes = torch.empty(route_rows_bytes(dims), dtype=torch.uint8, device=dev)
    if out is None:
        out = torch.empty((dims.tokens, dims.hidden), dtype=torch.bfloat16, device=dev)
    st = load().moe_a8w4_stages_fused(ctypes.byref(dims), block_m, _ptr(a_q), _ptr(a_s), _ptr(sorted_ids),
                                      _ptr(block_expert), _ptr(num_padded), _ptr(topk_ids),
                                      _ptr(topk_weights), _ptr(w13_p), _ptr(w13_s_p), _ptr(w2_p),
                                      _ptr(w2_s_p), _ptr(inter_q), _ptr(inter_s), _ptr(y_routes),
                                      _ptr(counters), _ptr(out), _stream(stream))
    _check("moe_a8w4_stages_fused", st)
    return inter_q, inter_s, y_routes, out


def moe_a16w4_workspace_bytes(dims) -> int:
    n = ctypes.c_size_t()
    _check("moe_a16w4_workspace_bytes", load().moe_a16w4_workspace_bytes(ctypes.byref(dims), ctypes.byref(n)))
    return n.value


def moe_a16w4_block_m(dims) -> int:
    bm = load().moe_a16w4_block_m(ctypes.byref(dims))
    if bm < 0:
        raise MoeError("moe_a16w4_block_m", bm)
    return bm


def moe_a16w4_forward(dims, hidden, topk_ids, topk_weights, w13_p, w13_s_p, w2_p, w2_s_p,
                      out=None, workspace=None, stream=None):
    """The A16W4 variant of the layer: BF16 hidden [M, H] -> BF16 out [M, H]."""
    dev = hidden.device
    if out is None:
        out = torch.empty((dims.tokens, dims.hidden), dtype=torch.bfloat16, device=dev)
    if workspace is None:
        workspace = torch.empty(max(moe_a16w4_workspace_bytes(dims), 1), dtype=torch.uint8, device=dev)
    st = load().moe_a16w4_forward(ctypes.byref(dims), _ptr(hidden), _ptr(topk_ids), _ptr(topk_weights),
                                  _ptr(w13_p), _ptr(w13_s_p), _ptr(w2_p), _ptr(w2_s_p), _ptr(out),
                                  _ptr(workspace), workspace.numel(), _stream(stream))
    _check("moe_a16w4_forward", st)
    return out


def moe_a16w4_stage1(dims, block_m, hidden, sorted_ids, block_expert, num_padded, w13_p, w13_s_p,
                     inter=None, stream=None):
    """A16W4 stage one -> BF16 intermediate [capacity, I] in sorted-row order."""
    if inter is None:
        cap = moe_a8w4_sort_capacity(dims, block_m)
        inter = torch.empty((cap, dims.inter), dtype=torch.bfloat16, device=hidden.device)
    st = load().moe_a16w4_stage1(ctypes.byref(dims), block_m, _ptr(hidden), _ptr(sorted_ids),
                                 _ptr(block_expert), _ptr(num_padded), _ptr(w13_p), _ptr(w13_s_p),
                                 _ptr(inter), _stream(stream))
    _check("moe_a16w4_stage1", st)
    return inter


def moe_a8w4_combine(dims, topk_ids, y_routes, out=None, stream=None):
    if out is None:
        out = torch.empty((dims.tokens, dims.hidden), dtype=torch.bfloat16, device=y_routes.device)
    st = load().moe_a8w4_combine(ctypes.byref(dims), _ptr(topk_ids), _ptr(y_routes), _ptr(out),
                                 _stream(stream))
    _check("moe_a8w4_combine", st)
    return out


def moe_a8w4_mfma_probe(a_fp4, a_scale, b_fp8, b_scale, byte_sel=0, d=None, stream=None):
    """n scaled MFMAs: a_fp4 [n,16,64], a_scale [n,16,4], b_fp8 [n,16,128],
    b_scale [n,16,4] uint8 -> d float32 [n,16,16]."""
    n = a_fp4.shape[0]
    if d is None:
        d = torch.empty((n, 16, 16), dtype=torch.float32, device=a_fp4.device)
    st = load().moe_a8w4_mfma_probe(n, byte_sel, _ptr(a_fp4), _ptr(a_scale), _ptr(b_fp8), _ptr(b_scale),
                                    _ptr(d), _stream(stream))
    _check("moe_a8w4_mfma_probe", st)
    return d


def moe_a16w4_mfma_probe(a_bf16, b_bf16, d=None, stream=None):
    """n BF16 MFMAs: a_bf16 [n,16,32], b_bf16 [n,16,32] (torch.bfloat16) -> d float32 [n,16,16]."""
    n = a_bf16.shape[0]
    if d is None:
        d = torch.empty((n, 16, 16), dtype=torch.float32, device=a_bf16.device)
    st = load().moe_a16w4_mfma_probe(n, _ptr(a_bf16), _ptr(b_bf16), _ptr(d), _stream(stream))
    _check("moe_a16w4_mfma_probe", st)
    return d


def moe_a8w4_stream_probe(layout, rows, K, w, w_s, out=None, stream=None):
    """Weight-streaming probe: layout 0 packed, 1 raw row-major; out uint32 [rows / 64 * 4]."""
    if out is None:
        out = torch.empty(rows // 64 * 4, dtype=torch.int32, device=w.device)
    st = load().moe_a8w4_stream_probe(layout, rows, K, _ptr(w), _ptr(w_s), _ptr(out), _stream(stream))
    _check("moe_a8w4_stream_probe", st)
    return out
