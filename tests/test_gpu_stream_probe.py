"""The weight-streaming probe behind the packed weight layout
(moe_a8w4_stream_probe): reading raw row-major MXFP4 weights and reading
their packed form (moe_a8w4_pack_weights) must load the same bytes into the
same lanes, so the two layouts give the same per-wave words; and those words
equal a host fold of the raw bytes in that lane assignment."""
import numpy as np
import pytest
import torch

from mixture_experts_fp8_amd import abi
from gpu_util import DEV

pytestmark = pytest.mark.gpu


def host_words(codes, scales, rows, K):
    """The probe's fold on the host from the raw layout: lane (m, q) of tile t
    at step s loads row 64 G + 16 (m >> 2) + 4 t + (m & 3), bytes 64 s + 16 q
    .. +16 (as 4 little-endian int32), and the tile's scale byte 4 s + q."""
    KS = K // 128
    c = codes.reshape(rows, K // 2)
    sc = scales.reshape(rows, K // 32).astype(np.uint32)
    out = np.zeros(rows // 64 * 4, np.uint32)
    m = np.arange(64) & 15
    q = np.arange(64) >> 4
    for G in range(rows // 64):
        for wave in range(4):
            acc = np.zeros(64, np.uint32)
            for s in range(wave * KS // 4, (wave + 1) * KS // 4):
                words, sw = [], np.zeros(64, np.uint32)
                for t in range(4):
                    row = G * 64 + 16 * (m >> 2) + 4 * t + (m & 3)
                    seg = np.stack([c[row[l], 64 * s + 16 * q[l]: 64 * s + 16 * q[l] + 16] for l in range(64)])
                    words.append(seg.view(np.uint32))     # [64, 4]
                    sw |= sc[row, 4 * s + q] << np.uint32(8 * t)
                acc += (words[0][:, 0] ^ words[1][:, 1] ^ words[2][:, 2] ^ words[3][:, 3]) + sw
            out[G * 4 + wave] = acc.sum(dtype=np.uint64) & 0xFFFFFFFF
    return out


def test_packed_and_raw_layouts_read_the_same_fragments():
    E, I, H = 2, 128, 1024            # w13: E x 2I rows of K = H
    rng = np.random.default_rng(31)
    w13 = rng.integers(0, 256, (E, 2 * I, H // 2), dtype=np.uint8)
    w13_s = rng.integers(100, 140, (E, 2 * I, H // 32), dtype=np.uint8)
    w2 = rng.integers(0, 256, (E, H, I // 2), dtype=np.uint8)
    w2_s = rng.integers(100, 140, (E, H, I // 32), dtype=np.uint8)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(DEV)
    d = abi.make_dims(1, H, I, E, 1)
    p13, p13_s, _, _ = abi.moe_a8w4_pack_weights(d, t(w13), t(w13_s), t(w2), t(w2_s))
    rows = E * 2 * I
    packed = abi.moe_a8w4_stream_probe(0, rows, H, p13, p13_s)
    raw = abi.moe_a8w4_stream_probe(1, rows, H, t(w13), t(w13_s))
    torch.cuda.synchronize()
    got_p = packed.cpu().numpy().view(np.uint32)
    got_r = raw.cpu().numpy().view(np.uint32)
    assert np.array_equal(got_p, got_r)
    assert np.array_equal(got_r, host_words(w13.reshape(-1), w13_s.reshape(-1), rows, H))
