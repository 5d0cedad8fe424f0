"""bench.py on the host: the one-GPU contract and the byte model behind its
roofline figure (no GPU needed)."""
import os
import subprocess
import sys

import numpy as np

import bench
from mixture_experts_fp8_amd import workloads as wl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_algorithmic_bytes_of_a_small_call():
    """Two tokens, top-2, four local experts at offset 0; one slot is
    non-local. Counted by hand: 3 local routes on 2 distinct experts."""
    w = wl.scaled(wl.WORKLOADS["draft-decode"], hidden=512, inter=128, inter_valid=128, num_experts=4,
                  routed_experts=8, expert_offset=0, topk=2)
    ids = np.array([[0, 1], [1, 5]], np.int32)
    a = bench.algorithmic(w, 2, ids)
    H, I, M, k = 512, 128, 2, 2
    w13 = 2 * I * (H // 2 + H // 32)          # 69,632 B per expert
    w2 = H * (I // 2 + I // 32)               # 34,816 B per expert
    act = M * (H + H // 32)                   # FP8 codes + scales of the tokens
    inter = 3 * (I + I // 32)                 # requantised intermediate of 3 routes
    assert (a["R"], a["D"]) == (3, 2)
    assert a["stage1_bytes"] == 2 * w13 + act + inter == 140_716
    # whole call: weights, BF16 in and out, ids + weights, quantised activations and
    # intermediate written and read once each
    assert a["bytes"] == 2 * (w13 + w2) + M * H * 2 + M * k * 8 + 2 * act + 2 * inter + M * H * 2
    assert a["stage1_flops"] == 4.0 * 3 * I * H and a["flops"] == 6.0 * 3 * I * H
