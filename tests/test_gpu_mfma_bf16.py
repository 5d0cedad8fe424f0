"""The BF16 matrix instruction of the A16W4 variant (16 x 16 x 32, FP32
result), run through the C ABI's probe entry point and compared with exact
arithmetic.  It pins the premise of the A16W4 intermediate budget: the
instruction's result is within 2^-16 of the sum of |products| of the exact
sum, and its operand layout is the one the A16W4 kernels assume.  A product
of two BF16 values is exact in FP64, and so (to 2^-46 relative) is a sum of
32 of them."""
import numpy as np
import pytest
import torch

from mixture_experts_fp8_amd import abi
from gpu_util import DEV, note

pytestmark = pytest.mark.gpu


def bf16(x):
    """float64 -> BF16 (round to nearest even, through float32) as torch.bfloat16."""
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.bfloat16)


def run(a, b):
    d = abi.moe_a16w4_mfma_probe(a.contiguous().to(DEV), b.contiguous().to(DEV))
    torch.cuda.synchronize()
    return d.cpu().numpy().astype(np.float64)


def operands(n, seed, spread):
    """A [n, 16, 32] and B [n, 16, 32] BF16, magnitudes 2^U(-spread, spread)."""
    rng = np.random.default_rng(seed)
    mk = lambda: rng.standard_normal((n, 16, 32)) * np.exp2(rng.uniform(-spread, spread, (n, 16, 32)))
    return bf16(mk()), bf16(mk())


@pytest.mark.parametrize("spread", [2, 12])
def test_accumulation_error_within_the_a16w4_budget(spread):
    a, b = operands(4096, [21, spread], spread)
    A, B = a.double().numpy(), b.double().numpy()
    P = A[:, :, None, :] * B[:, None, :, :]
    exact, l1 = P.sum(axis=3), np.abs(P).sum(axis=3)
    got = run(a, b)
    err = np.abs(got - exact)
    ratio = err[l1 > 0] / l1[l1 > 0]
    note("bf16 MFMA, exponent spread +-%d: error / sum |product|: worst 2^%.2f, median 2^%.2f" % (
        spread, np.log2(max(float(ratio.max()), 2.0 ** -80)), np.log2(max(float(np.median(ratio)), 2.0 ** -80))))
    assert np.all(err <= 2.0 ** -16 * l1)


def test_one_hot_layout():
    """A single nonzero element of A at (row m, k) and of B at (column c, k')
    gives a nonzero output only at (m, c), and only when k = k'."""
    rng = np.random.default_rng(23)
    n = 96
    A = np.zeros((n, 16, 32))
    B = np.zeros((n, 16, 32))
    m, c, k = rng.integers(0, 16, n), rng.integers(0, 16, n), rng.integers(0, 32, n)
    kb = np.where(np.arange(n) % 4 == 0, (k + 1 + rng.integers(0, 31, n)) % 32, k)
    A[np.arange(n), m, k] = 1.5
    B[np.arange(n), c, kb] = -2.0
    d = run(bf16(A), bf16(B))
    for i in range(n):
        want = np.zeros((16, 16))
        if kb[i] == k[i]:
            want[m[i], c[i]] = -3.0
        assert np.array_equal(d[i], want), i
