"""Pins of the oracle's route sort: an independent numpy statement of the same
grouping (stable sort by local expert), plus the closed-form size and the
per-block invariants, across block sizes and the boundary token counts that
the pages' validation lists (31/32/33/255/256/257)."""
import numpy as np
import pytest

from mixture_experts_fp8_amd import workloads as wl


def sort_numpy(ids, E, offset, bm):
    M, k = ids.shape
    le = ids.astype(np.int64).ravel() - offset
    f = np.arange(M * k)
    local = (le >= 0) & (le < E)
    f, le = f[local], le[local]
    order = np.argsort(le, kind="stable")      # stable: ascending f within an expert
    f, le = f[order], le[order]
    out, bexp = [], []
    for e in np.unique(le):
        fs = f[le == e]
        enc = ((fs % k) << 24) | (fs // k)
        pad = (-len(fs)) % bm
        out += enc.tolist() + [M] * pad
        bexp += [int(e)] * ((len(fs) + pad) // bm)
    return np.array(out, np.int32), np.array(bexp, np.int32)


CASES = []
for M in (1, 5, 31, 32, 33, 255, 256, 257):
    for bm in (16, 32, 64, 128, 256):
        CASES.append((M, bm))


@pytest.mark.parametrize("M,bm", CASES)
def test_sort_matches_independent_statement(oracle, M, bm):
    w = wl.WORKLOADS["backbone-decode"]
    _, ids, _ = wl.make_inputs(wl.scaled(w, hidden=64), M, "softmax", seed=[7, M])
    s, b = oracle.sort(ids, 384, 0, bm)
    s_ref, b_ref = sort_numpy(ids, 384, 0, bm)
    assert np.array_equal(s, s_ref)
    assert np.array_equal(b, b_ref)
    counts = np.bincount(ids.ravel(), minlength=384)
    assert len(s) == int(sum((c + bm - 1) // bm * bm for c in counts))


def test_sort_invariants_with_nonlocal_and_duplicates(oracle):
    rng = np.random.default_rng(4)
    M, k, E, off, bm = 257, 6, 96, 100, 32
    ids = rng.integers(-5, 400, size=(M, k)).astype(np.int32)
    ids[3, 1] = ids[3, 0]                        # a duplicated expert within a token
    s, b = oracle.sort(ids, E, off, bm)
    s_ref, b_ref = sort_numpy(ids, E, off, bm)
    assert np.array_equal(s, s_ref) and np.array_equal(b, b_ref)
    # every local route appears exactly once; every block is one expert, ascending f
    real = s[s != M]
    t, kk = real & 0xFFFFFF, real >> 24
    le = ids[t, kk].astype(np.int64) - off
    assert np.all((le >= 0) & (le < E))
    assert len(real) == int(((ids - off >= 0) & (ids - off < E)).sum())
    assert len(set((t * k + kk).tolist())) == len(real)
    for blk in range(len(b)):
        rows = s[blk * bm:(blk + 1) * bm]
        rr = rows[rows != M]
        assert len(rr) > 0
        assert np.all(ids[rr & 0xFFFFFF, rr >> 24] - off == b[blk])
        f = (rr & 0xFFFFFF) * k + (rr >> 24)
        assert np.all(np.diff(f) > 0)
    assert np.all(np.diff(b) >= 0)


def test_sort_empty_and_all_nonlocal(oracle):
    s, b = oracle.sort(np.zeros((0, 6), np.int32), 384, 0, 32)
    assert len(s) == 0 and len(b) == 0
    s, b = oracle.sort(np.full((9, 6), 999, np.int32), 384, 0, 32)
    assert len(s) == 0 and len(b) == 0
