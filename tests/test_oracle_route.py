"""Pins of the oracle's router (softmax top-k, renormalised, optional shared
slot) against torch's CPU top-k and softmax, closed forms and invariants."""
import numpy as np
import torch

import oracle


def test_matches_torch_topk_and_softmax():
    rng = np.random.default_rng(5)
    for M, Er, k in [(64, 384, 6), (33, 128, 3), (17, 100, 8), (5, 8, 1)]:
        logits = rng.standard_normal((M, Er), dtype=np.float32)
        ids, wts = oracle.softmax_topk(logits, k)
        tv, ti = torch.topk(torch.from_numpy(logits), k, dim=1, largest=True, sorted=True)
        assert np.array_equal(ids, ti.numpy().astype(np.int32))
        ref = torch.softmax(tv.double(), dim=1).numpy()
        assert np.abs(wts - ref).max() <= 1e-15
        # the renormalised full softmax is the same distribution
        full = torch.softmax(torch.from_numpy(logits).double(), dim=1).numpy()
        sel = np.take_along_axis(full, ids.astype(np.int64), axis=1)
        assert np.abs(wts - sel / sel.sum(axis=1, keepdims=True)).max() <= 1e-13


def test_closed_forms_and_ties():
    # two experts, logits 0 and 1: weights e / (1 + e) and 1 / (1 + e)
    ids, wts = oracle.softmax_topk(np.array([[0.0, 1.0]], np.float32), 2)
    assert ids.tolist() == [[1, 0]]
    assert abs(wts[0, 0] - np.e / (1 + np.e)) <= 1e-16 and abs(wts[0, 1] - 1 / (1 + np.e)) <= 1e-16
    # equal logits: lower ids first, equal weights
    ids, wts = oracle.softmax_topk(np.zeros((3, 10), np.float32), 4)
    assert ids.tolist() == [[0, 1, 2, 3]] * 3 and np.all(wts == 0.25)
    ids, wts = oracle.softmax_topk(np.array([[1, 3, 3, 2, 3]], np.float32), 3)
    assert ids.tolist() == [[1, 2, 4]] and np.allclose(wts, 1 / 3, rtol=0, atol=1e-16)


def test_shift_invariance_and_shared_slot():
    rng = np.random.default_rng(6)
    logits = rng.standard_normal((40, 384), dtype=np.float32)
    ids, wts = oracle.softmax_topk(logits, 6)
    ids2, wts2 = oracle.softmax_topk(logits + np.float32(4.0), 6)
    assert np.array_equal(ids, ids2)
    assert np.abs(wts - wts2).max() <= 1e-6   # the shift rounds the float32 logits
    assert np.allclose(wts.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    sid, swt = oracle.softmax_topk(logits, 6, shared_id=384)
    assert np.array_equal(sid[:, :6], ids) and np.all(sid[:, 6] == 384)
    assert np.array_equal(swt[:, :6], wts) and np.all(swt[:, 6] == 1.0)
