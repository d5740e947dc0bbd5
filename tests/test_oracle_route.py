"""Pins of the oracle's router (softmax over a token's logits -> top k -> optional
renormalization -> optional expert-parallel id map) against closed forms, brute force
and invariants, independent of the oracle's own code."""
import itertools

import numpy as np
import pytest

import oracle


def test_closed_form_weights():
    # logits log(c): softmax probabilities are c / sum(c), so the renormalized top-k
    # weights are c_i / sum over the k largest c, and the plain ones c_i / sum(c).
    c = np.array([3.0, 1.0, 7.0, 2.0, 5.0, 4.0, 6.0, 8.0])
    logits = np.log(c).astype(np.float32)[None, :]
    ids, w = oracle.topk_softmax(logits, 3, renormalize=True)
    assert ids.tolist() == [[7, 2, 6]]
    np.testing.assert_allclose(w[0], np.array([8.0, 7.0, 6.0]) / 21.0, rtol=1e-6)
    ids, w = oracle.topk_softmax(logits, 3, renormalize=False)
    assert ids.tolist() == [[7, 2, 6]]
    np.testing.assert_allclose(w[0], np.array([8.0, 7.0, 6.0]) / c.sum(), rtol=1e-6)


@pytest.mark.parametrize("E,k", [(5, 1), (6, 2), (7, 3), (8, 4), (8, 8)])
def test_brute_force_selection(E, k):
    rng = np.random.default_rng(100 + E * 10 + k)
    logits = rng.standard_normal((20, E)).astype(np.float32)
    ids, w = oracle.topk_softmax(logits, k)
    for t in range(20):
        l = logits[t].astype(np.float64)
        # distinct values: the top-k set is the unique k-subset with the largest sum
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(l[list(s)]))
        assert sorted(ids[t].tolist()) == sorted(best)
        assert all(l[ids[t][i]] > l[ids[t][i + 1]] for i in range(k - 1))
        p = np.exp(l - l.max()) / np.exp(l - l.max()).sum()
        np.testing.assert_allclose(w[t], p[ids[t]] / p[ids[t]].sum(), rtol=1e-12)


def test_ties_keep_the_lower_id_and_signed_zeros_are_equal():
    logits = np.array([[1.0, 3.0, 3.0, 2.0, 3.0],
                       [0.0, -0.0, -1.0, 0.0, -2.0]], np.float32)
    ids, w = oracle.topk_softmax(logits, 3)
    assert ids[0].tolist() == [1, 2, 4]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=1e-12)
    assert ids[1].tolist() == [0, 1, 3]
    np.testing.assert_allclose(w[1], [1 / 3] * 3, rtol=1e-12)


def test_shift_invariance_and_large_logits():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((50, 48)).astype(np.float32)
    ids0, w0 = oracle.topk_softmax(logits, 8)
    # exp of logits near 1e4 overflows without subtracting the maximum
    big = (logits.astype(np.float64) + 10000.0).astype(np.float32)
    ids1, w1 = oracle.topk_softmax(big, 8)
    assert np.all(np.isfinite(w1))
    same = ids0 == ids1  # fp32 rounding of the shift can merge close logits
    assert same.mean() > 0.9
    np.testing.assert_allclose(w1.sum(axis=1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(w0[:, 0][same[:, 0]], w1[:, 0][same[:, 0]], rtol=0.05)


def test_invariants_on_random_tokens():
    rng = np.random.default_rng(11)
    for E, k in [(48, 8), (384, 8), (16, 16)]:
        logits = rng.standard_normal((64, E)).astype(np.float32)
        ids, w = oracle.topk_softmax(logits, k)
        _, p = oracle.topk_softmax(logits, k, renormalize=False)
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-12)
        assert np.all(np.diff(w, axis=1) <= 0) and np.all(np.diff(p, axis=1) <= 0)
        assert all(len(set(r)) == k for r in ids.tolist())
        assert np.all(p.sum(axis=1) <= 1.0 + 1e-12)
        if k == E:
            np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-12)
        np.testing.assert_allclose(w, p / p.sum(axis=1, keepdims=True), rtol=1e-12)


def test_expert_map_changes_ids_only():
    rng = np.random.default_rng(5)
    E, k = 32, 4
    logits = rng.standard_normal((40, E)).astype(np.float32)
    emap = np.full(E, -1, np.int32)
    emap[8:16] = np.arange(8)  # this GPU holds global experts 8..15
    ids, w = oracle.topk_softmax(logits, k)
    mids, mw = oracle.topk_softmax(logits, k, expert_map=emap)
    np.testing.assert_array_equal(mw, w)
    np.testing.assert_array_equal(mids, emap[ids])
