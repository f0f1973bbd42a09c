"""Pins of the oracle's router (CPU only)."""
import numpy as np
import pytest
from scipy.special import softmax

from oracle import router


def test_weights_sum_to_one_and_follow_order():
    rng = np.random.default_rng(0)
    L = rng.normal(0, 2, size=(50, 32)).astype(np.float32)
    ids = router.select_topk(L, 4)
    w = router.topk_weights(L, ids)
    assert np.allclose(w.sum(axis=1), 1.0, atol=2.0 ** -40)
    assert np.all(np.diff(w, axis=1) <= 0)                 # descending logit -> descending weight


def test_selection_equals_bruteforce_lexsort():
    rng = np.random.default_rng(1)
    # few distinct values -> many exact ties
    L = rng.integers(-3, 3, size=(40, 16)).astype(np.float32)
    ids = router.select_topk(L, 5)
    for r in range(L.shape[0]):
        order = np.lexsort((np.arange(16), -L[r].astype(np.float64)))
        assert ids[r].tolist() == order[:5].tolist()
        # selected values are the 5 largest
        assert np.allclose(np.sort(L[r, ids[r]]), np.sort(L[r])[-5:])


def test_exact_ties_pick_lower_index():
    L = np.zeros((1, 8), dtype=np.float32)
    L[0, [2, 5, 7]] = 1.0
    assert router.select_topk(L, 2)[0].tolist() == [2, 5]
    assert router.select_topk(L, 4)[0].tolist() == [2, 5, 7, 0]


def test_k_equals_e_is_full_softmax():
    rng = np.random.default_rng(2)
    L = rng.normal(0, 3, size=(20, 8))
    ids = router.select_topk(L, 8)
    w = router.topk_weights(L, ids)
    ref = softmax(L, axis=1)
    got = np.zeros_like(ref)
    np.put_along_axis(got, ids.astype(np.int64), w, axis=1)
    assert np.allclose(got, ref, rtol=1e-14, atol=1e-16)


def test_renormalised_topk_equals_softmax_then_renormalise():
    rng = np.random.default_rng(3)
    L = rng.normal(0, 3, size=(20, 64))
    ids = router.select_topk(L, 8)
    w = router.topk_weights(L, ids)
    p = softmax(L, axis=1)
    sel = np.take_along_axis(p, ids.astype(np.int64), axis=1)
    assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-13)


def test_single_expert_weight_is_exactly_one():
    L = np.array([[3.5], [-2.0]], dtype=np.float32)
    ids = router.select_topk(L, 1)
    assert ids.tolist() == [[0], [0]]
    assert router.topk_weights(L, ids).tolist() == [[1.0], [1.0]]


def test_logits_definition_and_bias():
    rng = np.random.default_rng(4)
    x = rng.normal(size=(3, 5))
    w = rng.normal(size=(4, 5))
    b = rng.normal(size=4)
    L = router.logits_fp64(x, w, b)
    for t in range(3):
        for e in range(4):
            assert L[t, e] == pytest.approx(sum(x[t, i] * w[e, i] for i in range(5)) + b[e], rel=1e-14)


def test_bad_k_rejected():
    with pytest.raises(ValueError):
        router.select_topk(np.zeros((1, 4)), 5)
