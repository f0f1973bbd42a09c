"""Pins of the oracle's group-by-expert permutation (CPU only)."""
import numpy as np
import pytest

from oracle import permute


@pytest.mark.parametrize("t,k,e,seed", [(1, 1, 1, 0), (7, 2, 8, 1), (64, 8, 256, 2), (33, 3, 5, 3), (0, 2, 4, 4)])
def test_matches_library_stable_sort_and_invariants(t, k, e, seed):
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.permutation(e)[:k] for _ in range(t)]) if t else np.zeros((0, k), np.int64)
    counts, offsets, perm, inv = permute.permute(ids, e)
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=e))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=e))]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert counts.sum() == t * k
    assert np.array_equal(np.sort(perm), np.arange(t * k))
    assert np.array_equal(perm[inv], np.arange(t * k))
    assert np.all(np.diff(flat[perm]) >= 0)
    for ex in range(e):
        seg = perm[offsets[ex]:offsets[ex + 1]]
        assert np.all(np.diff(seg) > 0)
        assert np.all(flat[seg] == ex)
