"""Pins for oracle.topk: exact Top-K, ties to the lowest index, ascending output."""

import numpy as np

from oracle.topk import topk_select


def _brute(scores, nv, k):
    items = sorted(range(nv), key=lambda j: (-float(scores[j]), j))[:k]
    return sorted(items)


def test_against_python_sort_with_many_ties():
    rng = np.random.default_rng(0)
    for trial in range(200):
        n = int(rng.integers(1, 60))
        nv = int(rng.integers(0, n + 1))
        k = int(rng.integers(1, 70))
        s = rng.integers(-3, 4, n).astype(np.float32) * np.float32(0.5)
        idx, sc = topk_select(s, nv, k)
        want = _brute(s, nv, k)
        assert idx[: len(want)].tolist() == want
        assert np.all(idx[len(want):] == -1)
        assert np.array_equal(sc[: len(want)], s[want])
        assert np.all(np.isneginf(sc[len(want):]))


def test_special_cases():
    s = np.zeros(100, np.float32)
    assert topk_select(s, 100, 10)[0].tolist() == list(range(10))  # all ties -> first K
    s = np.arange(50, dtype=np.float32)[::-1].copy()
    idx, _ = topk_select(s, 50, 80)  # K >= visible -> every visible token
    assert idx[:50].tolist() == list(range(50)) and np.all(idx[50:] == -1)
    s = np.array([1, 5, 3, 5, 5], np.float32)
    assert topk_select(s, 5, 1)[0].tolist() == [1]  # K = 1 -> lowest-index argmax
    s = np.array([-0.0, 0.0, -0.0, 1.0], np.float32)
    assert topk_select(s, 4, 2)[0].tolist() == [0, 3]  # -0 ties +0
    assert topk_select(s, 0, 3)[0].tolist() == [-1, -1, -1]


def test_ids_map_positions_to_token_ids():
    s = np.array([2, 9, 9, 1], np.float32)
    ids = np.array([10, 20, 30, 40])
    idx, sc = topk_select(s, 4, 2, ids=ids)
    assert idx.tolist() == [20, 30] and sc.tolist() == [9, 9]
