"""Pins for oracle.indexer: exact dots, fixed-order float32 head sum, visibility."""

import os
from fractions import Fraction

import numpy as np
import torch

from oracle import indexer as I

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ints_to_e4m3(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_head_dots_equal_int64_dots():
    rng = np.random.default_rng(0)
    qi = rng.integers(-4, 5, (8, 128))
    ki = rng.integers(-4, 5, (700, 128))
    d = I.head_dots(_ints_to_e4m3(qi), _ints_to_e4m3(ki))
    want = qi.astype(np.int64) @ ki.astype(np.int64).T
    assert np.array_equal(d, want.astype(np.float64))


def test_head_dots_exact_for_general_e4m3():
    # Arbitrary finite E4M3 values: float64 must hold the exact rational dot.
    rng = np.random.default_rng(1)
    codes = rng.integers(0, 256, (3, 32))
    codes[(codes & 0x7F) == 0x7F] = 0x38
    kc = rng.integers(0, 256, (5, 32))
    kc[(kc & 0x7F) == 0x7F] = 0x38
    d = I.head_dots(codes.astype(np.uint8), kc.astype(np.uint8))
    qv = torch.tensor(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    kv = torch.tensor(kc.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    for h in range(3):
        for j in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(qv[h], kv[j]))
            assert Fraction(d[h, j]) == exact


def test_head_sum_order_golden():
    for line in open(os.path.join(GOLDEN, "indexer_order.txt")):
        if not line.strip() or line.startswith("#"):
            continue
        w, d, want = [p.split() for p in line.split(";")]
        w = np.array([float(x) for x in w], dtype=np.float32)
        d = np.array([[float(x)] for x in d], dtype=np.float64)
        got = I.combine_heads(d, w)
        assert got.dtype == np.float32
        assert got[0] == np.float32(float(want[0])), (line, got)


def test_dyadic_weights_give_the_exact_real_sum():
    rng = np.random.default_rng(2)
    qi = rng.integers(-4, 5, (8, 128))
    ki = rng.integers(-4, 5, (300, 128))
    w = (rng.integers(-64, 65, 8) / 64.0).astype(np.float32)
    s = I.index_scores(_ints_to_e4m3(qi), w, _ints_to_e4m3(ki), 300)
    for j in range(300):
        exact = sum(Fraction(float(w[h])) * max(int(qi[h] @ ki[j]), 0) for h in range(8))
        assert Fraction(float(s[j])) == exact


def test_visibility_prefix():
    rng = np.random.default_rng(3)
    q = _ints_to_e4m3(rng.integers(-4, 5, (4, 64)))
    k = _ints_to_e4m3(rng.integers(-4, 5, (50, 64)))
    w = rng.standard_normal(4).astype(np.float32)
    s = I.index_scores(q, w, k, 37)
    assert np.all(np.isneginf(s[37:])) and np.all(np.isfinite(s[:37]))
    full = I.index_scores(q, w, k, 50)
    assert np.array_equal(s[:37], full[:37])
    assert I.visible_count(100, None) == 100
    assert I.visible_count(100, 41) == 42
    assert I.visible_count(30, 41) == 30


def test_visible_entries_of_compressed_caches():
    """m = 1 is the token count; for m = 2 a brute-force count of entries whose
    two tokens are all at or before the query."""
    for p in range(0, 50):
        assert I.visible_entries(p, 1) == p + 1
        for m in (2, 3, 4):
            brute = sum(1 for j in range(100) if all(t <= p for t in range(m * j, m * j + m)))
            assert I.visible_entries(p, m) == brute
    assert I.visible_entries(131071, 2) == 65536 and I.visible_entries(131070, 2) == 65535
    assert I.visible_entries(-1, 2) == 0


def test_mxfp4_key_dots_and_scores_against_exact_rationals():
    """Dots with MXFP4 keys against a pure-Python Fraction computation of
    sum_c q_c * e2m1(code_c) * 2^(scale_{c/32} - 127), and the scores' fixed-
    order float32 head sum over them."""
    from fractions import Fraction
    rng = np.random.default_rng(5)
    H, D, N = 3, 128, 40
    qv = rng.integers(-4, 5, (H, D))
    q = _ints_to_e4m3(qv)
    codes = rng.integers(0, 256, (N, D // 2)).astype(np.uint8)
    scales = rng.integers(120, 135, (N, D // 32)).astype(np.uint8)
    mags = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    w = rng.standard_normal(H).astype(np.float32)
    d = I.head_dots_mxfp4(q, codes, scales)
    s = I.index_scores_mxfp4(q, w, codes, scales, N - 3)
    for j in range(N):
        exact = []
        for h in range(H):
            acc = Fraction(0)
            for c in range(D):
                nib = (int(codes[j, c // 2]) >> (4 * (c % 2))) & 0xF
                val = mags[nib & 7] * (-1 if nib & 8 else 1) * Fraction(2) ** (int(scales[j, c // 32]) - 127)
                acc += int(qv[h, c]) * val
            exact.append(acc)
            assert d[h, j] == float(acc)
        if j < N - 3:
            ref = np.float32(0)
            for h in range(H):
                ref = np.float32(ref + np.float32(w[h] * np.float32(max(float(exact[h]), 0.0))))
            assert s[j] == ref
        else:
            assert s[j] == -np.inf
