"""Pins for oracle.pool: hierarchical candidate pool and pool-restricted Top-K."""

import numpy as np
import torch

from oracle import indexer as I
from oracle import pool as P
from oracle.topk import topk_select


def _e4m3(v):
    return torch.tensor(np.asarray(v, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _brute_pool(scores, nv, block, nblocks):
    blocks = []
    for b in range((nv + block - 1) // block):
        toks = list(range(b * block, min((b + 1) * block, nv)))
        blocks.append((max(float(scores[j]) for j in toks), b, toks))
    blocks.sort(key=lambda t: (-t[0], t[1]))
    chosen = sorted(blocks[:nblocks], key=lambda t: t[1])
    return [j for _, _, toks in chosen for j in toks]


def test_pool_brute_force_tiny():
    rng = np.random.default_rng(0)
    for _ in range(100):
        n = int(rng.integers(1, 80))
        nv = int(rng.integers(0, n + 1))
        block = int(rng.choice([1, 2, 4, 8]))
        nb = int(rng.integers(1, 12))
        s = rng.integers(-2, 3, n).astype(np.float32)
        pool, plen = P.hier_pool(s, nv, block, nb)
        want = _brute_pool(s, nv, block, nb)
        assert plen == len(want) and pool[:plen].tolist() == want
        assert np.all(pool[plen:] == -1) and len(pool) == nb * block


def test_block_one_is_token_topk():
    rng = np.random.default_rng(1)
    s = rng.integers(-3, 4, 500).astype(np.float32)
    pool, plen = P.hier_pool(s, 480, 1, 64)
    idx, _ = topk_select(s, 480, 64)
    assert plen == 64 and np.array_equal(pool, idx)


def test_pool_of_all_tokens_equals_flat_topk():
    rng = np.random.default_rng(2)
    q = _e4m3(rng.integers(-4, 5, (8, 128)))
    k = _e4m3(rng.integers(-4, 5, (1000, 128)))
    w = rng.standard_normal(8).astype(np.float32)
    n = 997
    s = I.index_scores(q, w, k, n)
    pool, plen = P.hier_pool(s, n, 8, 125)  # 125 blocks x 8 cover all 997 tokens
    assert plen == n and pool[:n].tolist() == list(range(n))
    flat, flat_s = topk_select(s, n, 64)
    pk, pk_s = P.pool_topk(q, w, k, pool, plen, 64)
    assert np.array_equal(flat, pk) and np.array_equal(flat_s, pk_s)


def test_flat_topk_is_contained_in_pool():
    rng = np.random.default_rng(3)
    for trial in range(40):
        n = int(rng.integers(50, 400))
        s = rng.integers(-2, 3, n).astype(np.float32)  # heavy ties
        kk = int(rng.integers(1, 20))
        nb = kk + int(rng.integers(0, 5))
        pool, plen = P.hier_pool(s, n, 8, nb)
        flat, _ = topk_select(s, n, kk)
        assert set(flat[flat >= 0].tolist()) <= set(pool[:plen].tolist())
