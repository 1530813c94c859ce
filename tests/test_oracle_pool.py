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


def _brute_pool_topk(q, w, k_bytes, pool, plen, k, ctx):
    """Pure-Python restatement: score k_bytes[id] for every valid pool id with
    integer dots and the fixed-order float32 head sum, sort by (score desc,
    id asc), keep k, emit ascending ids."""
    dec = lambda b: torch.from_numpy(np.ascontiguousarray(b)).view(torch.float8_e4m3fn).double().numpy()
    qd = dec(q)
    cand = []
    for i in range(plen):
        t = int(pool[i])
        if t < 0 or t >= ctx:
            continue
        kd = dec(k_bytes[t])
        s = np.float32(0.0)
        for h in range(q.shape[0]):
            dot = sum(float(a) * float(b) for a, b in zip(qd[h], kd))
            s = np.float32(s + np.float32(np.float32(w[h]) * np.float32(max(dot, 0.0))))
        cand.append((float(s), t))
    cand.sort(key=lambda c: (-c[0], c[1]))
    take = sorted(cand[:k], key=lambda c: c[1])
    ids = [t for _, t in take] + [-1] * (k - len(take))
    scores = [s for s, _ in take] + [-np.inf] * (k - len(take))
    return np.array(ids, np.int32), np.array(scores, np.float32)


def test_pool_topk_sparse_pool_brute_force():
    """A sparse, non-contiguous pool (ids far from their positions), with -1
    and out-of-range ids inside pool_len: pool_topk must score k[pool_idx[i]]
    (not k[i]) and skip the invalid ids."""
    rng = np.random.default_rng(7)
    for trial in range(30):
        n, H, D = 300, 3, 16
        k_bytes = _e4m3(rng.integers(-4, 5, (n, D)))
        q = _e4m3(rng.integers(-4, 5, (H, D)))
        w = rng.standard_normal(H).astype(np.float32)
        if trial % 3 == 0:
            w = (rng.integers(-3, 4, H) / 4).astype(np.float32)   # many ties
        ctx = int(rng.integers(150, n + 1))
        ids = np.sort(rng.choice(n, int(rng.integers(5, 60)), replace=False))
        pool = np.full(80, -1, np.int32)
        pool[: len(ids)] = ids
        plen = len(ids)
        if trial % 2 == 1:   # invalid entries inside pool_len
            pool[1] = -1
            pool[plen] = n + 3
            plen += 1
        k = int(rng.integers(1, 40))
        got_i, got_s = P.pool_topk(q, w, k_bytes, pool, plen, k, ctx_len=ctx)
        want_i, want_s = _brute_pool_topk(q, w, k_bytes, pool, plen, k, ctx)
        assert np.array_equal(got_i, want_i), trial
        assert np.array_equal(got_s, want_s), trial


def test_pool_topk_mxfp4_against_flat_selection_and_a_loop():
    """The MXFP4 pool layer: a pool of all visible tokens gives the flat MXFP4
    Top-K; a sparse pool equals a loop scoring each pool id's own key row."""
    from oracle import quant as Q
    rng = np.random.default_rng(9)
    n, H, D = 200, 4, 128
    kc, ks = Q.mxfp4_quantize(rng.standard_normal((n, D)).astype(np.float32))
    q = _e4m3(rng.integers(-4, 5, (H, D)))
    w = rng.standard_normal(H).astype(np.float32)
    nv = 173
    flat, flat_s = topk_select(I.index_scores_mxfp4(q, w, kc, ks, nv), nv, 30)
    got, got_s = P.pool_topk_mxfp4(q, w, kc, ks, np.arange(n, dtype=np.int32), n, 30, ctx_len=nv)
    assert np.array_equal(got, flat) and np.array_equal(got_s, flat_s)
    ids = np.sort(rng.choice(n, 50, replace=False)).astype(np.int32)
    got, got_s = P.pool_topk_mxfp4(q, w, kc, ks, ids, len(ids), 12)
    cand = []
    for t in ids:
        sc = I.combine_heads(I.head_dots_mxfp4(q, kc[t:t + 1], ks[t:t + 1]), w)[0]
        cand.append((float(sc), int(t)))
    cand.sort(key=lambda c: (-c[0], c[1]))
    want = sorted(t for _, t in cand[:12])
    assert got.tolist() == want
