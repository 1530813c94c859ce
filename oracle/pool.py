"""Hierarchical Sparse Indexer candidate pool (oracle; test infrastructure).

[blog] CSA2 paragraph: the decoder's hierarchical indexer lets only the
first Full-mode layer score the whole context; it picks a candidate set, and
the indexers of deeper layers score that set alone, so their cost stays fixed
as the context grows; [facts] token
selection: the decoder's hierarchical indexer is limited to a candidate pool
of 2048 blocks x 8 positions; [map] technique tree, unfiled: blockwise
candidate-pool selection for sparse indexing; [atlas] OPD stage card: later
indexers score a pool an earlier one selected.

The pages give no block reduction.  Reading: a block's score is the MAX of
its visible tokens' scores (so a block size of 1 is token-level Top-K).
Blocks are [b*B, (b+1)*B) intersected with the visible prefix; the pool is
the top `nblocks` blocks by (block score desc, block index asc), expanded to
their visible tokens in ascending token order, padded with -1.

Later layers score only pool tokens and keep their Top-K with ties broken by
original token index (pool_topk).

Parity: pinned by brute force on tiny inputs, by "pool = all tokens gives the
flat Top-K", by block size 1 = token Top-K, by containment of the flat Top-K
in the pool when nblocks >= K, and, for pool_topk, by a pure-Python loop over
a sparse, unordered-in-score pool with invalid ids (tests/test_oracle_pool.py).
"""

import numpy as np

from .indexer import index_scores, combine_heads, head_dots
from .topk import topk_select


def block_scores(scores, n_visible, block):
    """Max score of each block of the visible prefix -> float32 [ceil(nv/block)]."""
    nv = max(0, min(int(n_visible), len(scores)))
    nb = (nv + block - 1) // block
    out = np.empty(nb, dtype=np.float32)
    for b in range(nb):
        out[b] = np.max(scores[b * block: min((b + 1) * block, nv)])
    return out


def hier_pool(scores, n_visible, block, nblocks):
    """Candidate pool of one query row.

    Returns (pool_idx int32 [nblocks*block] ascending, -1 padded; pool_len).
    """
    nv = max(0, min(int(n_visible), len(scores)))
    bs = block_scores(scores, nv, block)
    sel_blocks, _ = topk_select(bs, len(bs), nblocks)
    pool = []
    for b in sel_blocks:
        if b < 0:
            continue
        for j in range(b * block, min((b + 1) * block, nv)):
            pool.append(j)
    out = np.full(nblocks * block, -1, dtype=np.int32)
    out[: len(pool)] = pool
    return out, len(pool)


def pool_topk(q_bytes, w, k_bytes, pool_idx, pool_len, k, ctx_len=None):
    """Top-k over the pool tokens of one query row (later hierarchical layers).

    k_bytes: the full indexer key cache [N][D] of the sequence.  The first
    pool_len entries of pool_idx are the candidates (ascending token ids);
    an entry < 0 or >= ctx_len (default: the cache's row count) names no
    visible token and is skipped.
    Returns (idx int32 [k] ascending token ids, -1 padded; scores float32 [k]).
    """
    pl = max(0, min(int(pool_len), len(pool_idx)))
    n = np.asarray(k_bytes).shape[0] if ctx_len is None else int(ctx_len)
    ids = np.asarray(pool_idx[:pl], dtype=np.int64)
    ids = ids[(ids >= 0) & (ids < n)]
    if len(ids) == 0:
        return np.full(k, -1, np.int32), np.full(k, -np.inf, np.float32)
    s = combine_heads(head_dots(q_bytes, np.asarray(k_bytes)[ids]), w)
    return topk_select(s, len(ids), k, ids=ids)


def pool_topk_mxfp4(q_bytes, w, k_codes, k_scales, pool_idx, pool_len, k, ctx_len=None):
    """pool_topk over MXFP4 indexer keys (codes [N][D/2], E8M0 scales [N][D/32])."""
    from .indexer import head_dots_mxfp4
    pl = max(0, min(int(pool_len), len(pool_idx)))
    n = np.asarray(k_codes).shape[0] if ctx_len is None else int(ctx_len)
    ids = np.asarray(pool_idx[:pl], dtype=np.int64)
    ids = ids[(ids >= 0) & (ids < n)]
    if len(ids) == 0:
        return np.full(k, -1, np.int32), np.full(k, -np.inf, np.float32)
    s = combine_heads(head_dots_mxfp4(q_bytes, np.asarray(k_codes)[ids], np.asarray(k_scales)[ids]), w)
    return topk_select(s, len(ids), k, ids=ids)


__all__ = ["block_scores", "hier_pool", "pool_topk", "pool_topk_mxfp4", "index_scores"]
