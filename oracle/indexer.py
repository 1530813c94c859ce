"""Lightning-style indexer scores (oracle; test infrastructure).

[map] "Checked in its code", row "Indexer-selected sparse attention": the
model carries a separate indexer (its own head count and head width) in the
lightning-indexer style of DeepSeek Sparse Attention; its scores over the
cached tokens decide which k entries reach attention.  [facts] token
selection gives 32 heads x 128 and top-512; the indexer K cache keeps one
key row per token that every indexer head reads.

The pages print no formula.  Reading: the published lightning-indexer form
    I(t, j) = sum_h  w[t, h] * ReLU( q[t, h, :] . k[j, :] )
with per-query, per-head float32 weights w.  To make the result a single
well-defined float32 value, the sum is evaluated in a fixed order:
    d_h = q_h . k_j            exact (float64 holds every E4M3 product and
                                the sum of up to 2^10 of them exactly)
    r_h = float32(max(d_h, 0))
    s   = +0.0f; for h = 0, 1, ..., H-1:  s = fl32(s + fl32(w_h * r_h))
with every float32 operation rounded to nearest even and no fused
multiply-add.  NumPy float32 array arithmetic performs exactly these
roundings.

Visibility: token j is visible to a query at position p of sequence b when
j < ctx_len[b] and (no positions given, or j <= p).  Invisible tokens get
score -inf here and are never selected.

Parity: pinned by brute-force pure-Python loops on tiny inputs, by an int64
recomputation of the dots, and by dyadic weights (k/64) that make every
partial sum exact so the result must equal the real-number sum
(tests/test_oracle_indexer.py).
"""

import numpy as np

from .formats import e4m3fn_decode


def head_dots(q_bytes, k_bytes):
    """Exact dots d[h, j] = q_h . k_j for E4M3 bytes q [H][D], k [N][D] -> float64 [H][N]."""
    q = e4m3fn_decode(np.asarray(q_bytes, dtype=np.uint8))
    k = e4m3fn_decode(np.asarray(k_bytes, dtype=np.uint8))
    return q @ k.T


def combine_heads(d, w):
    """Fixed-order float32 head sum of w_h * ReLU(d_h); d float64 [H][N], w float32 [H] -> float32 [N]."""
    w = np.asarray(w, dtype=np.float32)
    r = np.maximum(d, 0.0).astype(np.float32)
    s = np.zeros(d.shape[1], dtype=np.float32)
    for h in range(d.shape[0]):
        s = (s + (w[h] * r[h]).astype(np.float32)).astype(np.float32)
    return s


def index_scores(q_bytes, w, k_bytes, n_visible):
    """Scores of the first n_visible keys for one query row.

    q_bytes [H][D] u8 (E4M3), w [H] f32, k_bytes [N][D] u8 (E4M3).
    Returns float32 [N] with -inf at positions >= n_visible.
    """
    k_bytes = np.asarray(k_bytes)
    n = k_bytes.shape[0]
    nv = max(0, min(int(n_visible), n))
    s = np.full(n, -np.inf, dtype=np.float32)
    if nv > 0:
        s[:nv] = combine_heads(head_dots(q_bytes, k_bytes[:nv]), w)
    return s


def head_dots_mxfp4(q_bytes, k_codes, k_scales):
    """Dots d[h, j] = q_h . k_j with E4M3 queries and MXFP4 keys (E2M1 codes,
    E8M0 scale per 32 channels) -> float64 [H][N].  Every product is exact in
    float64 and each sum too while a key's shared exponents span fewer than
    about 25 binades."""
    from .quant import mxfp4_dequantize
    q = e4m3fn_decode(np.asarray(q_bytes, dtype=np.uint8))
    k = mxfp4_dequantize(k_codes, k_scales, q.shape[1])
    return q @ k.T


def index_scores_mxfp4(q_bytes, w, k_codes, k_scales, n_visible):
    """index_scores with the pages' MXFP4 indexer keys ([facts] indexer K
    groups: E2M1 with E8M0 scales per 32 channels, 68 bytes per entry): the
    same ReLU, weights and fixed-order float32 head sum over exact dots."""
    k_codes = np.asarray(k_codes)
    n = k_codes.shape[0]
    nv = max(0, min(int(n_visible), n))
    s = np.full(n, -np.inf, dtype=np.float32)
    if nv > 0:
        s[:nv] = combine_heads(head_dots_mxfp4(q_bytes, k_codes[:nv], np.asarray(k_scales)[:nv]), w)
    return s


def visible_count(ctx_len, q_pos=None):
    """Length of the visible prefix for a query: min(ctx_len, q_pos + 1)."""
    n = int(ctx_len)
    if q_pos is not None:
        n = min(n, int(q_pos) + 1)
    return max(n, 0)


def visible_entries(q_pos, m):
    """Cache entries a query at token position q_pos may see when each entry
    compresses m consecutive tokens (entry j covers tokens m*j .. m*j + m - 1).

    [facts] layer pattern and attn.kv_groups: the encoder's CSA2 layers keep
    one main-KV / indexer-K entry per m = 2 tokens, the decoder's one per
    token.  Reading (the pages give no rule for a partly filled entry): an
    entry is visible once every token it covers is at or before q_pos, so the
    count is floor((q_pos + 1) / m).
    """
    return max(0, (int(q_pos) + 1) // int(m))
