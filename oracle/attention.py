"""Sparse MLA attention over the selected FP4 rows plus the FP8 window (oracle).

TEST INFRASTRUCTURE ONLY.

[map] "Checked in its code": multi-head latent attention whose single KV
head is the MLA latent, rotary position on the last 64 of the 512 head
channels only, one trainable logit per head that enters only the normaliser
of the softmax (its initial value is -inf), and a window of the last 128
tokens in every layer; [facts] one shared K=V entry per token, head dim
512 = nope + rope, the window cache of every layer; [blog] CSA2 paragraph:
attention runs over the Top-K entries chosen by the indexer.

Per query row and head h, with entry set E = {valid Top-K rows} U {valid
window rows}:
    k_e = dequantised row (all d_qk channels), v_e = its first d_v channels
    z_e = scale * (q_h . k_e)                       (float64)
    m   = max(z U {sink_h})
    den = sum_e exp(z_e - m) + [sink] exp(sink_h - m)
    o_h = sum_e exp(z_e - m) v_e / den,   lse_h = m + ln(den)
An empty E with no sink gives o = 0, lse = -inf.  A Top-K index < 0 or
>= ctx_len is skipped.  A main row and a window row of the same position are
two entries (different caches).

Readings: d_qk = 576 / d_v = 512 follow the measured workloads' "512 + 64"
latent; the pages' own 512-wide K=V row is the d_qk = d_v = 512 variant.
The inverse RoPE of the output is not part of this step.

Paged cache and ring window (a serving layout of the same caches, [map]
technique tree, KV cache management; [facts] every layer's own 128-token
window): a sequence's token j lives in pool row block_table[j // P] * P +
j % P; window position x lives in ring row x % R, and the ring holds the R
most recent positions.  Reading: the entries and the arithmetic are those of
the linear layout; only the addressing differs.

Parity: pinned by closed forms -- one entry returns exactly its V, q = 0
returns the mean of V, sink = -inf equals no sink, a huge sink drives o to 0,
K >= context equals dense softmax attention written independently, and the
result is invariant under permuting the Top-K list; the paged/ring row equals
the linear-layout row on caches scattered by a test-written block table and
ring placement (tests/test_oracle_attention.py).
"""

import numpy as np

from .quant import fp4_dequantize, mxfp8_dequantize


def attend(q, keys, d_v, scale, sink=None):
    """Softmax attention of q [H][d_qk] over key rows [E][d_qk] (V = keys[:, :d_v]).

    Returns (out float64 [H][d_v], lse float64 [H]).
    """
    q = np.asarray(q, dtype=np.float64)
    keys = np.asarray(keys, dtype=np.float64)
    H = q.shape[0]
    out = np.zeros((H, d_v), dtype=np.float64)
    lse = np.full(H, -np.inf, dtype=np.float64)
    for h in range(H):
        z = scale * (keys @ q[h]) if keys.shape[0] else np.zeros(0)
        terms = list(z)
        s_h = None if sink is None else float(sink[h])
        if s_h is not None and not np.isneginf(s_h):
            terms.append(s_h)
        if len(terms) == 0:
            continue
        m = max(terms)
        p = np.exp(z - m)
        den = p.sum()
        if s_h is not None and not np.isneginf(s_h):
            den += np.exp(s_h - m)
        if keys.shape[0]:
            out[h] = (p[:, None] * keys[:, :d_v]).sum(axis=0) / den
        lse[h] = m + np.log(den)
    return out, lse


def gather_entries(kv_codes, kv_scales, idx, ctx_len, swa_vals, swa_scales, swa_len, d_qk):
    """Dequantised entry rows for one query: valid Top-K rows, then valid window rows."""
    idx = np.asarray(idx, dtype=np.int64)
    ok = (idx >= 0) & (idx < int(ctx_len))
    sel = idx[ok]
    rows = [fp4_dequantize(kv_codes[sel], kv_scales[sel], d_qk)] if len(sel) else []
    n_swa = max(0, int(swa_len))
    if swa_vals is not None and n_swa > 0:
        rows.append(mxfp8_dequantize(swa_vals[:n_swa], swa_scales[:n_swa], d_qk))
    if not rows:
        return np.zeros((0, d_qk))
    return np.concatenate(rows, axis=0)


def sparse_attn_decode_row(q, kv_codes, kv_scales, idx, ctx_len, swa_vals, swa_scales, swa_len,
                           d_qk, d_v, scale, sink=None):
    """One decode query row: q [H][d_qk]; caches of its sequence; returns (out, lse)."""
    keys = gather_entries(kv_codes, kv_scales, idx, ctx_len, swa_vals, swa_scales, swa_len, d_qk)
    return attend(q, keys, d_v, scale, sink)


def prefill_window_rows(q_pos, swa_pos0, n_swa_rows, window):
    """Window rows (indices into the per-sequence window array) seen by a query at q_pos.

    The window array's row i holds position swa_pos0 + i; a query at position p
    sees positions max(p - window + 1, swa_pos0) .. p that the array holds.
    """
    lo = max(int(q_pos) - window + 1, int(swa_pos0))
    hi = min(int(q_pos), int(swa_pos0) + int(n_swa_rows) - 1)
    if hi < lo:
        return np.zeros(0, dtype=np.int64)
    return np.arange(lo - int(swa_pos0), hi - int(swa_pos0) + 1, dtype=np.int64)


def sparse_attn_prefill_row(q, kv_codes, kv_scales, idx, ctx_len, q_pos, swa_vals, swa_scales,
                            swa_pos0, window, d_qk, d_v, scale, sink=None):
    """One prefill query at position q_pos: Top-K rows (< ctx_len) + its causal window."""
    idx = np.asarray(idx, dtype=np.int64)
    ok = (idx >= 0) & (idx < int(ctx_len))
    sel = idx[ok]
    rows = [fp4_dequantize(kv_codes[sel], kv_scales[sel], d_qk)] if len(sel) else []
    wr = prefill_window_rows(q_pos, swa_pos0, swa_vals.shape[0], window)
    if len(wr):
        rows.append(mxfp8_dequantize(swa_vals[wr], swa_scales[wr], d_qk))
    keys = np.concatenate(rows, axis=0) if rows else np.zeros((0, d_qk))
    return attend(q, keys, d_v, scale, sink)


def paged_row(block_table, page_size, token):
    """Pool row of a sequence's token in a paged cache: the page named by the
    sequence's block-table entry token // page_size, at offset token % page_size.
    Returns -1 when the block table has no entry there or it is negative."""
    slot = int(token) // int(page_size)
    if slot < 0 or slot >= len(block_table) or int(block_table[slot]) < 0:
        return -1
    return int(block_table[slot]) * int(page_size) + int(token) % int(page_size)


def ring_window_rows(q_pos, window, swa_end, ring):
    """Ring rows of the window positions a query at q_pos sees: positions
    max(q_pos - window + 1, swa_end - ring, 0) .. min(q_pos, swa_end - 1), the
    ring holding position x at row x % ring (and positions swa_end - ring ..
    swa_end - 1 only)."""
    lo = max(int(q_pos) - int(window) + 1, int(swa_end) - int(ring), 0)
    hi = min(int(q_pos), int(swa_end) - 1)
    return np.array([x % int(ring) for x in range(lo, hi + 1)], dtype=np.int64)


def sparse_attn_paged_row(q, pool_codes, pool_scales, block_table, page_size, n_pages, idx, ctx_len, q_pos,
                          ring_vals, ring_scales, ring, swa_end, window, d_qk, d_v, scale, sink=None):
    """One query of a paged main cache with a ring window.

    pool_codes / pool_scales: the page pool's rows [n_pages * page_size][...];
    block_table: the sequence's page numbers; idx: logical token ids (Top-K),
    skipped when < 0, >= ctx_len, or when their page entry is missing or not
    a page of the pool; ring_vals / ring_scales: the sequence's ring [ring][...].
    """
    rows = []
    for t in np.asarray(idx, dtype=np.int64):
        if t < 0 or t >= int(ctx_len):
            continue
        r = paged_row(block_table, page_size, t)
        if r < 0 or r >= int(n_pages) * int(page_size):
            continue
        rows.append(r)
    keys = []
    if rows:
        rows = np.array(rows, dtype=np.int64)
        keys.append(fp4_dequantize(pool_codes[rows], pool_scales[rows], d_qk))
    wr = ring_window_rows(q_pos, window, swa_end, ring) if ring_vals is not None else np.zeros(0, np.int64)
    if len(wr):
        keys.append(mxfp8_dequantize(ring_vals[wr], ring_scales[wr], d_qk))
    keys = np.concatenate(keys, axis=0) if keys else np.zeros((0, d_qk))
    return attend(q, keys, d_v, scale, sink)


def rotate_pairs(x, cs, sign):
    """Rotate the channel pairs (2i, 2i+1) of x [..., 2n] by sign * theta_i,
    where cs [n][2] holds (cos theta_i, sin theta_i): (a, b) ->
    (a cos - sign b sin, sign a sin + b cos)."""
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(cs, dtype=np.float64)[:, 0]
    s = sign * np.asarray(cs, dtype=np.float64)[:, 1]
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = a * s + b * c
    return out


def sparse_attn_decode_rope_row(q, kv_codes, kv_scales, idx, ctx_len, swa_vals, swa_scales, swa_len, d, scale,
                                rope_cs, rope_dim, rotate_q, sink=None):
    """Decode attention over the pages' 512-wide K = V row with the rotary part
    handled around it ([facts] attention: partial RoPE on the last 64 dims of
    Q and KV, inverse rotation on the attention output; [map] inference
    kernel: fused RoPE-attention-RoPE-cast).

    The last rope_dim channels of q are rotated forward by the query
    position's angles when rotate_q (else q arrives rotated), attention runs
    as sparse_attn_decode_row with d_qk = d_v = d, and the last rope_dim
    channels of the output are rotated back by the same angles.  rope_cs
    [rope_dim/2][2] holds (cos, sin) of the query position; channel pairs are
    adjacent (2i, 2i+1) -- a reading, the pages give no pair convention.
    """
    q = np.asarray(q, dtype=np.float64).copy()
    r0 = d - rope_dim
    if rotate_q:
        q[:, r0:] = rotate_pairs(q[:, r0:], rope_cs, +1)
    out, lse = sparse_attn_decode_row(q, kv_codes, kv_scales, idx, ctx_len, swa_vals, swa_scales, swa_len, d, d,
                                      scale, sink)
    out = out.copy()
    out[:, r0:] = rotate_pairs(out[:, r0:], rope_cs, -1)
    return out, lse
