"""Sparse MLA attention over the selected FP4 rows plus the FP8 window (oracle).

TEST INFRASTRUCTURE ONLY.

[map] "Checked in its code": multi-head latent attention with a single latent
KV head (num_key_value_heads = 1 is the MLA latent), partial RoPE on the last
64 of the 512 head dims, a learnable per-head sink logit added to the
sparse-MLA softmax denominator (initialised to -inf), and a 128-token sliding
window kept by every layer; [facts] one shared K=V entry per token, head dim
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

Parity: pinned by closed forms -- one entry returns exactly its V, q = 0
returns the mean of V, sink = -inf equals no sink, a huge sink drives o to 0,
K >= context equals dense softmax attention written independently, and the
result is invariant under permuting the Top-K list (tests/test_oracle_attention.py).
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
