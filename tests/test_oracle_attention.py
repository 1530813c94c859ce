"""Pins for oracle.attention: closed forms and an independent dense softmax."""

import numpy as np
from scipy.special import logsumexp, softmax

from oracle import attention as A
from oracle import quant as Q


def _cache(rng, n, d):
    x = rng.standard_normal((n, d)).astype(np.float32)
    codes, scales = Q.fp4_quantize(x)
    return codes, scales, Q.fp4_dequantize(codes, scales, d)


def _swa(rng, w, d):
    x = rng.standard_normal((w, d)).astype(np.float32)
    v, s = Q.mxfp8_quantize(x)
    return v, s, Q.mxfp8_dequantize(v, s, d)


def test_topk_covering_context_equals_dense_attention():
    rng = np.random.default_rng(0)
    n, d, dv, H, W = 300, 576, 512, 16, 20
    codes, scales, kv = _cache(rng, n, d)
    sv, ss, sw = _swa(rng, W, d)
    q = rng.standard_normal((H, d)).astype(np.float32)
    idx = np.concatenate([rng.permutation(n), [-1, -1, n + 5]])  # K >= N (with padding/out of range)
    scale = 1 / np.sqrt(576)
    out, lse = A.sparse_attn_decode_row(q, codes, scales, idx, n, sv, ss, 17, d, dv, scale)
    keys = np.concatenate([kv, sw[:17]])  # independent dense formulation
    z = scale * (q.astype(np.float64) @ keys.T)
    want = softmax(z, axis=1) @ keys[:, :dv]
    assert np.allclose(out, want, rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, logsumexp(z, axis=1), rtol=1e-13)


def test_closed_forms():
    rng = np.random.default_rng(1)
    n, d, dv, H = 64, 512, 512, 4
    codes, scales, kv = _cache(rng, n, d)
    q = rng.standard_normal((H, d)).astype(np.float32)
    # one entry -> exactly its V, lse = its logit
    out, lse = A.sparse_attn_decode_row(q, codes, scales, [7, -1], n, None, None, 0, d, dv, 0.1)
    assert np.array_equal(out, np.broadcast_to(kv[7, :dv], (H, dv)))
    assert np.allclose(lse, 0.1 * (q.astype(np.float64) @ kv[7]))
    # q = 0 -> mean of V, lse = ln(count)
    idx = np.arange(0, 40)
    out, lse = A.sparse_attn_decode_row(np.zeros((H, d), np.float32), codes, scales, idx, n, None, None, 0, d, dv, 0.1)
    assert np.allclose(out, kv[:40, :dv].mean(0)[None], rtol=1e-12, atol=1e-15)
    assert np.allclose(lse, np.log(40.0))
    # sink = -inf is no sink; a huge sink drives o to 0 and lse to the sink
    o1, l1 = A.sparse_attn_decode_row(q, codes, scales, idx, n, None, None, 0, d, dv, 0.1)
    o2, l2 = A.sparse_attn_decode_row(q, codes, scales, idx, n, None, None, 0, d, dv, 0.1, sink=np.full(H, -np.inf))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = A.sparse_attn_decode_row(q, codes, scales, idx, n, None, None, 0, d, dv, 0.1, sink=np.full(H, 1e3))
    assert np.max(np.abs(o3)) < 1e-300 and np.allclose(l3, 1e3)
    # a finite sink adds exp(sink) to the denominator
    o4, l4 = A.sparse_attn_decode_row(q, codes, scales, idx, n, None, None, 0, d, dv, 0.1, sink=np.full(H, 0.5))
    z = 0.1 * (q.astype(np.float64) @ kv[:40].T)
    den = np.exp(z).sum(1) + np.exp(0.5)
    assert np.allclose(o4, (np.exp(z) @ kv[:40, :dv]) / den[:, None], rtol=1e-12)
    assert np.allclose(l4, np.log(den), rtol=1e-13)
    # no entries and no sink -> zeros, -inf
    o5, l5 = A.sparse_attn_decode_row(q, codes, scales, [-1, -1], n, None, None, 0, d, dv, 0.1)
    assert np.all(o5 == 0) and np.all(np.isneginf(l5))


def test_permutation_invariance_and_reuse():
    rng = np.random.default_rng(2)
    n, d, dv, H = 200, 576, 512, 8
    codes, scales, _ = _cache(rng, n, d)
    sv, ss, _ = _swa(rng, 128, d)
    q = rng.standard_normal((H, d)).astype(np.float32)
    idx = rng.choice(n, 50, replace=False)
    o1, l1 = A.sparse_attn_decode_row(q, codes, scales, np.sort(idx), n, sv, ss, 128, d, dv, 0.05)
    o2, l2 = A.sparse_attn_decode_row(q, codes, scales, idx, n, sv, ss, 128, d, dv, 0.05)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-15) and np.allclose(l1, l2, rtol=1e-13)


def test_prefill_window_rows():
    # window array row i holds position 90 + i; window 8
    assert A.prefill_window_rows(100, 90, 30, 8).tolist() == list(range(3, 11))
    assert A.prefill_window_rows(92, 90, 30, 8).tolist() == [0, 1, 2]
    assert A.prefill_window_rows(89, 90, 30, 8).tolist() == []
    assert A.prefill_window_rows(150, 90, 30, 8).tolist() == []  # array ends at 119


def test_prefill_row_equals_dense_softmax_over_hand_built_entries():
    """sparse_attn_prefill_row against an independent dense softmax whose entry
    list is written out here: the Top-K rows with 0 <= id < ctx_len, then the
    window rows of positions max(p - W + 1, swa_pos0) .. p that the window
    array holds (row i = position swa_pos0 + i), clipped at both ends."""
    rng = np.random.default_rng(11)
    n, d, dv, H, W = 400, 576, 512, 8, 16
    codes, scales, kv = _cache(rng, n, d)
    swa_pos0, n_rows = 300, 40            # window array covers positions 300 .. 339
    sv, ss, sw = _swa(rng, n_rows, d)
    scale = 0.07
    cases = [(320, 350), (305, 330), (302, 310), (339, 400), (350, 400), (299, 299), (315, 316)]
    for p, ctx in cases:
        q = rng.standard_normal((H, d)).astype(np.float32)
        idx = np.concatenate([rng.choice(n, 30, replace=False), [-1, n + 2, ctx, ctx - 1]])
        out, lse = A.sparse_attn_prefill_row(q, codes, scales, idx, ctx, p, sv, ss, swa_pos0, W, d, dv, scale)
        entries = [kv[i] for i in idx if 0 <= i < ctx]
        for pos in range(p - W + 1, p + 1):
            if pos >= swa_pos0 and pos - swa_pos0 < n_rows:
                entries.append(sw[pos - swa_pos0])
        keys = np.array(entries)
        z = scale * (q.astype(np.float64) @ keys.T)
        want = softmax(z, axis=1) @ keys[:, :dv]
        assert np.allclose(out, want, rtol=1e-12, atol=1e-14), (p, ctx)
        assert np.allclose(lse, logsumexp(z, axis=1), rtol=1e-13), (p, ctx)


def test_paged_ring_row_equals_the_linear_layout():
    """The same rows scattered into a page pool by a random block table (with
    unused and missing pages) and the window into a ring: the paged row must
    equal the linear row built from the original arrays (decode: the last
    W positions; multi-query: each query's causal window)."""
    rng = np.random.default_rng(21)
    n, d, dv, H, W, P = 333, 576, 512, 8, 16, 16
    codes, scales, _ = _cache(rng, n, d)
    n_pages = 40
    npg = (n + P - 1) // P
    pages = rng.permutation(n_pages)[:npg]            # logical page -> pool page
    pool_c = np.zeros((n_pages * P, codes.shape[1]), np.uint8)
    pool_s = np.zeros((n_pages * P, scales.shape[1]), np.uint8)
    for j in range(n):
        r = pages[j // P] * P + j % P
        pool_c[r], pool_s[r] = codes[j], scales[j]
    bt = np.full(npg + 3, -1, np.int64)
    bt[:npg] = pages
    R = 24                                            # ring of 24 rows, positions up to 339 written
    swa_end = 340
    sv_lin, ss_lin, _ = _swa(rng, swa_end, d)         # linear window array: row i = position i
    ring_v = np.zeros((R, sv_lin.shape[1]), np.uint8)
    ring_s = np.zeros((R, ss_lin.shape[1]), np.uint8)
    for x in range(swa_end - R, swa_end):
        ring_v[x % R], ring_s[x % R] = sv_lin[x], ss_lin[x]
    scale = 0.05
    for p in (339, 336, 330):
        q = rng.standard_normal((H, d)).astype(np.float32)
        idx = np.concatenate([rng.choice(n, 40, replace=False), [-1, n + 4]])
        o1, l1 = A.sparse_attn_paged_row(q, pool_c, pool_s, bt, P, n_pages, idx, n, p, ring_v, ring_s, R,
                                         swa_end, W, d, dv, scale)
        # the ring holds positions swa_end - R .. swa_end - 1 (330's window
        # starts at 315, which the ring has already overwritten)
        o2, l2 = A.sparse_attn_prefill_row(q, codes, scales, idx, n, p, sv_lin[swa_end - R:], ss_lin[swa_end - R:],
                                           swa_end - R, W, d, dv, scale)
        assert np.array_equal(o1, o2) and np.array_equal(l1, l2), p
    # a missing page entry drops exactly the tokens of that page
    bt2 = bt.copy()
    bt2[3] = -1
    q = rng.standard_normal((H, d)).astype(np.float32)
    idx = np.arange(40, 80)
    o1, l1 = A.sparse_attn_paged_row(q, pool_c, pool_s, bt2, P, n_pages, idx, n, 339, None, None, R, swa_end, W,
                                     d, dv, scale)
    keep = idx[(idx // P) != 3]
    o2, l2 = A.sparse_attn_decode_row(q, codes, scales, keep, n, None, None, 0, d, dv, scale)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # hand example of the addressing
    assert A.paged_row([5, 2, 7], 4, 9) == 7 * 4 + 1      # token 9: slot 2, offset 1
    assert A.paged_row([5, 2, 7], 4, 5) == 2 * 4 + 1      # token 5: slot 1, offset 1
    assert A.paged_row([5, -1], 4, 5) == -1 and A.paged_row([5], 4, 4) == -1
    assert A.ring_window_rows(10, 4, 11, 6).tolist() == [7 % 6, 8 % 6, 9 % 6, 10 % 6]
    assert A.ring_window_rows(10, 8, 11, 6).tolist() == [5, 0, 1, 2, 3, 4]   # ring keeps 5..10 only


def test_rope_rotation_and_the_inverse_rotation_epilogue():
    """Pins of the RoPE handling: the pair rotation is orthogonal and its
    inverse undoes it (closed form for theta = pi/2); zero angles leave plain
    attention; and with a single entry whose rotary channels were rotated by
    the query's own angles (a key at the query's position), the epilogue
    returns that entry's un-rotated channels exactly as V."""
    rng = np.random.default_rng(31)
    cs = np.stack([np.cos(t := rng.uniform(-3, 3, 32)), np.sin(t)], axis=1)
    x = rng.standard_normal((5, 64))
    y = A.rotate_pairs(x, cs, +1)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(x, axis=1), rtol=1e-14)
    assert np.allclose(A.rotate_pairs(y, cs, -1), x, rtol=1e-13, atol=1e-14)
    quarter = np.tile([[0.0, 1.0]], (32, 1))                  # theta = pi/2: (a, b) -> (-b, a)
    z = A.rotate_pairs(x, quarter, +1)
    assert np.array_equal(z[:, 0::2], -x[:, 1::2]) and np.array_equal(z[:, 1::2], x[:, 0::2])
    d, n, H = 512, 100, 4
    codes, scales, kv = _cache(rng, n, d)
    q = rng.standard_normal((H, d)).astype(np.float32)
    ident = np.tile([[1.0, 0.0]], (32, 1))
    o1, l1 = A.sparse_attn_decode_rope_row(q, codes, scales, np.arange(30), n, None, None, 0, d, 0.05, ident, 64,
                                           True)
    o2, l2 = A.sparse_attn_decode_row(q, codes, scales, np.arange(30), n, None, None, 0, d, d, 0.05)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # single entry: V's rotary part comes back un-rotated once the row was
    # rotated by the query's angles (rows are built exactly representable)
    raw = Q.fp4_dequantize(codes[7:8], scales[7:8], d)[0]
    o3, _ = A.sparse_attn_decode_rope_row(q, codes, scales, [7], n, None, None, 0, d, 0.05, cs, 64, False)
    assert np.allclose(A.rotate_pairs(o3[:, 448:], cs, +1), np.broadcast_to(raw[448:], (H, 64)), rtol=1e-12,
                       atol=1e-13)
