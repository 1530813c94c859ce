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
