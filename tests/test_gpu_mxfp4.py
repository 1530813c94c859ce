"""GPU parity of the pages' MXFP4 indexer keys (E2M1 codes + one E8M0 scale per
32 channels, 68 bytes per 128-channel entry): the cache writer bit for bit,
and scores / Top-K indices / pools bit for bit against the oracle on the
scaled FP4 matrix-core path (decode, multi-query, pool layers, prefill)."""

import numpy as np
import pytest
import torch

import fp4_kv_cache_index_amd as csa2
from fp4_kv_cache_index_amd import inputs
from oracle import indexer as I
from oracle import pool as P
from oracle import quant as Q
from oracle.topk import topk_select
from tests.gpu_util import announce, gpu, np_, require_gpu


def _mx_tie_rows():
    """Rows on every E2M1 threshold (and float32 neighbours) at shared exponents
    -20 .. 20, plus zero, subnormal, huge and single-spike groups."""
    ts = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 5.99, 6.5, 7.9]
    rows = []
    for X in range(-20, 21):
        s = 2.0 ** X
        for t in ts:
            x = np.float32(t * s)
            v = [np.float32(7.5 * s), x, np.nextafter(x, np.float32(np.inf)), np.nextafter(x, np.float32(0)),
                 -x, -np.nextafter(x, np.float32(np.inf)), np.float32(-0.0)]
            v += [np.float32(t * s * 0.5)] * (32 - len(v))
            rows.append(v)
    rows.append([0.0] * 32)
    rows.append([1e-40] * 16 + [-3e-39] * 16)
    rows.append([3e38, -3e38] + [1.0] * 30)
    rows.append([0.0] * 31 + [1e-30])
    x = np.array(rows, dtype=np.float32)
    pad = (-x.shape[0]) % 4
    x = np.concatenate([x, np.zeros((pad, 32), np.float32)])
    return x.reshape(-1, 128)


@gpu
def test_idx_mxfp4_quantize_bit_exact():
    require_gpu()
    announce("idx_mxfp4_quantize: ties at 41 exponents + random rows")
    x = torch.from_numpy(_mx_tie_rows()).cuda()
    c, s = csa2.idx_mxfp4_quantize(x)
    r = inputs.normal_f32((3000, 128), 91, 0, "k_idx", device="cuda") * 3.0
    c2, s2 = csa2.idx_mxfp4_quantize(r)
    torch.cuda.synchronize()
    for got_c, got_s, src in ((c, s, x), (c2, s2, r)):
        want_c, want_s = Q.mxfp4_quantize(np_(src))
        assert np.array_equal(np_(got_c), want_c)
        assert np.array_equal(np_(got_s), want_s)


def _mx_keys(B, N, seed, layout="soa"):
    """MXFP4 keys of float32 N(0, 1) rows: (codes view [B][N][64], scales view
    [B][N][4]) in separate arrays, or both inside padded 80-byte rows."""
    x = inputs.normal_f32((B, N, 128), seed, 0, "k_idx", device="cuda")
    if layout == "soa":
        return csa2.idx_mxfp4_quantize(x)
    rows = torch.zeros((B, N, 80), dtype=torch.uint8, device="cuda")
    csa2.idx_mxfp4_quantize(x, codes=rows[..., :64], scales=rows[..., 64:68])
    return rows[..., :64], rows[..., 64:68]


def _oracle_rows(q_idx, w, kc, ks, ctx, K, q_pos=None):
    B, Tq = q_idx.shape[:2]
    idx = np.zeros((B, Tq, K), np.int32)
    sc = np.zeros((B, Tq, K), np.float32)
    for b in range(B):
        for t in range(Tq):
            nv = I.visible_count(ctx[b], None if q_pos is None else q_pos[b, t])
            nv = min(nv, kc.shape[1])
            s = I.index_scores_mxfp4(q_idx[b, t], w[b, t], kc[b], ks[b], nv)
            idx[b, t], sc[b, t] = topk_select(s, nv, K)
    return idx, sc


def _run(q_idx, w, kc, ks, ctx, K, q_pos=None, stored=False):
    res = csa2.csa2_index_score_topk_mxfp4(q_idx, w, kc, ks, ctx, K, q_pos=q_pos, want_scores=True,
                                           stored_keys=stored)
    torch.cuda.synchronize()
    want_i, want_s = _oracle_rows(np_(q_idx), np_(w), np_(kc), np_(ks), np_(ctx), K,
                                  None if q_pos is None else np_(q_pos))
    assert np.array_equal(np_(res["topk_idx"]), want_i)
    assert np.array_equal(np_(res["topk_score"]), want_s)


@gpu
@pytest.mark.parametrize("N", [3 * 4096 + 577, 70001])
@pytest.mark.parametrize("H_I,K,layout", [(8, 2048, "soa"), (4, 300, "padded"), (16, 512, "soa"), (32, 512, "soa")])
def test_mxfp4_decode_scores_and_topk(H_I, K, layout, N):
    require_gpu()
    announce(f"mxfp4 decode H_I={H_I} K={K} {layout} N={N}")
    B = 3
    kc, ks = _mx_keys(B, N, 92, layout)
    q = inputs.int_e4m3((B, 1, H_I, 128), 92, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, 1, H_I), 92, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 33, N // 2 + 5], dtype=torch.int32, device="cuda")
    _run(q, w, kc, ks, ctx, K)


@gpu
@pytest.mark.parametrize("Tq", [2, 4, 5])
def test_mxfp4_multi_query_decode(Tq):
    require_gpu()
    announce(f"mxfp4 multi-query Tq={Tq}")
    B, N, H_I, K = 3, 20000, 8, 512
    kc, ks = _mx_keys(B, N, 93)
    q = inputs.int_e4m3((B, Tq, H_I, 128), 93, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 93, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 17, 9000], dtype=torch.int32, device="cuda")
    q_pos = (ctx[:, None].to(torch.int64) - Tq + torch.arange(Tq, device="cuda")[None, :]).to(torch.int32)
    _run(q, w, kc, ks, ctx, K, q_pos=q_pos.contiguous())


@gpu
def test_mxfp4_prefill_chunk():
    require_gpu()
    announce("mxfp4 prefill chunk Tq=40 on 30000 keys")
    B, N, Tq, H_I, K = 2, 30000, 40, 8, 600
    kc, ks = _mx_keys(B, N, 94)
    q = inputs.int_e4m3((B, Tq, H_I, 128), 94, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 94, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 1000], dtype=torch.int32, device="cuda")
    q_pos = (ctx[:, None].to(torch.int64) - Tq + torch.arange(Tq, device="cuda")[None, :] * 1).to(torch.int32)
    q_pos[0, :3] = torch.tensor([5, 700, 2047], dtype=torch.int32, device="cuda")
    _run(q, w, kc, ks, ctx, K, q_pos=q_pos.contiguous())
    _run(q, w, kc, ks, ctx, K, q_pos=q_pos.contiguous(), stored=True)


@gpu
@pytest.mark.parametrize("H_I", [13, 32])
def test_mxfp4_prefill_chunk_wide_heads(H_I):
    """MXFP4 prefill chunks with more than 8 indexer heads (the pages' 32 x
    128 shape; 13: padded head groups) on the query-major matrix-core
    product, with the selection passes and with stored keys."""
    require_gpu()
    announce(f"mxfp4 prefill chunk H_I={H_I} Tq=20 on 12000 keys")
    B, N, Tq, K = 1, 12000, 20, 512
    kc, ks = _mx_keys(B, N, 95)
    q = inputs.int_e4m3((B, Tq, H_I, 128), 95, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 95, 1, "w", device="cuda")
    ctx = torch.tensor([N], dtype=torch.int32, device="cuda")
    q_pos = (N - Tq + torch.arange(Tq, device="cuda")[None, :]).to(torch.int32).contiguous()
    q_pos[0, :2] = torch.tensor([3, 600], dtype=torch.int32, device="cuda")
    _run(q, w, kc, ks, ctx, K, q_pos=q_pos)
    _run(q, w, kc, ks, ctx, K, q_pos=q_pos, stored=True)


@gpu
@pytest.mark.parametrize("nblocks,K", [(64, 256), (2048, 2048), (4500, 512)])
def test_mxfp4_hierarchical_pool_and_pool_layers(nblocks, K):
    require_gpu()
    announce(f"mxfp4 pool nblocks={nblocks} K={K}")
    B, N, H_I, D_I = 2, 9 * 4096 + 3, 8, 128
    kc, ks = _mx_keys(B, N, 95)
    q0 = inputs.int_e4m3((B, 1, H_I, D_I), 95, 1, "q_idx", device="cuda")
    w0 = inputs.normal_f32((B, 1, H_I), 95, 1, "w", device="cuda")
    q1 = inputs.int_e4m3((B, 1, H_I, D_I), 95, 2, "q_idx", device="cuda")
    w1 = inputs.normal_f32((B, 1, H_I), 95, 2, "w", device="cuda")
    ctx = torch.tensor([N, N - 5], dtype=torch.int32, device="cuda")
    res = csa2.csa2_index_score_topk_mxfp4(q0, w0, kc, ks, ctx, K, pool_block=8, pool_nblocks=nblocks)
    later = csa2.csa2_hier_pool_topk_mxfp4(q1, w1, kc, ks, res["pool_idx"], res["pool_len"], K, ctx_len=ctx,
                                           want_scores=True)
    torch.cuda.synchronize()
    kch, ksh, ch = np_(kc), np_(ks), np_(ctx)
    for b in range(B):
        s0 = I.index_scores_mxfp4(np_(q0[b, 0]), np_(w0[b, 0]), kch[b], ksh[b], ch[b])
        pool, plen = P.hier_pool(s0, ch[b], 8, nblocks)
        assert int(np_(res["pool_len"])[b, 0]) == plen
        assert np.array_equal(np_(res["pool_idx"])[b, 0], pool)
        flat, _ = topk_select(s0, ch[b], K)
        assert np.array_equal(np_(res["topk_idx"])[b, 0], flat)
        want_i, want_s = P.pool_topk_mxfp4(np_(q1[b, 0]), np_(w1[b, 0]), kch[b], ksh[b], pool, plen, K,
                                           ctx_len=ch[b])
        assert np.array_equal(np_(later["topk_idx"])[b, 0], want_i)
        assert np.array_equal(np_(later["topk_score"])[b, 0], want_s)


@gpu
def test_mxfp4_decode64k_sampled_rows():
    """64 x 64K MXFP4 keys in the launch shape the benchmark times."""
    require_gpu()
    announce("mxfp4 decode 64 x 64K, sequences 0 and 63 sampled")
    B, N, H_I, K = 64, 65536, 8, 2048
    kc, ks = _mx_keys(B, N, 96)
    q = inputs.int_e4m3((B, 1, H_I, 128), 96, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, 1, H_I), 96, 1, "w", device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    res = csa2.csa2_index_score_topk_mxfp4(q, w, kc, ks, ctx, K, want_scores=True)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        s = I.index_scores_mxfp4(np_(q[b, 0]), np_(w[b, 0]), np_(kc[b]), np_(ks[b]), N)
        want_i, want_s = topk_select(s, N, K)
        assert np.array_equal(np_(res["topk_idx"][b, 0]), want_i)
        assert np.array_equal(np_(res["topk_score"][b, 0]), want_s)
