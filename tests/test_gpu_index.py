"""GPU parity of indexer scoring + Top-K + hierarchical pool: bit-exact indices."""

import numpy as np
import pytest
import torch

import fp4_kv_cache_index_amd as csa2
from fp4_kv_cache_index_amd import inputs
from oracle import indexer as I
from oracle import pool as P
from oracle.topk import topk_select
from tests.gpu_util import announce, gpu, np_, require_gpu


def _oracle_rows(q_idx, w, k_idx, ctx_len, k_top, q_pos=None):
    """Oracle Top-K of every (b, t) row."""
    B, Tq = q_idx.shape[:2]
    idx = np.zeros((B, Tq, k_top), np.int32)
    sc = np.zeros((B, Tq, k_top), np.float32)
    for b in range(B):
        for t in range(Tq):
            nv = I.visible_count(ctx_len[b], None if q_pos is None else q_pos[b, t])
            nv = min(nv, k_idx.shape[1])
            s = I.index_scores(q_idx[b, t], w[b, t], k_idx[b], nv)
            idx[b, t], sc[b, t] = topk_select(s, nv, k_top)
    return idx, sc


def _run_and_check(q_idx, w, k_idx, ctx_len, k_top, q_pos=None):
    res = csa2.csa2_index_score_topk(q_idx, w, k_idx, ctx_len, k_top, q_pos=q_pos, want_scores=True)
    torch.cuda.synchronize()
    want_i, want_s = _oracle_rows(np_(q_idx), np_(w), np_(k_idx), np_(ctx_len), k_top,
                                  None if q_pos is None else np_(q_pos))
    got_i, got_s = np_(res["topk_idx"]), np_(res["topk_score"])
    assert np.array_equal(got_i, want_i)
    assert np.array_equal(got_s, want_s)
    return res


@gpu
def test_tiny_config_full_layer_topk():
    require_gpu()
    wl = inputs.WORKLOADS["tiny"]
    announce("index_score_topk tiny B1 N4096 4x64 K256")
    k_idx = inputs.shared_cache_inputs(wl, device="cuda")["k_idx"]
    lay = inputs.decode_layer_inputs(wl, 0, device="cuda")
    ctx = torch.full((wl.B,), wl.N, dtype=torch.int32, device="cuda")
    _run_and_check(lay["q_idx"], lay["w"], k_idx, ctx, wl.K)


# Rows of at most 65536 positions are selected by one workgroup per row
# (holding 16K, 32K or 64K positions), longer rows by the tiled multi-kernel
# select: sizes in each class.
@gpu
@pytest.mark.parametrize("N", [3 * 4096 + 577, 5 * 4096 + 577, 16 * 4096 + 577])
@pytest.mark.parametrize("H_I,D_I,K", [(8, 128, 2048), (32, 128, 512), (4, 64, 256), (3, 32, 100), (16, 256, 64)])
def test_ragged_contexts_and_shapes(H_I, D_I, K, N):
    require_gpu()
    announce(f"index_score_topk ragged H_I={H_I} D_I={D_I} K={K} N={N}")
    B = 4
    k_idx = inputs.int_e4m3((B, N, D_I), 11, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, 1, H_I, D_I), 11, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, 1, H_I), 11, 1, "w", device="cuda")
    ctx = torch.tensor([N, 4096 + 17, K - 5 if K > 5 else 1, 0], dtype=torch.int32, device="cuda")
    _run_and_check(q_idx, w, k_idx, ctx, K)


@gpu
@pytest.mark.parametrize("N", [9000, 30000, 70000])
def test_all_ties_and_padding(N):
    require_gpu()
    announce(f"index_score_topk all ties (q = 0) and K > context N={N}")
    B, H_I, D_I = 2, 8, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 12, 0, "k_idx", device="cuda")
    q_idx = torch.zeros((B, 1, H_I, D_I), dtype=torch.uint8, device="cuda")
    w = inputs.normal_f32((B, 1, H_I), 12, 1, "w", device="cuda")
    ctx = torch.tensor([N, 700], dtype=torch.int32, device="cuda")
    res = _run_and_check(q_idx, w, k_idx, ctx, 1024)
    got = np_(res["topk_idx"])
    assert got[0].tolist()[0] == list(range(1024))
    assert got[1, 0, :700].tolist() == list(range(700)) and np.all(got[1, 0, 700:] == -1)


@gpu
@pytest.mark.parametrize("N", [12000, 20000, 70000])
def test_heavy_ties_small_integer_weights(N):
    require_gpu()
    announce(f"index_score_topk heavy ties N={N}")
    B, H_I, D_I = 2, 8, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 13, 0, "k_idx", lo=-1, hi=1, device="cuda")
    q_idx = inputs.int_e4m3((B, 1, H_I, D_I), 13, 1, "q_idx", lo=0, hi=1, device="cuda")
    w = torch.ones((B, 1, H_I), dtype=torch.float32, device="cuda")
    ctx = torch.tensor([N, N - 3], dtype=torch.int32, device="cuda")
    _run_and_check(q_idx, w, k_idx, ctx, 2048)


@gpu
@pytest.mark.parametrize("N", [16384, 16385, 32768, 32769, 65536, 65537])
def test_select_size_boundary(N):
    """Longest rows of each one-workgroup select size and one position past
    them; the second sequence has fewer visible positions than K."""
    require_gpu()
    announce(f"index_score_topk select boundary N={N}")
    B, H_I, D_I = 2, 8, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 16, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, 1, H_I, D_I), 16, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, 1, H_I), 16, 1, "w", device="cuda")
    ctx = torch.tensor([N, 2000], dtype=torch.int32, device="cuda")
    _run_and_check(q_idx, w, k_idx, ctx, 2048)


@gpu
def test_causal_rows_with_q_pos():
    require_gpu()
    announce("index_score_topk Tq=6 causal rows")
    B, Tq, N, H_I, D_I = 2, 6, 10000, 8, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 14, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 14, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 14, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 100], dtype=torch.int32, device="cuda")
    q_pos = torch.tensor([[9994, 9995, 9996, 9997, 9998, 9999], [10, 300, 5000, 8191, 8192, 9899]],
                         dtype=torch.int32, device="cuda")
    _run_and_check(q_idx, w, k_idx, ctx, 512, q_pos=q_pos)


@gpu
@pytest.mark.parametrize("H_I,D_I,Tq,K", [(8, 128, 40, 512), (3, 128, 17, 100), (32, 128, 20, 300),
                                         (8, 256, 33, 256), (13, 256, 16, 64), (8, 128, 70, 2048)])
def test_prefill_chunk_dense_scoring(H_I, D_I, Tq, K):
    """Chunks of 16 or more queries per sequence take the matrix-core product
    path; causal positions, a context shorter than some positions, a partial
    last query tile and K above the visible count all appear."""
    require_gpu()
    announce(f"index_score_topk prefill chunk H_I={H_I} D_I={D_I} Tq={Tq} K={K}")
    B, N = 3, 2 * 8192 + 1234
    k_idx = inputs.int_e4m3((B, N, D_I), 31, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 31, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 31, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 700, 5000], dtype=torch.int32, device="cuda")
    base = torch.tensor([N - Tq, N - Tq - 900, 4000], dtype=torch.int64)
    steps = torch.arange(Tq, dtype=torch.int64) * 37
    q_pos = (base[:, None] + steps[None, :]).clamp(max=N - 1)
    q_pos[0, :3] = torch.tensor([0, 5, K // 2])          # tiny visible prefixes
    q_pos = q_pos.to(torch.int32).cuda().contiguous()
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos)


@gpu
@pytest.mark.parametrize("block,nblocks,K", [(8, 64, 256), (8, 2048, 2048), (4, 100, 64), (1, 300, 300), (16, 40, 128),
                                             (16, 1100, 512), (16, 2100, 512), (1, 150, 64)])
def test_hierarchical_pool_and_pool_topk(block, nblocks, K):
    require_gpu()
    announce(f"pool block={block} nblocks={nblocks} K={K}")
    B, N, H_I, D_I = 3, 2 * 4096 + 4001, 8, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 15, 0, "k_idx", device="cuda")
    q0 = inputs.int_e4m3((B, 1, H_I, D_I), 15, 1, "q_idx", device="cuda")
    w0 = inputs.normal_f32((B, 1, H_I), 15, 1, "w", device="cuda")
    q1 = inputs.int_e4m3((B, 1, H_I, D_I), 15, 2, "q_idx", device="cuda")
    w1 = inputs.normal_f32((B, 1, H_I), 15, 2, "w", device="cuda")
    ctx = torch.tensor([N, N - 3, 1001], dtype=torch.int32, device="cuda")
    res = csa2.csa2_index_score_topk(q0, w0, k_idx, ctx, K, pool_block=block, pool_nblocks=nblocks)
    later = csa2.csa2_hier_pool_topk(q1, w1, k_idx, res["pool_idx"], res["pool_len"], K, want_scores=True)
    torch.cuda.synchronize()
    kh, q0h, w0h, q1h, w1h, ch = map(np_, (k_idx, q0, w0, q1, w1, ctx))
    for b in range(B):
        s0 = I.index_scores(q0h[b, 0], w0h[b, 0], kh[b], ch[b])
        pool, plen = P.hier_pool(s0, ch[b], block, nblocks)
        assert int(np_(res["pool_len"])[b, 0]) == plen
        assert np.array_equal(np_(res["pool_idx"])[b, 0], pool)
        flat, _ = topk_select(s0, ch[b], K)
        assert np.array_equal(np_(res["topk_idx"])[b, 0], flat)
        want_i, want_s = P.pool_topk(q1h[b, 0], w1h[b, 0], kh[b], pool, plen, K)
        assert np.array_equal(np_(later["topk_idx"])[b, 0], want_i)
        assert np.array_equal(np_(later["topk_score"])[b, 0], want_s)
        if nblocks >= K:   # containment: the flat Top-K lies inside the pool
            assert set(flat[flat >= 0].tolist()) <= set(pool[:plen].tolist())


@gpu
def test_decode64k_full_size_sampled_rows():
    """The 64-sequence x 64K configuration in the launch shape the benchmark
    times; two sequences are checked against the oracle element by element."""
    require_gpu()
    wl = inputs.WORKLOADS["decode64k"]
    announce("index_score_topk decode64k full size, rows 0 and 63 sampled")
    k_idx = inputs.int_e4m3((wl.B, wl.N, wl.D_I), wl.seed, 0, "k_idx", device="cuda")
    lay = inputs.decode_layer_inputs(wl, 0, device="cuda")
    ctx = torch.full((wl.B,), wl.N, dtype=torch.int32, device="cuda")
    res = csa2.csa2_index_score_topk(lay["q_idx"], lay["w"], k_idx, ctx, wl.K, want_scores=True)
    torch.cuda.synchronize()
    for b in (0, wl.B - 1):
        s = I.index_scores(np_(lay["q_idx"][b, 0]), np_(lay["w"][b, 0]), np_(k_idx[b]), wl.N)
        want_i, want_s = topk_select(s, wl.N, wl.K)
        assert np.array_equal(np_(res["topk_idx"][b, 0]), want_i)
        assert np.array_equal(np_(res["topk_score"][b, 0]), want_s)
    # every row: ascending, distinct, in range
    got = np_(res["topk_idx"])[:, 0]
    assert np.all(np.diff(got, axis=1) > 0) and got.min() >= 0 and got.max() < wl.N
