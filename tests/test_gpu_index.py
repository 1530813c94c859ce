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


def _run_and_check(q_idx, w, k_idx, ctx_len, k_top, q_pos=None, stored=False):
    res = csa2.csa2_index_score_topk(q_idx, w, k_idx, ctx_len, k_top, q_pos=q_pos, want_scores=True,
                                     stored_keys=stored)
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
@pytest.mark.parametrize("pool", [False, True])
@pytest.mark.parametrize("N", [65536, 200_003])
def test_repeated_calls_give_identical_results(N, pool):
    """The multi-pass select appends candidates with atomics, so their order in
    the workspace differs from call to call; the results must not.  Heavy ties
    at the threshold (scores in a few integer values); five calls, each
    followed by an unrelated call on the same workspace, all bit-identical to
    the first, which equals the oracle (Top-K and, with the pool, pool_idx and
    pool_len)."""
    require_gpu()
    announce(f"index_score_topk repeated calls N={N} pool={pool}")
    B, H_I, D_I, K = 3, 8, 128, 2048
    pb, nb = (8, 512) if pool else (0, 0)
    k_idx = inputs.int_e4m3((B, N, D_I), 21, 0, "k_idx", lo=-1, hi=1, device="cuda")
    q_idx = inputs.int_e4m3((B, 1, H_I, D_I), 21, 1, "q_idx", lo=0, hi=1, device="cuda")
    w = torch.ones((B, 1, H_I), dtype=torch.float32, device="cuda")
    ctx = torch.tensor([N, N - 5, N // 3], dtype=torch.int32, device="cuda")
    need = csa2.csa2_index_score_topk_workspace_size(B, 1, N, K, pb, nb)
    raw = torch.empty(need + 256, dtype=torch.uint8, device="cuda")
    off = (-raw.data_ptr()) % 256
    ws = raw[off:off + need]
    other_q = inputs.int_e4m3((B, 1, H_I, D_I), 22, 1, "q_idx", device="cuda")
    other_w = inputs.normal_f32((B, 1, H_I), 22, 1, "w", device="cuda")
    runs = []
    for _ in range(5):
        r = csa2.csa2_index_score_topk(q_idx, w, k_idx, ctx, K, want_scores=True, pool_block=pb, pool_nblocks=nb,
                                       workspace=ws)
        torch.cuda.synchronize()
        runs.append({key: np_(v).copy() for key, v in r.items() if v is not None})
        csa2.csa2_index_score_topk(other_q, other_w, k_idx, ctx, K, pool_block=pb, pool_nblocks=nb, workspace=ws)
    for r in runs[1:]:
        assert r.keys() == runs[0].keys()
        for key in runs[0]:
            assert np.array_equal(r[key], runs[0][key]), key
    qn, wn, kn, cn = np_(q_idx), np_(w), np_(k_idx), np_(ctx)
    want_i, want_s = _oracle_rows(qn, wn, kn, cn, K)
    assert np.array_equal(runs[0]["topk_idx"], want_i)
    assert np.array_equal(runs[0]["topk_score"], want_s)
    if pool:
        for bb in range(B):
            sc = I.index_scores(qn[bb, 0], wn[bb, 0], kn[bb], int(cn[bb]))
            pi, pl = P.hier_pool(sc, int(cn[bb]), pb, nb)
            assert runs[0]["pool_len"][bb, 0] == pl
            assert np.array_equal(runs[0]["pool_idx"][bb, 0], pi)


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
@pytest.mark.parametrize("stored", [False, True], ids=["passes", "stored_keys"])
@pytest.mark.parametrize("H_I,D_I,Tq,K", [(8, 128, 40, 512), (3, 128, 17, 100), (32, 128, 20, 300),
                                         (8, 256, 33, 256), (13, 256, 16, 64), (8, 128, 70, 2048),
                                         (8, 128, 24, 8192)])
def test_prefill_chunk_dense_scoring(H_I, D_I, Tq, K, stored):
    """Chunks of 16 or more queries per sequence take the matrix-core product
    path; causal positions, a context shorter than some positions, a partial
    last query tile and K above the visible count all appear.  The default
    workspace selects by scoring passes, the stored-key workspace from the
    stored score keys."""
    require_gpu()
    announce(f"index_score_topk prefill chunk H_I={H_I} D_I={D_I} Tq={Tq} K={K} stored={stored}")
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
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos, stored=stored)


@gpu
@pytest.mark.parametrize("qmax,K", [(1, 300), (0, 700), (1, 2500)])
def test_prefill_selection_passes_under_heavy_ties(qmax, K):
    """Dense prefill chunks in the default workspace select without storing
    their score keys, by repeated scoring passes.  Keys in {-1, 0, 1}, queries in {0 .. qmax} and
    unit weights give a handful of integer scores: the bucket at the
    threshold holds thousands of keys, so rows go through the second and
    third digit levels and the tie count / tie emission passes (qmax = 0:
    every score is 0 and the K lowest positions win).  Early rows see fewer
    than K positions."""
    require_gpu()
    announce(f"index_score_topk prefill heavy ties qmax={qmax} K={K}")
    B, N, Tq, H_I, D_I = 2, 3 * 8192 + 321, 40, 8, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 41, 0, "k_idx", lo=-1, hi=1, device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 41, 1, "q_idx", lo=0, hi=qmax, device="cuda")
    w = torch.ones((B, Tq, H_I), dtype=torch.float32, device="cuda")
    ctx = torch.tensor([N, N - 4000], dtype=torch.int32, device="cuda")
    base = torch.tensor([N - Tq, N - 4000 - Tq], dtype=torch.int64)
    q_pos = base[:, None] + torch.arange(Tq, dtype=torch.int64)[None, :]
    q_pos[0, :4] = torch.tensor([0, 7, K - 1, K])
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos.to(torch.int32).cuda().contiguous())


@gpu
@pytest.mark.parametrize("D_I,H_I", [(128, 8), (256, 8)])
def test_prefill_selection_guess_on_small_samples(D_I, H_I):
    """Rows that see only a little more than K positions: the first pass's
    sample holds a few dozen keys, the guessed window reaches down to the
    lowest key, and every visible key not emitted becomes a candidate."""
    require_gpu()
    announce(f"index_score_topk prefill guess on small samples D_I={D_I}")
    B, N, Tq, K = 1, 2000, 32, 512
    k_idx = inputs.int_e4m3((B, N, D_I), 46, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 46, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 46, 1, "w", device="cuda")
    ctx = torch.tensor([N], dtype=torch.int32, device="cuda")
    q_pos = (K + 5 * torch.arange(Tq, dtype=torch.int32, device="cuda"))[None, :].contiguous()
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos)


@gpu
def test_prefill_selection_blocks_across_sequences():
    """2,100 query rows select in two blocks of query tiles (at most 1,920
    rows each), the block boundary inside the second sequence; every
    sequence ends with a partial query tile, and the third has no visible
    key at all (every index -1, every score -inf)."""
    require_gpu()
    announce("index_score_topk prefill blocks across sequences B=3 Tq=700 N=5000")
    B, N, Tq, H_I, D_I, K = 3, 5000, 700, 8, 128, 300
    k_idx = inputs.int_e4m3((B, N, D_I), 47, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 47, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 47, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 300, 0], dtype=torch.int32, device="cuda")
    base = torch.tensor([N - Tq, N - 300 - Tq, 0], dtype=torch.int64)
    q_pos = (base[:, None] + torch.arange(Tq, dtype=torch.int64)[None, :]).to(torch.int32).cuda().contiguous()
    res = _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos)
    assert bool((res["topk_idx"][2] == -1).all())


@gpu
def test_prefill_selection_sorts_many_candidates():
    """About half of the keys score exactly 0 (keys in {-1, 0, 1}, a query
    of ones, unit weights) and K falls inside them: the candidates at the
    threshold number between 2,048 and 4,096, past the register sort, and the
    lowest positions among the ties are taken."""
    require_gpu()
    announce("index_score_topk prefill with 2048..4096 candidates")
    B, N, Tq, H_I, D_I, K = 1, 6000, 32, 8, 128, 3500
    k_idx = inputs.int_e4m3((B, N, D_I), 48, 0, "k_idx", lo=-1, hi=1, device="cuda")
    q_idx = torch.full((B, Tq, H_I, D_I), 0x38, dtype=torch.uint8, device="cuda")   # E4M3 1.0
    w = torch.ones((B, Tq, H_I), dtype=torch.float32, device="cuda")
    ctx = torch.tensor([N], dtype=torch.int32, device="cuda")
    q_pos = torch.full((B, Tq), N - 1, dtype=torch.int32, device="cuda")
    sc = I.index_scores(np_(q_idx)[0, 0], np_(w)[0, 0], np_(k_idx)[0], N)
    zeros = int(np.sum(sc == 0.0))
    assert 2048 < zeros <= 4096 and int(np.sum(sc > 0.0)) < K < int(np.sum(sc >= 0.0))
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos)


@gpu
def test_prefill_selection_takes_a_whole_bucket():
    """The K-th largest score's bucket is taken whole (the K selected keys are
    exactly the keys at or above one score value): every row has the same
    query, so K can be set to such a count from the oracle's scores."""
    require_gpu()
    announce("index_score_topk prefill whole threshold bucket")
    B, N, Tq, H_I, D_I = 1, 20000, 32, 4, 128
    k_idx = inputs.int_e4m3((B, N, D_I), 43, 0, "k_idx", lo=-1, hi=1, device="cuda")
    q_one = inputs.int_e4m3((1, 1, H_I, D_I), 43, 1, "q_idx", lo=0, hi=1, device="cuda")
    q_idx = q_one.expand(B, Tq, H_I, D_I).contiguous()
    w = torch.ones((B, Tq, H_I), dtype=torch.float32, device="cuda")
    ctx = torch.tensor([N], dtype=torch.int32, device="cuda")
    q_pos = torch.full((B, Tq), N - 1, dtype=torch.int32, device="cuda")
    sc = I.index_scores(np_(q_one)[0, 0], np_(w)[0, 0], np_(k_idx)[0], N)
    vals = np.unique(sc)[::-1]
    K = int(np.sum(sc >= vals[3]))
    assert 0 < K < N
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos)


@gpu
def test_prefill_selection_final_order_long_and_short_rows():
    """The last kernel of the selection puts a row's positions in ascending
    order by their rank in a position bitmap while the row sees at most
    335,872 positions, and by a sort beyond that: one chunk with a row on
    each side of the bound, one exactly at it, and a row with fewer than K
    positions."""
    require_gpu()
    announce("index_score_topk prefill final order, rows of 2K to 340K positions")
    B, N, Tq, H_I, D_I, K = 1, 340_000, 16, 8, 128, 2048
    k_idx = inputs.int_e4m3((B, N, D_I), 49, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 49, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 49, 1, "w", device="cuda")
    ctx = torch.tensor([N], dtype=torch.int32, device="cuda")
    # (one row beyond the bound, one at it, the rest short; the first short
    # one sees fewer than K positions)
    pos = [N - 1, 335_871] + [1_900 + 700 * i for i in range(14)]
    q_pos = torch.tensor([pos], dtype=torch.int32, device="cuda")
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos)


@gpu
@pytest.mark.parametrize("D_I,H_I,Tq", [(64, 8, 20), (32, 4, 33)])
def test_prefill_chunks_of_row_scans(D_I, H_I, Tq):
    """Chunk shapes the matrix-core product does not take are scanned a few
    query rows at a time through the default workspace."""
    require_gpu()
    announce(f"index_score_topk prefill as row scans D_I={D_I} H_I={H_I} Tq={Tq}")
    B, N, K = 2, 9000, 256
    k_idx = inputs.int_e4m3((B, N, D_I), 44, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 44, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 44, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 500], dtype=torch.int32, device="cuda")
    q_pos = (ctx[:, None].to(torch.int64) - Tq + torch.arange(Tq, device="cuda")[None, :]).to(torch.int32)
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos.contiguous())


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
    later = csa2.csa2_hier_pool_topk(q1, w1, k_idx, res["pool_idx"], res["pool_len"], K, ctx_len=ctx,
                                     want_scores=True)
    torch.cuda.synchronize()
    kh, q0h, w0h, q1h, w1h, ch = map(np_, (k_idx, q0, w0, q1, w1, ctx))
    for b in range(B):
        s0 = I.index_scores(q0h[b, 0], w0h[b, 0], kh[b], ch[b])
        pool, plen = P.hier_pool(s0, ch[b], block, nblocks)
        assert int(np_(res["pool_len"])[b, 0]) == plen
        assert np.array_equal(np_(res["pool_idx"])[b, 0], pool)
        flat, _ = topk_select(s0, ch[b], K)
        assert np.array_equal(np_(res["topk_idx"])[b, 0], flat)
        want_i, want_s = P.pool_topk(q1h[b, 0], w1h[b, 0], kh[b], pool, plen, K, ctx_len=ch[b])
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


@gpu
def test_maximum_context_with_a_huge_zero_tie_bucket():
    """Rows at the documented limit of 4,194,304 positions (one whole, one
    ragged by 777), every key row zero except 3,000 random ones per sequence.
    A zero key row scores +0 under the oracle's definition, so the positive
    scores (about half of the 3,000) are taken first and the rest of the
    Top-2048 is the lowest-index ties at +0, out of a bucket of some four
    million equal keys (the crowded-bucket path of the long-row select);
    negative scores rank below the ties."""
    require_gpu()
    B, N, H_I, D_I, K, S = 2, 1 << 22, 8, 128, 2048, 3000
    announce(f"index_score_topk at the row limit: B={B} N={N} ctx N and N-777, {S} nonzero keys per row, K={K}")
    g = torch.Generator().manual_seed(4_194_304)
    pos = [torch.randperm(N - 777, generator=g)[:S].sort().values for _ in range(B)]
    rows = inputs.int_e4m3((B, S, D_I), 9, 11, "k_idx", device="cuda")
    k_idx = torch.zeros((B, N, D_I), dtype=torch.uint8, device="cuda")
    for b in range(B):
        k_idx[b, pos[b].cuda()] = rows[b]
    q_idx = inputs.int_e4m3((B, 1, H_I, D_I), 9, 11, "q_idx", device="cuda")
    w = inputs.normal_f32((B, 1, H_I), 9, 11, "w", device="cuda")
    ctx = torch.tensor([N, N - 777], dtype=torch.int32, device="cuda")
    res = csa2.csa2_index_score_topk(q_idx, w, k_idx, ctx, K, want_scores=True)
    torch.cuda.synchronize()
    zero = I.index_scores(np_(q_idx[0, 0]), np_(w[0, 0]), np.zeros((4, D_I), np.uint8), 4)
    assert np.all(zero == 0) and not np.any(np.signbit(zero))
    for b in range(B):
        nv = int(ctx[b])
        s = np.zeros(N, dtype=np.float32)
        s[nv:] = -np.inf
        s[np_(pos[b])] = I.index_scores(np_(q_idx[b, 0]), np_(w[b, 0]), np_(rows[b]), S)
        want_i, want_s = topk_select(s, nv, K)
        assert 0 < int((want_s > 0).sum()) < K and int((want_s == 0).sum()) > 0   # both kinds are taken
        assert np.array_equal(np_(res["topk_idx"][b, 0]), want_i)
        assert np.array_equal(np_(res["topk_score"][b, 0]), want_s)


def _dot_rows(dots, D_I=128):
    """E4M3 key rows whose dot with an all-ones query row is the given integer
    (the first `dot` bytes are 1.0, the rest 0)."""
    dots = np.asarray(dots, dtype=np.int64)
    rows = (np.arange(D_I)[None, :] < dots[:, None]).astype(np.float32)
    return torch.from_numpy(rows).to(torch.float8_e4m3fn).view(torch.uint8)


# Block-pool thresholds.  Head 0 has weight -1/8 and an all-ones query, the
# other heads weight 0, so a token's score is -dot/8 exactly: dot 22 -> -2.75,
# 24 -> -3.0 (the order-preserving key 0x3FBFFFFF: the bucket 0x3FB with all 20
# low bits set), 25 -> -3.125, 26 or more -> -3.25 or less.  The context ends
# in a 3-token partial block whose maximum is -3.0 in every case.
#   whole_bucket: 64 blocks at -2.75 = the whole top bucket; the threshold is
#                 the key just below it, which is the last block's key;
#   ties_partial: 60 blocks at -2.75, 10 at -3.0 (the last among them), 5 at
#                 -3.125: 4 of the 10 ties are taken, the last block is not;
#   ties_all:     60 at -2.75, 4 at -3.0 (the last among them), 5 at -3.125:
#                 every tie is taken, the last (partial) block too.
@gpu
@pytest.mark.parametrize("case", ["whole_bucket", "ties_partial", "ties_all"])
def test_pool_length_at_threshold_keys(case):
    require_gpu()
    announce(f"pool length threshold case {case}")
    rng = np.random.default_rng({"whole_bucket": 1, "ties_partial": 2, "ties_all": 3}[case])
    nblk, nsel, H_I, D_I, K = 200, 64, 8, 128, 256
    N = 8 * (nblk - 1) + 3
    dots = rng.integers(26, 60, N)                      # every block at <= -3.25 by default
    blocks = rng.permutation(nblk - 1)                  # full blocks in random order
    n_top = 64 if case == "whole_bucket" else 60
    n_tie = {"whole_bucket": 20, "ties_partial": 9, "ties_all": 3}[case]   # full tie blocks besides the last
    top, tie = blocks[:n_top], blocks[n_top:n_top + n_tie]
    low = blocks[n_top + n_tie:n_top + n_tie + (0 if case == "whole_bucket" else 5)]
    for c in top:
        dots[8 * c + rng.integers(0, 8)] = 22
    for c in tie:
        dots[8 * c + rng.integers(0, 8)] = 24
    for c in low:
        dots[8 * c + rng.integers(0, 8)] = 25
    dots[N - 3:] = [30, 24, 27]                         # the partial last block: max -3.0
    k_idx = _dot_rows(dots, D_I).reshape(1, N, D_I).cuda()
    q = np.zeros((1, 1, H_I, D_I), np.float32)
    q[0, 0, 0] = 1.0
    q[0, 0, 1:] = rng.integers(-4, 5, (H_I - 1, D_I))
    q_idx = torch.from_numpy(q).to(torch.float8_e4m3fn).view(torch.uint8).cuda()
    w = torch.zeros(1, 1, H_I, dtype=torch.float32)
    w[0, 0, 0] = -0.125
    w = w.cuda()
    q1 = inputs.int_e4m3((1, 1, H_I, D_I), 21, 1, "q_idx", device="cuda")
    w1 = inputs.normal_f32((1, 1, H_I), 21, 1, "w", device="cuda")
    ctx = torch.tensor([N], dtype=torch.int32, device="cuda")
    res = csa2.csa2_index_score_topk(q_idx, w, k_idx, ctx, K, pool_block=8, pool_nblocks=nsel)
    later = csa2.csa2_hier_pool_topk(q1, w1, k_idx, res["pool_idx"], res["pool_len"], K, ctx_len=ctx,
                                     want_scores=True)
    torch.cuda.synchronize()
    kh = np_(k_idx[0])
    s0 = I.index_scores(np_(q_idx[0, 0]), np_(w[0, 0]), kh, N)
    assert np.array_equal(s0, (-dots / 8.0).astype(np.float32))   # the construction holds
    pool, plen = P.hier_pool(s0, N, 8, nsel)
    want_len = 8 * nsel - (5 if case == "ties_all" else 0)
    assert plen == want_len
    assert int(np_(res["pool_len"])[0, 0]) == plen
    assert np.array_equal(np_(res["pool_idx"])[0, 0], pool)
    flat, _ = topk_select(s0, N, K)
    assert np.array_equal(np_(res["topk_idx"])[0, 0], flat)
    want_i, want_s = P.pool_topk(np_(q1[0, 0]), np_(w1[0, 0]), kh, pool, plen, K, ctx_len=N)
    assert np.array_equal(np_(later["topk_idx"])[0, 0], want_i)
    assert np.array_equal(np_(later["topk_score"])[0, 0], want_s)


@gpu
@pytest.mark.parametrize("pool_cap", [3000, 40000])
def test_pool_ids_outside_the_context_are_skipped(pool_cap):
    """-1, negative, stale (>= ctx_len but inside the cache) and far out-of-range
    ids inside pool_len name no token: never read, never selected.  Both select
    designs (pools up to 32K positions and longer)."""
    require_gpu()
    announce(f"pool with invalid ids, pool_cap={pool_cap}")
    B, N, H_I, D_I, K = 2, 60000, 8, 128, 700
    rng = np.random.default_rng(pool_cap)
    k_idx = inputs.int_e4m3((B, N, D_I), 23, 0, "k_idx", device="cuda")
    q1 = inputs.int_e4m3((B, 1, H_I, D_I), 23, 1, "q_idx", device="cuda")
    w1 = inputs.normal_f32((B, 1, H_I), 23, 1, "w", device="cuda")
    ctx = torch.tensor([N - 5000, N], dtype=torch.int32, device="cuda")
    pool = np.full((B, 1, pool_cap), -1, np.int32)
    plen = np.zeros((B, 1), np.int32)
    for b in range(B):
        n = pool_cap - 37
        ids = np.sort(rng.choice(N, n, replace=False)).astype(np.int32)
        bad = rng.choice(n, n // 10, replace=False)
        ids[bad[0::3]] = -1
        ids[bad[1::3]] = -123456
        ids[bad[2::3]] = 1 << 30
        pool[b, 0, :n] = ids
        plen[b, 0] = n
    pool_t, plen_t = torch.from_numpy(pool).cuda(), torch.from_numpy(plen).cuda()
    later = csa2.csa2_hier_pool_topk(q1, w1, k_idx, pool_t, plen_t, K, ctx_len=ctx, want_scores=True)
    torch.cuda.synchronize()
    kh, ch = np_(k_idx), np_(ctx)
    for b in range(B):
        want_i, want_s = P.pool_topk(np_(q1[b, 0]), np_(w1[b, 0]), kh[b], pool[b, 0], plen[b, 0], K, ctx_len=ch[b])
        assert np.array_equal(np_(later["topk_idx"])[b, 0], want_i)
        assert np.array_equal(np_(later["topk_score"])[b, 0], want_s)
        got = np_(later["topk_idx"])[b, 0]
        assert got[got >= 0].max() < ch[b]


@gpu
@pytest.mark.parametrize("Tq", [2, 3, 4, 7])
@pytest.mark.parametrize("N,H_I", [(20000, 8), (70001, 5)])
def test_multi_query_decode_shares_one_key_pass(Tq, N, H_I):
    """2..15 query rows per sequence (speculative verification): one scan
    workgroup scores 2 or 4 rows against each key tile.  Every row must equal
    its own single-row oracle: causal positions at the end of the context,
    a row with a short visible prefix, ragged contexts, both select designs."""
    require_gpu()
    announce(f"multi-query decode Tq={Tq} N={N} H_I={H_I}")
    B, D_I, K = 3, 128, 512
    k_idx = inputs.int_e4m3((B, N, D_I), 61, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 61, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 61, 1, "w", device="cuda")
    ctx = torch.tensor([N, N - 17, N // 3], dtype=torch.int32, device="cuda")
    q_pos = (ctx[:, None].to(torch.int64) - Tq + torch.arange(Tq, device="cuda")[None, :]).to(torch.int32)
    q_pos[1, 0] = 300        # a short visible prefix inside a group
    _run_and_check(q_idx, w, k_idx, ctx, K, q_pos=q_pos.contiguous())
    _run_and_check(q_idx, w, k_idx, ctx, K)   # no positions: every row sees its whole context


@gpu
def test_multi_query_decode64k_sampled_rows():
    """Two query tokens per sequence at 64 x 64K, the launch shape the
    benchmark times; rows of the first and last sequence are checked."""
    require_gpu()
    announce("multi-query decode B64 x 64K Tq=2, sequences 0 and 63 sampled")
    B, N, Tq, H_I, D_I, K = 64, 65536, 2, 8, 128, 2048
    k_idx = inputs.int_e4m3((B, N, D_I), 62, 0, "k_idx", device="cuda")
    q_idx = inputs.int_e4m3((B, Tq, H_I, D_I), 62, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), 62, 1, "w", device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    q_pos = (torch.arange(Tq, dtype=torch.int32, device="cuda") + N - Tq).repeat(B, 1).contiguous()
    res = csa2.csa2_index_score_topk(q_idx, w, k_idx, ctx, K, q_pos=q_pos, want_scores=True)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        for t in range(Tq):
            s = I.index_scores(np_(q_idx[b, t]), np_(w[b, t]), np_(k_idx[b]), N - Tq + t + 1)
            want_i, want_s = topk_select(s, N - Tq + t + 1, K)
            assert np.array_equal(np_(res["topk_idx"][b, t]), want_i), (b, t)
            assert np.array_equal(np_(res["topk_score"][b, t]), want_s), (b, t)
