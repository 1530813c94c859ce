"""GPU parity of the paged main cache + ring window attention
(csa2_sparse_attn_paged) against the float64 oracle, and against the linear
layouts holding the same rows (bit-identical: same entries in the same order,
same arithmetic)."""

import numpy as np
import pytest
import torch

import fp4_kv_cache_index_amd as csa2
from fp4_kv_cache_index_amd import inputs
from oracle import attention as A
from oracle import quant as Q
from tests.gpu_util import ATTN_TOL, LSE_TOL, announce, gpu, np_, require_gpu, rowwise_rel_err


def _paged_case(B, N, d_qk, page, n_pages, R, swa_end, seed):
    """Linear caches of B sequences and the same rows scattered into a page
    pool (random page order, unused pages) and rings of R rows."""
    g = np.random.default_rng(seed)
    kv_x = inputs.normal_f32((B, N, d_qk), seed, 0, "kv", device="cuda")
    lin = torch.empty((B, N, d_qk // 2 + d_qk // 16), dtype=torch.uint8, device="cuda")
    csa2.kv_fp4_quantize(kv_x, codes=lin[..., : d_qk // 2], scales=lin[..., d_qk // 2:])
    npg = (N + page - 1) // page
    perm = torch.from_numpy(g.permutation(n_pages)[: B * npg].astype(np.int64)).cuda()
    bt = torch.full((B, npg + 2), -1, dtype=torch.int32, device="cuda")
    bt[:, :npg] = perm.view(B, npg).to(torch.int32)
    pool = torch.zeros((n_pages * page, lin.shape[-1]), dtype=torch.uint8, device="cuda")
    j = torch.arange(N, device="cuda")
    for b in range(B):
        rows = bt[b, j // page].to(torch.int64) * page + j % page
        pool[rows] = lin[b]
    # window positions 0 .. max(swa_end) - 1 in a linear array, then the ring
    swa_x = inputs.normal_f32((B, int(max(swa_end)), d_qk), seed, 1, "swa", device="cuda")
    sv, ss = csa2.swa_fp8_quantize(swa_x)
    ring_v = torch.zeros((B, R, d_qk), dtype=torch.uint8, device="cuda")
    ring_s = torch.zeros((B, R, d_qk // 32), dtype=torch.uint8, device="cuda")
    for b in range(B):
        for x in range(max(0, swa_end[b] - R), swa_end[b]):
            ring_v[b, x % R], ring_s[b, x % R] = sv[b, x], ss[b, x]
    return dict(kv_x=kv_x, lin=lin, bt=bt, pool=pool, swa_x=swa_x, sv=sv, ss=ss, ring_v=ring_v, ring_s=ring_s,
                end=torch.tensor(swa_end, dtype=torch.int32, device="cuda"))


def _oracle(c, q, idx, ctx, q_pos, page, n_pages, R, W, d_qk, scale):
    B, Tq = q.shape[:2]
    pool = np_(c["pool"])
    pc, ps = pool[:, : d_qk // 2], pool[:, d_qk // 2:]
    outs = np.zeros(q.shape[:3] + (512,))
    lses = np.zeros(q.shape[:3])
    for b in range(B):
        rv, rs = np_(c["ring_v"][b]), np_(c["ring_s"][b])
        for t in range(Tq):
            o, l = A.sparse_attn_paged_row(np_(q[b, t]), pc, ps, np_(c["bt"][b]), page, n_pages, np_(idx[b, t]),
                                           int(ctx[b]), int(q_pos[b, t]), rv, rs, R, int(c["end"][b]), W, d_qk, 512,
                                           scale)
            outs[b, t], lses[b, t] = o, l
    return outs, lses


@gpu
@pytest.mark.parametrize("Tq,page,R,K", [(1, 64, 128, 700), (1, 16, 200, 700), (3, 64, 131, 700), (2, 64, 128, 0)])
def test_paged_attention_against_the_oracle(Tq, page, R, K):
    require_gpu()
    announce(f"paged attention Tq={Tq} page={page} ring={R} K={K}")
    B, N, d_qk, H, W = 3, 3000, 576, 64, 128
    n_pages = 3 * ((N + page - 1) // page) + 11
    swa_end = [N, N - 40, 97]                     # a wrapped ring, a partial one
    c = _paged_case(B, N, d_qk, page, n_pages, R, swa_end, 71 + page)
    ctx = torch.tensor([N, N - 40, 2000], dtype=torch.int32, device="cuda")
    idx = torch.stack([inputs.random_index_lists(B, K, N, 71, layer=t, device="cuda", n_invalid=9 if K else 0)
                       for t in range(Tq)], dim=1).contiguous()
    c["bt"][1, 5] = -1                            # a missing page
    c["bt"][2, 7] = n_pages + 3                   # an entry outside the pool
    q = inputs.normal_f32((B, Tq, H, d_qk), 71, 2, "q", device="cuda")
    q_pos = (ctx[:, None].to(torch.int64) - Tq + torch.arange(Tq, device="cuda")[None, :]).to(torch.int32)
    q_pos[2, 0] = 60                              # before most of the window
    q_pos = q_pos.contiguous()
    scale = 1 / np.sqrt(576.0)
    out, lse = csa2.csa2_sparse_attn_paged(q, c["pool"][:, : d_qk // 2], c["pool"][:, d_qk // 2:], c["bt"], page, idx,
                                           ctx, q_pos, c["ring_v"], c["ring_s"], c["end"], W, scale, want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle(c, q, idx, np_(ctx), np_(q_pos), page, n_pages, R, W, d_qk, scale)
    err = rowwise_rel_err(np_(out), want_o)
    assert err <= ATTN_TOL, err
    fin = np.isfinite(want_l)
    assert np.array_equal(fin, np.isfinite(np_(lse)))
    assert np.max(np.abs(np_(lse)[fin] - want_l[fin]), initial=0.0) <= LSE_TOL


@gpu
def test_paged_decode_without_positions_and_equal_to_the_linear_layout():
    """Tq = 1 with q_pos NULL (the query sits at ctx_len - 1) must give exactly
    the linear prefill layout's result over the same rows: Top-K rows in the
    same order, window rows in position order."""
    require_gpu()
    announce("paged decode == linear layout, 64 x 5000")
    B, N, d_qk, H, K, W, page, R = 64, 5000, 576, 64, 2048, 128, 64, 128
    n_pages = B * ((N + page - 1) // page) + 5
    c = _paged_case(B, N, d_qk, page, n_pages, R, [N] * B, 81)
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    idx = inputs.random_index_lists(B, K, N, 81, device="cuda").view(B, 1, K).contiguous()
    q = inputs.normal_f32((B, 1, H, d_qk), 81, 2, "q", device="cuda")
    scale = 1 / np.sqrt(576.0)
    o1, l1 = csa2.csa2_sparse_attn_paged(q, c["pool"][:, : d_qk // 2], c["pool"][:, d_qk // 2:], c["bt"], page, idx,
                                         ctx, None, c["ring_v"], c["ring_s"], c["end"], W, scale, want_lse=True)
    q_pos = (ctx - 1).view(B, 1).contiguous()
    pos0 = torch.full((B,), N - W, dtype=torch.int32, device="cuda")
    o2, l2 = csa2.csa2_sparse_attn_prefill(q, c["lin"][..., : d_qk // 2], c["lin"][..., d_qk // 2:], idx, ctx, q_pos,
                                           c["sv"][:, N - W:], c["ss"][:, N - W:], pos0, W, scale, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
