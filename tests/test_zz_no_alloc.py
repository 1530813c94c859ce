"""GPU check of csa2_index_score_topk_noalloc (the no-allocation variant of the
indexer scoring + Top-K call, whose workspace is a static device array).

It is called through the C ABI and compared, element by element, with
csa2_index_score_topk given a workspace of its own, on calls in a row where
a later call has a smaller input: first a pool call (the multi-pass select,
whose counters and histograms must be cleared in the static array), then a
smaller pool call, then a 64K-token decode call and a smaller decode call,
then dense prefill chunks (one whose score keys do not fit the array, so it
selects by scoring passes inside it, then one whose keys do).  A call whose
inputs need more than the array holds returns CSA2_ESCRATCH.
"""

import ctypes

import numpy as np
import pytest
import torch

import fp4_kv_cache_index_amd as csa2
from fp4_kv_cache_index_amd import inputs
from tests.gpu_util import announce, gpu, np_, require_gpu

CSA2_ESCRATCH = 5


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc(q_idx, w, k_idx, ctx, k_top, pool_block=0, pool_nblocks=0, q_pos=None):
    B, Tq, H_I, D_I = q_idx.shape
    N = k_idx.shape[1]
    dev = q_idx.device
    idx = torch.full((B, Tq, k_top), -7, dtype=torch.int32, device=dev)
    sc = torch.full((B, Tq, k_top), 7.0, dtype=torch.float32, device=dev)
    pool_idx = pool_len = None
    if pool_nblocks:
        pool_idx = torch.full((B, Tq, pool_block * pool_nblocks), -7, dtype=torch.int32, device=dev)
        pool_len = torch.full((B, Tq), -7, dtype=torch.int32, device=dev)
    st = csa2.lib().csa2_index_score_topk_noalloc(
        _p(q_idx), _p(w), _p(k_idx), k_idx.stride(0), k_idx.stride(1), _p(ctx), _p(q_pos), B, Tq, H_I, D_I, N, k_top,
        _p(idx), _p(sc), pool_block, pool_nblocks, _p(pool_idx), _p(pool_len),
        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == 0, csa2.lib().csa2_status_string(st)
    return {"topk_idx": idx, "topk_score": sc, "pool_idx": pool_idx, "pool_len": pool_len}


def _case(seed, B, N, H_I, D_I, K, ctx_vals, pool_block=0, pool_nblocks=0, Tq=1):
    k_idx = inputs.int_e4m3((B, N, D_I), seed, 0, "k_idx", device="cuda")
    q = inputs.int_e4m3((B, Tq, H_I, D_I), seed, 1, "q_idx", device="cuda")
    w = inputs.normal_f32((B, Tq, H_I), seed, 1, "w", device="cuda")
    ctx = torch.tensor(ctx_vals, dtype=torch.int32, device="cuda")
    q_pos = None
    if Tq > 1:   # causal rows ending at each sequence's last token
        q_pos = (ctx[:, None].to(torch.int64) - Tq + torch.arange(Tq, device="cuda")[None, :]).clamp(min=0)
        q_pos = q_pos.to(torch.int32).contiguous()
    got = _noalloc(q, w, k_idx, ctx, K, pool_block, pool_nblocks, q_pos)
    want = csa2.csa2_index_score_topk(q, w, k_idx, ctx, K, q_pos=q_pos, pool_block=pool_block,
                                      pool_nblocks=pool_nblocks, want_scores=True)
    torch.cuda.synchronize()
    for key in ("topk_idx", "topk_score", "pool_idx", "pool_len"):
        if want[key] is not None:
            assert np.array_equal(np_(got[key]), np_(want[key])), key


@gpu
def test_noalloc_matches_the_workspace_call_on_consecutive_calls():
    require_gpu()
    announce("noalloc: pool 3 x 200K, then pool 1 x 70K")
    _case(31, 3, 200_000, 8, 128, 2048, [200_000, 199_997, 150_001], pool_block=8, pool_nblocks=2048)
    _case(32, 1, 70_000, 8, 128, 512, [69_995], pool_block=8, pool_nblocks=300)
    announce("noalloc: decode 64 x 64K, then 3 x 9000")
    _case(33, 64, 65536, 8, 128, 2048, [65536] * 64)
    _case(34, 3, 9000, 4, 64, 256, [9000, 8999, 17])
    announce("noalloc: prefill chunk 1 x 1200 queries on 20000 keys, then 2 x 40 on 9000")
    assert csa2.csa2_index_score_topk_workspace_size_stored(1, 1200, 20_000, 1024) > (64 << 20)
    assert csa2.csa2_index_score_topk_workspace_size(1, 1200, 20_000, 1024) <= (64 << 20)
    _case(35, 1, 20_000, 8, 128, 1024, [20_000], Tq=1200)
    _case(36, 2, 9000, 8, 128, 300, [9000, 8500], Tq=40)


@gpu
def test_noalloc_rejects_inputs_beyond_the_static_scratch():
    require_gpu()
    announce("noalloc: inputs beyond the static scratch")
    B, N, H_I, D_I = 64, 1 << 20, 8, 128
    need = csa2.csa2_index_score_topk_workspace_size(B, 1, N, 2048)
    assert need > (64 << 20)
    dev = torch.device("cuda")
    q = torch.zeros(1, dtype=torch.uint8, device=dev)
    st = csa2.lib().csa2_index_score_topk_noalloc(
        _p(q), _p(q), _p(q), N * D_I, D_I, _p(q), None, B, 1, H_I, D_I, N, 2048, _p(q), None, 0, 0, None, None,
        ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream))
    assert st == CSA2_ESCRATCH
