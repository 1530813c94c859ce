"""GPU parity of the sparse attention (decode and prefill) against the float64 oracle.

Tolerance: for every (query row, head), max|o - o_ref| / max|o_ref| <= 2e-3,
and |lse - lse_ref| <= 2e-3.  Derivation: K/V rows enter the fp16 matrix
cores exactly (main rows always; window rows while every block's E8M0 code
lies in [112, 134]); q and P are rounded to fp16 once (relative 2^-11), which
moves each logit by about scale * |q| |k| * 2^-12 (~3e-4 for unit-variance
rows at scale 1/sqrt(576)) and each weight by the same relative amount; fp32
accumulation adds < 1e-6.  The bound therefore holds up to a logit spread of
about 4x that of the configurations (unit-variance q and k at 4 / sqrt(576));
beyond it the fp16 rounding of q dominates (the documented limit of the ABI).
"""

import numpy as np
import pytest
import torch

import fp4_kv_cache_index_amd as csa2
from fp4_kv_cache_index_amd import inputs
from oracle import attention as A
from oracle import quant as Q
from tests.gpu_util import ATTN_TOL, LSE_TOL, announce, gpu, np_, require_gpu, rowwise_rel_err


def _make_caches(B, N, d_qk, W, seed, interleaved=True):
    kv_x = inputs.normal_f32((B, N, d_qk), seed, 0, "kv", device="cuda")
    if interleaved:
        cache = torch.empty((B, N, d_qk // 2 + d_qk // 16), dtype=torch.uint8, device="cuda")
        codes, scales = cache[..., : d_qk // 2], cache[..., d_qk // 2:]
        csa2.kv_fp4_quantize(kv_x, codes=codes, scales=scales)
    else:
        codes, scales = csa2.kv_fp4_quantize(kv_x)
    swa_x = inputs.normal_f32((B, W, d_qk), seed, 1, "swa", device="cuda")
    sv, ss = csa2.swa_fp8_quantize(swa_x) if W > 0 else (None, None)
    return kv_x, codes, scales, swa_x, sv, ss


def _oracle_decode(q, kv_x, idx, ctx, swa_x, swa_len, d_qk, d_v, scale, sink=None):
    B = q.shape[0]
    outs, lses = [], []
    for b in range(B):
        codes, scales = Q.fp4_quantize(kv_x[b])
        if swa_x is not None:
            sv, ss = Q.mxfp8_quantize(swa_x[b])
        else:
            sv = ss = None
        o, l = A.sparse_attn_decode_row(q[b], codes, scales, idx[b], ctx[b], sv, ss,
                                        0 if swa_len is None else swa_len[b], d_qk, d_v, scale, sink)
        outs.append(o)
        lses.append(l)
    return np.stack(outs), np.stack(lses)


def _check(out, lse, want_o, want_l):
    err = rowwise_rel_err(np_(out), want_o)
    assert err <= ATTN_TOL, err
    wl, gl = want_l, np_(lse)
    fin = np.isfinite(wl)
    assert np.array_equal(fin, np.isfinite(gl))
    assert np.max(np.abs(gl[fin] - wl[fin]), initial=0.0) <= LSE_TOL
    return err


@gpu
def test_tiny_config_decode_attention():
    require_gpu()
    wl = inputs.WORKLOADS["tiny"]
    announce("attn decode tiny H16 K256 W128")
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(wl.B, wl.N, wl.d_qk, wl.W, wl.seed)
    q = inputs.normal_f32((wl.B, wl.H, wl.d_qk), wl.seed, 0, "q", device="cuda")
    idx = inputs.random_index_lists(wl.B, wl.K, wl.N, wl.seed, device="cuda")
    ctx = torch.full((wl.B,), wl.N, dtype=torch.int32, device="cuda")
    swa_len = torch.full((wl.B,), wl.W, dtype=torch.int32, device="cuda")
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, wl.softmax_scale,
                                            want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), np_(swa_x), np_(swa_len),
                                    wl.d_qk, wl.d_v, wl.softmax_scale)
    _check(out, lse, want_o, want_l)


@gpu
@pytest.mark.parametrize("d_qk,H,K,W,n_invalid", [(576, 64, 2048, 128, 0), (576, 64, 300, 50, 40),
                                                  (512, 64, 512, 128, 7), (576, 32, 64, 0, 3),
                                                  (576, 48, 200, 17, 5), (512, 16, 33, 1, 0),
                                                  (576, 64, 0, 128, 0), (512, 32, 0, 128, 0)])
def test_decode_shapes_invalid_entries_and_ragged_windows(d_qk, H, K, W, n_invalid):
    require_gpu()
    announce(f"attn decode d_qk={d_qk} H={H} K={K} W={W} invalid={n_invalid}")
    B, N = 3, 5000
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(B, N, d_qk, W, 21, interleaved=(d_qk == 576))
    q = inputs.normal_f32((B, H, d_qk), 21, 2, "q", device="cuda")
    idx = inputs.random_index_lists(B, K, N, 21, device="cuda", n_invalid=n_invalid)
    ctx = torch.tensor([N, N - 1000, 4000], dtype=torch.int32, device="cuda")
    swa_len = torch.tensor([W, max(W - 3, 0), min(W, 1)], dtype=torch.int32, device="cuda") if W else None
    scale = 1.0 / np.sqrt(d_qk)
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, scale, want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), None if W == 0 else np_(swa_x),
                                    None if W == 0 else np_(swa_len), d_qk, 512, scale)
    _check(out, lse, want_o, want_l)


@gpu
def test_rising_scores_move_the_softmax_reference():
    """Entries ordered by rising head-0 score and a large softmax scale: the
    running maximum of that head moves by more than 2^8 (log2 units) in many
    chunks of a split, so the accumulated O is rescaled between chunks, and
    the other heads see random orders.  q takes quarter steps, exact in fp16,
    so at this scale the logits still meet the tolerance."""
    require_gpu()
    announce("attn decode rising scores B64 K1024 scale 0.5")
    B, N, d_qk, H, K = 64, 1100, 576, 64, 1024
    kv_x, codes, scales, _, _, _ = _make_caches(B, N, d_qk, 0, 31)
    q = (torch.round(inputs.normal_f32((B, H, d_qk), 31, 2, "q", device="cuda") * 4) / 4).contiguous()
    s0 = torch.bmm(kv_x, q[:, 0, :, None].contiguous()).squeeze(-1)
    idx = torch.argsort(s0, dim=1)[:, N - K:].to(torch.int32).contiguous()   # top K, ascending
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    scale = 0.5
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, None, None, None, scale, want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), None, None, d_qk, 512, scale)
    _check(out, lse, want_o, want_l)


@gpu
def test_topk_covering_context_is_dense_attention_and_sink():
    require_gpu()
    announce("attn decode K >= N (dense) with sink")
    B, N, d_qk, H, W = 2, 700, 576, 64, 128
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(B, N, d_qk, W, 22)
    q = inputs.normal_f32((B, H, d_qk), 22, 2, "q", device="cuda")
    idx = torch.arange(N, dtype=torch.int32, device="cuda").repeat(B, 1)
    idx = torch.cat([idx, torch.full((B, 68), -1, dtype=torch.int32, device="cuda")], dim=1).contiguous()
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    swa_len = torch.full((B,), W, dtype=torch.int32, device="cuda")
    sink = inputs.normal_f32((H,), 22, 3, "sink", device="cuda") * 3.0
    sink[0] = float("-inf")
    scale = 1.0 / np.sqrt(576.0)
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, scale, sink=sink,
                                            want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), np_(swa_x), np_(swa_len), d_qk, 512,
                                    scale, sink=np_(sink))
    _check(out, lse, want_o, want_l)


@gpu
def test_single_split_rows_normalise_in_place():
    """256 rows fill the chip with one workgroup each: a row's entries form a
    single split (several chunks), which writes the normalised output and lse
    itself; sink (one head without), invalid entries, ragged windows."""
    require_gpu()
    announce("attn decode 256 rows, single split per row, sink")
    B, N, d_qk, H, K, W = 256, 400, 576, 16, 200, 32
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(B, N, d_qk, W, 24)
    q = inputs.normal_f32((B, H, d_qk), 24, 2, "q", device="cuda")
    idx = inputs.random_index_lists(B, K, N, 24, device="cuda", n_invalid=9)
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    ctx[1::3] = N - 150
    swa_len = torch.arange(B, dtype=torch.int32, device="cuda") % (W + 1)
    sink = inputs.normal_f32((H,), 24, 3, "sink", device="cuda")
    sink[5] = float("-inf")
    scale = 1.0 / np.sqrt(576.0)
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, scale, sink=sink,
                                            want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), np_(swa_x), np_(swa_len), d_qk, 512,
                                    scale, sink=np_(sink))
    _check(out, lse, want_o, want_l)


@gpu
def test_empty_entry_sets():
    require_gpu()
    announce("attn decode empty entry sets")
    B, N, d_qk, H = 2, 100, 576, 16
    kv_x, codes, scales, _, _, _ = _make_caches(B, N, d_qk, 0, 23)
    q = inputs.normal_f32((B, H, d_qk), 23, 2, "q", device="cuda")
    idx = torch.full((B, 64), -1, dtype=torch.int32, device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    sink = torch.full((H,), 0.25, dtype=torch.float32, device="cuda")
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, None, None, None, 0.05, want_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, None, None, None, 0.05, sink=sink,
                                            want_lse=True)
    torch.cuda.synchronize()
    assert torch.all(out == 0) and torch.allclose(lse, torch.full_like(lse, 0.25))


@gpu
@pytest.mark.parametrize("K", [256, 0])
def test_prefill_attention_causal_windows(K):
    """Causal windows of nine consecutive queries, with Top-K rows and with
    the window alone (k_top = 0: up to 128 window rows, four chunks)."""
    require_gpu()
    announce(f"attn prefill B2 Tq=9 K={K} W=128")
    B, Tq, N0, d_qk, H, W = 2, 9, 3000, 576, 64, 128
    N = N0 + Tq
    kv_x, codes, scales, _, _, _ = _make_caches(B, N, d_qk, 0, 24)
    S = W - 1 + Tq
    swa_x = inputs.normal_f32((B, S, d_qk), 24, 1, "swa", device="cuda")
    sv, ss = csa2.swa_fp8_quantize(swa_x)
    q = inputs.normal_f32((B, Tq, H, d_qk), 24, 2, "q", device="cuda")
    idx = inputs.random_index_lists(B * Tq, K, N0, 24, device="cuda", n_invalid=5 if K else 0).reshape(B, Tq, K)
    idx = idx.contiguous()
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    q_pos = (torch.arange(Tq, dtype=torch.int32, device="cuda") + N0).repeat(B, 1).contiguous()
    swa_pos0 = torch.tensor([N0 - W + 1, N0 - W + 1], dtype=torch.int32, device="cuda")
    scale = 1.0 / np.sqrt(576.0)
    out, lse = csa2.csa2_sparse_attn_prefill(q, codes, scales, idx, ctx, q_pos, sv, ss, swa_pos0, W, scale,
                                             want_lse=True)
    torch.cuda.synchronize()
    kvh, svh, ssh = np_(kv_x), np_(sv), np_(ss)
    want_o = np.zeros((B, Tq, H, 512))
    want_l = np.zeros((B, Tq, H))
    for b in range(B):
        c, s = Q.fp4_quantize(kvh[b])
        v8, s8 = Q.mxfp8_quantize(np_(swa_x[b]))
        for t in range(Tq):
            want_o[b, t], want_l[b, t] = A.sparse_attn_prefill_row(np_(q[b, t]), c, s, np_(idx[b, t]), N,
                                                                   np_(q_pos)[b, t], v8, s8, np_(swa_pos0)[b], W,
                                                                   d_qk, 512, scale)
    _check(out, lse, want_o, want_l)


@gpu
def test_decode64k_attention_sampled_rows():
    """The 64 x 2048 (+128 window) attention of the benchmark configuration;
    rows 0 and 63 checked against the oracle."""
    require_gpu()
    wl = inputs.WORKLOADS["decode64k"]
    announce("attn decode decode64k full batch, rows 0/63 sampled")
    B, N = wl.B, 8192   # cache rows beyond the selected ids never enter attention
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(B, N, wl.d_qk, wl.W, wl.seed)
    q = inputs.normal_f32((B, wl.H, wl.d_qk), wl.seed, 0, "q", device="cuda")
    idx = inputs.random_index_lists(B, wl.K, N, wl.seed, device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    swa_len = torch.full((B,), wl.W, dtype=torch.int32, device="cuda")
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, wl.softmax_scale,
                                            want_lse=True)
    torch.cuda.synchronize()
    rows = [0, B - 1]
    want_o, want_l = _oracle_decode(np_(q[rows]), np_(kv_x[rows]), np_(idx[rows]), np_(ctx[rows]),
                                    np_(swa_x[rows]), np_(swa_len[rows]), wl.d_qk, wl.d_v, wl.softmax_scale)
    _check(out[rows], lse[rows], want_o, want_l)


# Documented accuracy range of the fp16 q: within ATTN_TOL up to 4x the
# configurations' logit spread; at larger spreads the error grows about
# linearly with softmax_scale * |q| |k| (2^-12 relative per logit) and is
# checked against that looser, documented bound.
SCALE_TOL = {1: ATTN_TOL, 4: ATTN_TOL, 12: 1e-2}


@gpu
@pytest.mark.parametrize("mult", [1, 4, 12])
def test_gaussian_q_at_larger_softmax_scales(mult):
    """Unrounded Gaussian q at 1, 4 and 12 times 1/sqrt(576): within 2e-3 up
    to 4x, within the documented 1e-2 at 12x (q's fp16 rounding moves each
    logit by ~scale * |q||k| * 2^-12)."""
    require_gpu()
    announce(f"attn decode Gaussian q, softmax scale {mult} / sqrt(576)")
    B, N, d_qk, H, K, W = 4, 6000, 576, 64, 2048, 128
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(B, N, d_qk, W, 41 + mult)
    q = inputs.normal_f32((B, H, d_qk), 41 + mult, 2, "q", device="cuda")
    idx = inputs.random_index_lists(B, K, N, 41 + mult, device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    swa_len = torch.full((B,), W, dtype=torch.int32, device="cuda")
    scale = mult / np.sqrt(576.0)
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, scale, want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), np_(swa_x), np_(swa_len), d_qk, 512,
                                    scale)
    err = rowwise_rel_err(np_(out), want_o)
    print(f"softmax scale x{mult}: max row relative error {err:.2e}")
    assert err <= SCALE_TOL[mult], err
    fin = np.isfinite(want_l)
    assert np.max(np.abs(np_(lse)[fin] - want_l[fin]), initial=0.0) <= (LSE_TOL if mult <= 4 else 1e-2)


@gpu
@pytest.mark.parametrize("code", [112, 134])
def test_window_rows_at_the_ends_of_the_exact_scale_range(code):
    """Window rows whose every 32-channel block gets the E8M0 code 112 (the
    smallest E4M3 step lands on fp16's smallest subnormal, 2^-24) or 134
    (448 * 2^7 stays below fp16's largest finite value): the conversion to
    fp16 is still exact, and attention over the window alone meets the
    tolerance."""
    require_gpu()
    announce(f"attn decode window only, E8M0 code {code}")
    B, N, d_qk, H, W = 2, 256, 576, 64, 128
    kv_x, codes, scales, _, _, _ = _make_caches(B, N, d_qk, 0, 51)
    base = inputs.normal_f32((B, W, d_qk), 51, 1, "swa", device="cuda")
    # amax of each block in [256, 480) * 2^(code - 127): the quantiser's code
    # floor(log2 amax) - 8 + 127 is then exactly `code`.
    blk = base.view(B, W, d_qk // 32, 32)
    amax = blk.abs().amax(-1, keepdim=True)
    blk = blk / amax * 300.0 * (2.0 ** (code - 127))
    swa_x = blk.reshape(B, W, d_qk).contiguous()
    sv, ss = csa2.swa_fp8_quantize(swa_x)
    assert bool((ss == code).all())
    q = inputs.normal_f32((B, H, d_qk), 51, 2, "q", device="cuda")
    idx = torch.full((B, 8), -1, dtype=torch.int32, device="cuda")
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    swa_len = torch.full((B,), W, dtype=torch.int32, device="cuda")
    scale = (1.0 / np.sqrt(576.0)) * (2.0 ** (127 - code)) / 300.0 * 8.0
    out, lse = csa2.csa2_sparse_attn_decode(q, codes, scales, idx, ctx, sv, ss, swa_len, scale, want_lse=True)
    torch.cuda.synchronize()
    want_o, want_l = _oracle_decode(np_(q), np_(kv_x), np_(idx), np_(ctx), np_(swa_x), np_(swa_len), d_qk, 512,
                                    scale)
    _check(out, lse, want_o, want_l)


@gpu
@pytest.mark.parametrize("B,rotate_q", [(3, True), (3, False), (300, True)])
def test_pages_row_with_fused_rope(B, rotate_q):
    """The pages' 512-wide K = V row with the rotary steps fused around the
    attention: q's last 64 channels rotated forward (or given rotated), the
    output's last 64 rotated back.  B = 3 runs several splits per row (the
    rotation in the combine), B = 300 one split per row (in the split kernel)."""
    require_gpu()
    announce(f"attn decode rope B={B} rotate_q={rotate_q}")
    N, d, H, K, W = 3000, 512, 64, 512, 128
    kv_x, codes, scales, swa_x, sv, ss = _make_caches(B, N, d, W, 101, interleaved=True)
    q = inputs.normal_f32((B, H, d), 101, 2, "q", device="cuda")
    idx = inputs.random_index_lists(B, K, N, 101, device="cuda", n_invalid=3)
    ctx = torch.full((B,), N, dtype=torch.int32, device="cuda")
    swa_len = torch.full((B,), W, dtype=torch.int32, device="cuda")
    theta = inputs.normal_f32((B, 32), 101, 3, "q", device="cuda") * 100.0
    rope_cs = torch.stack([torch.cos(theta), torch.sin(theta)], dim=-1).reshape(B, 64).contiguous()
    scale = 1 / np.sqrt(512.0)
    out, lse = csa2.csa2_sparse_attn_decode_rope(q, codes, scales, idx, ctx, sv, ss, swa_len, scale, rope_cs,
                                                 rotate_q=rotate_q, want_lse=True)
    torch.cuda.synchronize()
    qh, kvh, swh, idh, csh = np_(q), np_(kv_x), np_(swa_x), np_(idx), np_(rope_cs).reshape(B, 32, 2)
    rows = range(B) if B <= 8 else (0, 137, B - 1)
    want_o, want_l, got_o, got_l = [], [], [], []
    for b in rows:
        c_, s_ = Q.fp4_quantize(kvh[b])
        v8, s8 = Q.mxfp8_quantize(swh[b])
        o, l = A.sparse_attn_decode_rope_row(qh[b], c_, s_, idh[b], N, v8, s8, W, d, scale, csh[b], 64, rotate_q)
        want_o.append(o)
        want_l.append(l)
        got_o.append(np_(out[b]))
        got_l.append(np_(lse[b]))
    _check(torch.from_numpy(np.stack(got_o)), torch.from_numpy(np.stack(got_l)), np.stack(want_o), np.stack(want_l))
