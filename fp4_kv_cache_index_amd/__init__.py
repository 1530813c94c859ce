"""Python binding of libcsa2.so, the CSA2 hot path for MI355X (gfx950).

The functions below carry the C ABI's names and only marshal arguments:
they check dtypes/devices, allocate outputs and workspaces with torch, pass
raw device pointers, strides and the current HIP stream, and raise on a
non-zero status.  Every step of the path runs in the library's HIP kernels.
There is no fallback: importing works without a GPU (for inspection), but
any call needs the built library and a GPU tensor.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcsa2.so")

c_void_p, c_int32, c_int64, c_size_t, c_float = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                                ctypes.c_size_t, ctypes.c_float)

# (name, restype, argtypes) of every exported symbol of include/csa2.h.
_SIGS = {
    "csa2_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "csa2_version": (ctypes.c_char_p, []),
    "kv_fp4_quantize": (ctypes.c_int, [c_void_p, c_int64, c_int32, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                       c_void_p]),
    "swa_fp8_quantize": (ctypes.c_int, [c_void_p, c_int64, c_int32, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                        c_void_p]),
    "idx_mxfp4_quantize": (ctypes.c_int, [c_void_p, c_int64, c_int32, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                          c_void_p]),
    "csa2_index_score_topk_workspace_size": (c_size_t, [c_int32, c_int32, c_int64, c_int32, c_int32, c_int32]),
    "csa2_index_score_topk_workspace_size_stored": (c_size_t, [c_int32, c_int32, c_int64, c_int32, c_int32,
                                                               c_int32]),
    "csa2_index_score_topk": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                             c_int32, c_int32, c_int32, c_int32, c_int64, c_int32, c_void_p,
                                             c_void_p, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                                             c_void_p]),
    "csa2_index_score_topk_mxfp4": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                                                   c_int64, c_int64, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                                   c_int32, c_int64, c_int32, c_void_p, c_void_p, c_int32, c_int32,
                                                   c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa2_hier_pool_topk_mxfp4": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64,
                                                 c_int64, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_int32,
                                                 c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_size_t,
                                                 c_void_p]),
    "csa2_index_score_topk_noalloc": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                                                     c_void_p, c_int32, c_int32, c_int32, c_int32, c_int64, c_int32,
                                                     c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                                     c_void_p]),
    "csa2_hier_pool_topk_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "csa2_hier_pool_topk": (ctypes.c_int, [c_void_p, c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_void_p,
                                           c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p,
                                           c_void_p, c_size_t, c_void_p]),
    "csa2_sparse_attn_decode_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32]),
    "csa2_sparse_attn_decode": (ctypes.c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64,
                                               c_void_p, c_int32, c_void_p, c_void_p, c_int64, c_int64, c_void_p,
                                               c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int32, c_int32,
                                               c_int32, c_int32, c_float, c_void_p, c_void_p, c_void_p, c_size_t,
                                               c_void_p]),
    "csa2_sparse_attn_decode_rope": (ctypes.c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64,
                                                    c_int64, c_void_p, c_int32, c_void_p, c_void_p, c_int64, c_int64,
                                                    c_void_p, c_int64, c_int64, c_void_p, c_int32, c_void_p, c_int32,
                                                    c_int32, c_int32, c_float, c_void_p, c_int32, c_int32, c_void_p,
                                                    c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa2_sparse_attn_prefill_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "csa2_sparse_attn_prefill": (ctypes.c_int, [c_void_p, c_void_p, c_int64, c_int64, c_void_p, c_int64, c_int64,
                                                c_void_p, c_int32, c_void_p, c_void_p, c_void_p, c_int64, c_int64,
                                                c_void_p, c_int64, c_int64, c_void_p, c_int32, c_int32, c_void_p,
                                                c_int32, c_int32, c_int32, c_int32, c_int32, c_float, c_void_p,
                                                c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa2_sparse_attn_paged_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32, c_int32, c_int32]),
    "csa2_sparse_attn_paged": (ctypes.c_int, [c_void_p, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                              c_int32, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
                                              c_int64, c_int64, c_void_p, c_int64, c_int64, c_int32, c_void_p,
                                              c_int32, c_void_p, c_int32, c_int32, c_int32, c_int32, c_int32,
                                              c_float, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "csa2_trace_attach": (ctypes.c_int, [ctypes.POINTER(c_void_p), ctypes.POINTER(ctypes.c_char_p), c_int32]),
    "csa2_trace_only": (ctypes.c_int, [ctypes.c_char_p]),
    "csa2_trace_detach": (ctypes.c_int, [ctypes.POINTER(c_int32)]),
}
EXPORTS = tuple(_SIGS)

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m fp4_kv_cache_index_amd.build_lib` (there is no fallback path)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


class Csa2Error(RuntimeError):
    pass


def _check(status, what):
    if status != 0:
        msg = lib().csa2_status_string(status).decode()
        raise Csa2Error(f"{what}: status {status} ({msg})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _gpu(t, name, dtype=None):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _workspace(nbytes, device, ws=None):
    """A 256-byte aligned device buffer of nbytes (uses `ws` when large enough)."""
    if ws is not None:
        _gpu(ws, "workspace", torch.uint8)
        if ws.numel() >= nbytes and ws.data_ptr() % 256 == 0:
            return ws, ws.numel()
    buf = torch.empty(max(int(nbytes), 1) + 256, dtype=torch.uint8, device=device)
    off = (-buf.data_ptr()) % 256
    return buf[off:off + max(int(nbytes), 1)], max(int(nbytes), 1)


def _row_strides(t, name):
    """(batch stride, row stride) in bytes of a [B][rows][bytes] uint8 view."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError(f"{name} must be [B][rows][bytes] with unit inner stride")
    return t.stride(0) * t.element_size(), t.stride(1) * t.element_size()


# ------------------------------------------------------------ cache writers ---

def kv_fp4_quantize(x, codes=None, scales=None):
    """FP4 main-KV write of float32 rows x [..., d] -> (codes [..., d/2] u8, scales [..., d/16] u8)."""
    _gpu(x, "x", torch.float32)
    d = x.shape[-1]
    x2 = x.reshape(-1, d)
    if x2.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    lead = x.shape[:-1]
    if codes is None:
        codes = torch.empty(*lead, d // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*lead, d // 16, dtype=torch.uint8, device=x.device)
    c2, s2 = codes.view(-1, codes.shape[-1]), scales.view(-1, scales.shape[-1])
    _check(lib().kv_fp4_quantize(_ptr(x2), x2.shape[0], d, x2.stride(0), _ptr(c2), c2.stride(0), _ptr(s2),
                                 s2.stride(0), _stream(x.device)), "kv_fp4_quantize")
    return codes, scales


def swa_fp8_quantize(x, vals=None, scales=None):
    """Sliding-window write of float32 rows x [..., d] -> (vals [..., d] E4M3 u8, scales [..., d/32] E8M0 u8)."""
    _gpu(x, "x", torch.float32)
    d = x.shape[-1]
    x2 = x.reshape(-1, d)
    if x2.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    lead = x.shape[:-1]
    if vals is None:
        vals = torch.empty(*lead, d, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*lead, d // 32, dtype=torch.uint8, device=x.device)
    v2, s2 = vals.view(-1, vals.shape[-1]), scales.view(-1, scales.shape[-1])
    _check(lib().swa_fp8_quantize(_ptr(x2), x2.shape[0], d, x2.stride(0), _ptr(v2), v2.stride(0), _ptr(s2),
                                  s2.stride(0), _stream(x.device)), "swa_fp8_quantize")
    return vals, scales


def idx_mxfp4_quantize(x, codes=None, scales=None):
    """MXFP4 indexer-K write of float32 rows x [..., d] -> (codes [..., d/2] u8, scales [..., d/32] u8 E8M0)."""
    _gpu(x, "x", torch.float32)
    d = x.shape[-1]
    x2 = x.reshape(-1, d)
    if x2.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    lead = x.shape[:-1]
    if codes is None:
        codes = torch.empty(*lead, d // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(*lead, d // 32, dtype=torch.uint8, device=x.device)
    c2, s2 = codes.view(-1, codes.shape[-1]), scales.view(-1, scales.shape[-1])
    _check(lib().idx_mxfp4_quantize(_ptr(x2), x2.shape[0], d, x2.stride(0), _ptr(c2), c2.stride(0), _ptr(s2),
                                    s2.stride(0), _stream(x.device)), "idx_mxfp4_quantize")
    return codes, scales


# ----------------------------------------------------------- indexer + topk ---

def csa2_index_score_topk_workspace_size(B, Tq, n_max, k_top, pool_block=0, pool_nblocks=0):
    return lib().csa2_index_score_topk_workspace_size(B, Tq, n_max, k_top, pool_block, pool_nblocks)


def csa2_index_score_topk_workspace_size_stored(B, Tq, n_max, k_top, pool_block=0, pool_nblocks=0):
    return lib().csa2_index_score_topk_workspace_size_stored(B, Tq, n_max, k_top, pool_block, pool_nblocks)


def _index_ws(B, Tq, n_max, k_top, pool_block, pool_nblocks, stored, dev, workspace):
    """The indexer's workspace: a given one is used when it holds at least
    the default size (its size then picks the prefill selection)."""
    need = csa2_index_score_topk_workspace_size(B, Tq, n_max, k_top, pool_block, pool_nblocks)
    if stored:
        need = max(need, csa2_index_score_topk_workspace_size_stored(B, Tq, n_max, k_top, pool_block, pool_nblocks))
    return _workspace(need, dev, workspace)


def csa2_index_score_topk(q_idx, w, k_idx, ctx_len, k_top, q_pos=None, pool_block=0, pool_nblocks=0,
                          want_scores=False, workspace=None, out=None, stored_keys=False):
    """Indexer scores + exact Top-K (and optionally the hierarchical pool).

    stored_keys: allocate csa2_index_score_topk_workspace_size_stored() bytes
    (dense prefill chunks then store their score keys and select in one
    scoring pass instead of selecting by scoring passes).

    q_idx [B][Tq][H_I][D_I] u8 (E4M3), w [B][Tq][H_I] f32, k_idx [B][N][D_I] u8
    (any batch/row strides), ctx_len [B] i32, q_pos [B][Tq] i32 or None.
    Returns dict(topk_idx [B][Tq][k_top] i32, topk_score or None,
    pool_idx [B][Tq][nblocks*block] i32 or None, pool_len [B][Tq] i32 or None).
    """
    _gpu(q_idx, "q_idx", torch.uint8)
    _gpu(w, "w", torch.float32)
    _gpu(k_idx, "k_idx", torch.uint8)
    _gpu(ctx_len, "ctx_len", torch.int32)
    B, Tq, H_I, D_I = q_idx.shape
    if not q_idx.is_contiguous() or not w.is_contiguous() or tuple(w.shape) != (B, Tq, H_I):
        raise ValueError("q_idx / w must be contiguous [B][Tq][H_I][D_I] / [B][Tq][H_I]")
    kb, kr = _row_strides(k_idx, "k_idx")
    n_max = k_idx.shape[1]
    if q_pos is not None:
        _gpu(q_pos, "q_pos", torch.int32)
        if not q_pos.is_contiguous() or tuple(q_pos.shape) != (B, Tq):
            raise ValueError("q_pos must be contiguous [B][Tq]")
    dev = q_idx.device
    out = out or {}
    topk_idx = out.get("topk_idx")
    if topk_idx is None:
        topk_idx = torch.empty(B, Tq, k_top, dtype=torch.int32, device=dev)
    topk_score = out.get("topk_score")
    if want_scores and topk_score is None:
        topk_score = torch.empty(B, Tq, k_top, dtype=torch.float32, device=dev)
    pool_idx = pool_len = None
    if pool_nblocks > 0:
        pool_idx = out.get("pool_idx")
        if pool_idx is None:
            pool_idx = torch.empty(B, Tq, pool_nblocks * pool_block, dtype=torch.int32, device=dev)
        pool_len = out.get("pool_len")
        if pool_len is None:
            pool_len = torch.empty(B, Tq, dtype=torch.int32, device=dev)
    ws, ws_bytes = _index_ws(B, Tq, n_max, k_top, pool_block, pool_nblocks, stored_keys, dev, workspace)
    _check(lib().csa2_index_score_topk(_ptr(q_idx), _ptr(w), _ptr(k_idx), kb, kr, _ptr(ctx_len), _ptr(q_pos), B, Tq,
                                       H_I, D_I, n_max, k_top, _ptr(topk_idx), _ptr(topk_score), pool_block,
                                       pool_nblocks, _ptr(pool_idx), _ptr(pool_len), _ptr(ws), ws_bytes,
                                       _stream(dev)), "csa2_index_score_topk")
    return {"topk_idx": topk_idx, "topk_score": topk_score, "pool_idx": pool_idx, "pool_len": pool_len}


def _mx_keys(k_codes, k_scales):
    _gpu(k_codes, "k_codes", torch.uint8)
    _gpu(k_scales, "k_scales", torch.uint8)
    cb, cr = _row_strides(k_codes, "k_codes")
    sb, sr = _row_strides(k_scales, "k_scales")
    return cb, cr, sb, sr


def csa2_index_score_topk_mxfp4(q_idx, w, k_codes, k_scales, ctx_len, k_top, q_pos=None, pool_block=0,
                                pool_nblocks=0, want_scores=False, workspace=None, out=None,
                                stored_keys=False):
    """csa2_index_score_topk over MXFP4 keys: k_codes [B][N][D_I/2] u8, k_scales [B][N][D_I/32] u8 (E8M0)."""
    _gpu(q_idx, "q_idx", torch.uint8)
    _gpu(w, "w", torch.float32)
    _gpu(ctx_len, "ctx_len", torch.int32)
    B, Tq, H_I, D_I = q_idx.shape
    if not q_idx.is_contiguous() or not w.is_contiguous() or tuple(w.shape) != (B, Tq, H_I):
        raise ValueError("q_idx / w must be contiguous [B][Tq][H_I][D_I] / [B][Tq][H_I]")
    cb, cr, sb, sr = _mx_keys(k_codes, k_scales)
    n_max = k_codes.shape[1]
    if q_pos is not None:
        _gpu(q_pos, "q_pos", torch.int32)
    dev = q_idx.device
    out = out or {}
    topk_idx = out.get("topk_idx")
    if topk_idx is None:
        topk_idx = torch.empty(B, Tq, k_top, dtype=torch.int32, device=dev)
    topk_score = out.get("topk_score")
    if want_scores and topk_score is None:
        topk_score = torch.empty(B, Tq, k_top, dtype=torch.float32, device=dev)
    pool_idx = pool_len = None
    if pool_nblocks > 0:
        pool_idx = out.get("pool_idx")
        if pool_idx is None:
            pool_idx = torch.empty(B, Tq, pool_nblocks * pool_block, dtype=torch.int32, device=dev)
        pool_len = out.get("pool_len")
        if pool_len is None:
            pool_len = torch.empty(B, Tq, dtype=torch.int32, device=dev)
    ws, ws_bytes = _index_ws(B, Tq, n_max, k_top, pool_block, pool_nblocks, stored_keys, dev, workspace)
    _check(lib().csa2_index_score_topk_mxfp4(_ptr(q_idx), _ptr(w), _ptr(k_codes), cb, cr, _ptr(k_scales), sb, sr,
                                             _ptr(ctx_len), _ptr(q_pos), B, Tq, H_I, D_I, n_max, k_top,
                                             _ptr(topk_idx), _ptr(topk_score), pool_block, pool_nblocks,
                                             _ptr(pool_idx), _ptr(pool_len), _ptr(ws), ws_bytes, _stream(dev)),
           "csa2_index_score_topk_mxfp4")
    return {"topk_idx": topk_idx, "topk_score": topk_score, "pool_idx": pool_idx, "pool_len": pool_len}


def csa2_hier_pool_topk_mxfp4(q_idx, w, k_codes, k_scales, pool_idx, pool_len, k_top, ctx_len=None,
                              want_scores=False, workspace=None, out=None):
    """csa2_hier_pool_topk over MXFP4 keys (arrays as in csa2_index_score_topk_mxfp4)."""
    _gpu(q_idx, "q_idx", torch.uint8)
    _gpu(w, "w", torch.float32)
    _gpu(pool_idx, "pool_idx", torch.int32)
    _gpu(pool_len, "pool_len", torch.int32)
    B, Tq, H_I, D_I = q_idx.shape
    cb, cr, sb, sr = _mx_keys(k_codes, k_scales)
    pool_cap = pool_idx.shape[-1]
    dev = q_idx.device
    if ctx_len is None:
        ctx_len = torch.full((B,), k_codes.shape[1], dtype=torch.int32, device=dev)
    _gpu(ctx_len, "ctx_len", torch.int32)
    out = out or {}
    topk_idx = out.get("topk_idx")
    if topk_idx is None:
        topk_idx = torch.empty(B, Tq, k_top, dtype=torch.int32, device=dev)
    topk_score = out.get("topk_score")
    if want_scores and topk_score is None:
        topk_score = torch.empty(B, Tq, k_top, dtype=torch.float32, device=dev)
    need = csa2_hier_pool_topk_workspace_size(B, Tq, pool_cap, k_top)
    ws, ws_bytes = _workspace(need, dev, workspace)
    _check(lib().csa2_hier_pool_topk_mxfp4(_ptr(q_idx), _ptr(w), _ptr(k_codes), cb, cr, _ptr(k_scales), sb, sr,
                                           _ptr(ctx_len), _ptr(pool_idx), _ptr(pool_len), pool_cap, B, Tq, H_I,
                                           D_I, k_top, _ptr(topk_idx), _ptr(topk_score), _ptr(ws), ws_bytes,
                                           _stream(dev)), "csa2_hier_pool_topk_mxfp4")
    return {"topk_idx": topk_idx, "topk_score": topk_score}


def csa2_hier_pool_topk_workspace_size(B, Tq, pool_cap, k_top):
    return lib().csa2_hier_pool_topk_workspace_size(B, Tq, pool_cap, k_top)


def csa2_hier_pool_topk(q_idx, w, k_idx, pool_idx, pool_len, k_top, ctx_len=None, want_scores=False,
                        workspace=None, out=None):
    """Later hierarchical layer: Top-K over the pool tokens only.

    pool_idx [B][Tq][pool_cap] i32 ascending token ids, pool_len [B][Tq] i32,
    ctx_len [B] i32 (default: every sequence holds k_idx.shape[1] rows); pool
    ids outside [0, ctx_len[b]) are skipped.
    Returns dict(topk_idx [B][Tq][k_top], topk_score or None).
    """
    _gpu(q_idx, "q_idx", torch.uint8)
    _gpu(w, "w", torch.float32)
    _gpu(k_idx, "k_idx", torch.uint8)
    _gpu(pool_idx, "pool_idx", torch.int32)
    _gpu(pool_len, "pool_len", torch.int32)
    B, Tq, H_I, D_I = q_idx.shape
    if not (q_idx.is_contiguous() and w.is_contiguous() and pool_idx.is_contiguous() and pool_len.is_contiguous()):
        raise ValueError("q_idx, w, pool_idx and pool_len must be contiguous")
    pool_cap = pool_idx.shape[-1]
    kb, kr = _row_strides(k_idx, "k_idx")
    dev = q_idx.device
    if ctx_len is None:
        ctx_len = torch.full((B,), k_idx.shape[1], dtype=torch.int32, device=dev)
    _gpu(ctx_len, "ctx_len", torch.int32)
    out = out or {}
    topk_idx = out.get("topk_idx")
    if topk_idx is None:
        topk_idx = torch.empty(B, Tq, k_top, dtype=torch.int32, device=dev)
    topk_score = out.get("topk_score")
    if want_scores and topk_score is None:
        topk_score = torch.empty(B, Tq, k_top, dtype=torch.float32, device=dev)
    need = csa2_hier_pool_topk_workspace_size(B, Tq, pool_cap, k_top)
    ws, ws_bytes = _workspace(need, dev, workspace)
    _check(lib().csa2_hier_pool_topk(_ptr(q_idx), _ptr(w), _ptr(k_idx), kb, kr, _ptr(ctx_len), _ptr(pool_idx), _ptr(pool_len),
                                     pool_cap, B, Tq, H_I, D_I, k_top, _ptr(topk_idx), _ptr(topk_score), _ptr(ws),
                                     ws_bytes, _stream(dev)), "csa2_hier_pool_topk")
    return {"topk_idx": topk_idx, "topk_score": topk_score}


# -------------------------------------------------------------- attention ---

def _attn_caches(kv_codes, kv_scales, swa_vals, swa_scales):
    _gpu(kv_codes, "kv_codes", torch.uint8)
    _gpu(kv_scales, "kv_scales", torch.uint8)
    cb, cr = _row_strides(kv_codes, "kv_codes")
    sb, sr = _row_strides(kv_scales, "kv_scales")
    if swa_vals is not None:
        _gpu(swa_vals, "swa_vals", torch.uint8)
        _gpu(swa_scales, "swa_scales", torch.uint8)
        vb, vr = _row_strides(swa_vals, "swa_vals")
        xb, xr = _row_strides(swa_scales, "swa_scales")
    else:
        vb = vr = xb = xr = 0
    return cb, cr, sb, sr, vb, vr, xb, xr


def csa2_sparse_attn_decode_workspace_size(B, H, d_v, k_top, W):
    return lib().csa2_sparse_attn_decode_workspace_size(B, H, d_v, k_top, W)


def csa2_sparse_attn_decode(q, kv_codes, kv_scales, topk_idx, ctx_len, swa_vals, swa_scales, swa_len,
                            softmax_scale, d_v=512, sink=None, want_lse=False, workspace=None, out=None, lse=None):
    """Sparse decode attention.  q [B][H][d_qk] f32; kv_codes [B][N][d_qk/2] u8 and
    kv_scales [B][N][d_qk/16] u8 (views of one interleaved cache are fine);
    topk_idx [B][K] i32; swa_vals [B][W][d_qk] u8, swa_scales [B][W][d_qk/32] u8,
    swa_len [B] i32 (or all None for no window).  Returns (out [B][H][d_v], lse or None).
    """
    _gpu(q, "q", torch.float32)
    _gpu(topk_idx, "topk_idx", torch.int32)
    _gpu(ctx_len, "ctx_len", torch.int32)
    if not q.is_contiguous() or not topk_idx.is_contiguous():
        raise ValueError("q and topk_idx must be contiguous")
    B, H, d_qk = q.shape
    k_top = topk_idx.shape[-1]
    W = 0 if swa_vals is None else swa_vals.shape[1]
    if sink is not None:
        _gpu(sink, "sink", torch.float32)
    cb, cr, sb, sr, vb, vr, xb, xr = _attn_caches(kv_codes, kv_scales, swa_vals, swa_scales)
    dev = q.device
    if out is None:
        out = torch.empty(B, H, d_v, dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    need = csa2_sparse_attn_decode_workspace_size(B, H, d_v, k_top, W)
    ws, ws_bytes = _workspace(need, dev, workspace)
    _check(lib().csa2_sparse_attn_decode(_ptr(q), _ptr(kv_codes), cb, cr, _ptr(kv_scales), sb, sr, _ptr(topk_idx),
                                         k_top, _ptr(ctx_len), _ptr(swa_vals), vb, vr, _ptr(swa_scales), xb, xr,
                                         _ptr(swa_len), W, _ptr(sink), B, H, d_qk, d_v, float(softmax_scale),
                                         _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(dev)),
           "csa2_sparse_attn_decode")
    return out, lse


def csa2_sparse_attn_decode_rope(q, kv_codes, kv_scales, topk_idx, ctx_len, swa_vals, swa_scales, swa_len,
                                 softmax_scale, rope_cs, rotate_q=False, sink=None, want_lse=False, workspace=None,
                                 out=None, lse=None):
    """Decode attention over the pages' 512-wide K = V row with fused RoPE:
    rope_cs [B][rope_dim] f32 = (cos, sin) per channel pair of the last rope_dim
    channels; q's rotary channels rotated forward when rotate_q, the output's
    rotated back.  Other arguments as csa2_sparse_attn_decode.  Returns (out, lse)."""
    _gpu(q, "q", torch.float32)
    _gpu(topk_idx, "topk_idx", torch.int32)
    _gpu(ctx_len, "ctx_len", torch.int32)
    _gpu(rope_cs, "rope_cs", torch.float32)
    if not (q.is_contiguous() and topk_idx.is_contiguous() and rope_cs.is_contiguous()):
        raise ValueError("q, topk_idx and rope_cs must be contiguous")
    B, H, d = q.shape
    rope_dim = rope_cs.shape[-1]
    k_top = topk_idx.shape[-1]
    W = 0 if swa_vals is None else swa_vals.shape[1]
    if sink is not None:
        _gpu(sink, "sink", torch.float32)
    cb, cr, sb, sr, vb, vr, xb, xr = _attn_caches(kv_codes, kv_scales, swa_vals, swa_scales)
    dev = q.device
    if out is None:
        out = torch.empty(B, H, d, dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty(B, H, dtype=torch.float32, device=dev)
    need = csa2_sparse_attn_decode_workspace_size(B, H, d, k_top, W)
    ws, ws_bytes = _workspace(need, dev, workspace)
    _check(lib().csa2_sparse_attn_decode_rope(_ptr(q), _ptr(kv_codes), cb, cr, _ptr(kv_scales), sb, sr,
                                              _ptr(topk_idx), k_top, _ptr(ctx_len), _ptr(swa_vals), vb, vr,
                                              _ptr(swa_scales), xb, xr, _ptr(swa_len), W, _ptr(sink), B, H, d,
                                              float(softmax_scale), _ptr(rope_cs), rope_dim, int(bool(rotate_q)),
                                              _ptr(out), _ptr(lse), _ptr(ws), ws_bytes, _stream(dev)),
           "csa2_sparse_attn_decode_rope")
    return out, lse


def csa2_sparse_attn_prefill_workspace_size(B, Tq, H, d_v, k_top, W):
    return lib().csa2_sparse_attn_prefill_workspace_size(B, Tq, H, d_v, k_top, W)


def csa2_sparse_attn_prefill(q, kv_codes, kv_scales, topk_idx, ctx_len, q_pos, swa_vals, swa_scales, swa_pos0, W,
                             softmax_scale, d_v=512, sink=None, want_lse=False, workspace=None, out=None, lse=None):
    """Sparse attention of a causal chunk.  q [B][Tq][H][d_qk]; topk_idx [B][Tq][K];
    q_pos [B][Tq]; swa_vals [B][S][d_qk] / swa_scales [B][S][d_qk/32] with row i
    at position swa_pos0[b] + i; W the window.  Returns (out [B][Tq][H][d_v], lse)."""
    _gpu(q, "q", torch.float32)
    _gpu(topk_idx, "topk_idx", torch.int32)
    _gpu(ctx_len, "ctx_len", torch.int32)
    _gpu(q_pos, "q_pos", torch.int32)
    if not (q.is_contiguous() and topk_idx.is_contiguous() and q_pos.is_contiguous()):
        raise ValueError("q, topk_idx and q_pos must be contiguous")
    B, Tq, H, d_qk = q.shape
    k_top = topk_idx.shape[-1]
    swa_rows = 0 if swa_vals is None else swa_vals.shape[1]
    if sink is not None:
        _gpu(sink, "sink", torch.float32)
    cb, cr, sb, sr, vb, vr, xb, xr = _attn_caches(kv_codes, kv_scales, swa_vals, swa_scales)
    dev = q.device
    if out is None:
        out = torch.empty(B, Tq, H, d_v, dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev)
    need = csa2_sparse_attn_prefill_workspace_size(B, Tq, H, d_v, k_top, W)
    ws, ws_bytes = _workspace(need, dev, workspace)
    _check(lib().csa2_sparse_attn_prefill(_ptr(q), _ptr(kv_codes), cb, cr, _ptr(kv_scales), sb, sr, _ptr(topk_idx),
                                          k_top, _ptr(ctx_len), _ptr(q_pos), _ptr(swa_vals), vb, vr,
                                          _ptr(swa_scales), xb, xr, _ptr(swa_pos0), swa_rows, W, _ptr(sink), B, Tq,
                                          H, d_qk, d_v, float(softmax_scale), _ptr(out), _ptr(lse), _ptr(ws),
                                          ws_bytes, _stream(dev)), "csa2_sparse_attn_prefill")
    return out, lse


def csa2_sparse_attn_paged_workspace_size(B, Tq, H, d_v, k_top, W):
    return lib().csa2_sparse_attn_paged_workspace_size(B, Tq, H, d_v, k_top, W)


def csa2_sparse_attn_paged(q, pool_codes, pool_scales, block_table, page_size, topk_idx, ctx_len, q_pos, ring_vals,
                           ring_scales, swa_end, W, softmax_scale, d_v=512, sink=None, want_lse=False,
                           workspace=None, out=None, lse=None):
    """Attention over a paged main cache and ring windows.

    q [B][Tq][H][d_qk] f32; pool_codes [rows][d_qk/2] u8 and pool_scales
    [rows][d_qk/16] u8 (the page pool, rows = n_pages * page_size; views of one
    interleaved pool are fine); block_table [B][max_pages] i32; topk_idx
    [B][Tq][K] i32 token ids; q_pos [B][Tq] i32 (None when Tq == 1);
    ring_vals [B][R][d_qk] u8, ring_scales [B][R][d_qk/32] u8, swa_end [B] i32
    (or all None for no window).  Returns (out [B][Tq][H][d_v], lse or None).
    """
    _gpu(q, "q", torch.float32)
    _gpu(pool_codes, "pool_codes", torch.uint8)
    _gpu(pool_scales, "pool_scales", torch.uint8)
    _gpu(block_table, "block_table", torch.int32)
    _gpu(topk_idx, "topk_idx", torch.int32)
    _gpu(ctx_len, "ctx_len", torch.int32)
    if not (q.is_contiguous() and topk_idx.is_contiguous() and block_table.is_contiguous()):
        raise ValueError("q, topk_idx and block_table must be contiguous")
    if pool_codes.dim() != 2 or pool_codes.stride(1) != 1 or pool_scales.dim() != 2 or pool_scales.stride(1) != 1:
        raise ValueError("pool_codes / pool_scales must be [rows][bytes] with unit inner stride")
    B, Tq, H, d_qk = q.shape
    k_top = topk_idx.shape[-1]
    n_rows = pool_codes.shape[0]
    if n_rows % page_size:
        raise ValueError("the pool must hold whole pages")
    if q_pos is not None:
        _gpu(q_pos, "q_pos", torch.int32)
    if ring_vals is not None:
        _gpu(ring_vals, "ring_vals", torch.uint8)
        _gpu(ring_scales, "ring_scales", torch.uint8)
        _gpu(swa_end, "swa_end", torch.int32)
        vb, vr = _row_strides(ring_vals, "ring_vals")
        xb, xr = _row_strides(ring_scales, "ring_scales")
        R = ring_vals.shape[1]
    else:
        vb = vr = xb = xr = 0
        R = 0
        W = 0
    if sink is not None:
        _gpu(sink, "sink", torch.float32)
    dev = q.device
    if out is None:
        out = torch.empty(B, Tq, H, d_v, dtype=torch.float32, device=dev)
    if want_lse and lse is None:
        lse = torch.empty(B, Tq, H, dtype=torch.float32, device=dev)
    need = csa2_sparse_attn_paged_workspace_size(B, Tq, H, d_v, k_top, W)
    ws, ws_bytes = _workspace(need, dev, workspace)
    _check(lib().csa2_sparse_attn_paged(_ptr(q), _ptr(pool_codes), pool_codes.stride(0), _ptr(pool_scales),
                                        pool_scales.stride(0), _ptr(block_table), block_table.stride(0), page_size,
                                        n_rows // page_size, _ptr(topk_idx), k_top, _ptr(ctx_len), _ptr(q_pos),
                                        _ptr(ring_vals), vb, vr, _ptr(ring_scales), xb, xr, R, _ptr(swa_end), W,
                                        _ptr(sink), B, Tq, H, d_qk, d_v, float(softmax_scale), _ptr(out),
                                        _ptr(lse), _ptr(ws), ws_bytes, _stream(dev)), "csa2_sparse_attn_paged")
    return out, lse


# ------------------------------------------------------------------ tracing ---

class KernelTrace:
    """Per-kernel HIP-event timing of the library's launches on this thread.

    with KernelTrace(capacity) as tr: ...launch...; then tr.durations_ms()
    returns [(kernel name, ms)] after the stream has been synchronised.
    only="name" records just the launches of that kernel (two events per
    launch instead of two per library launch).
    """

    # hipEventDisableSystemFence: the events only carry timestamps, so they
    # need no system-scope acquire / release around the timed dispatch (with
    # it, each traced launch paid an L2 write-back inside its own timing and
    # a gap of several microseconds before the next kernel).
    EVENT_FLAGS = 0x20000000

    def __init__(self, capacity=4096, only=None, flags=None):
        self.capacity = capacity
        self.only = only
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(c_void_p), ctypes.c_uint]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), c_void_p, c_void_p]
        self._hip.hipEventDestroy.argtypes = [c_void_p]
        fl = self.EVENT_FLAGS if flags is None else flags
        self.events = (c_void_p * (2 * capacity))()
        for i in range(2 * capacity):
            e = c_void_p()
            if self._hip.hipEventCreateWithFlags(ctypes.byref(e), fl) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.events[i] = e
        self.names = (ctypes.c_char_p * capacity)()
        self.count = 0

    def __enter__(self):
        _check(lib().csa2_trace_attach(self.events, self.names, self.capacity), "csa2_trace_attach")
        if self.only is not None:
            _check(lib().csa2_trace_only(self.only.encode()), "csa2_trace_only")
        return self

    def __exit__(self, *exc):
        n = c_int32()
        lib().csa2_trace_detach(ctypes.byref(n))
        self.count = n.value
        return False

    def durations_ms(self):
        res = []
        for i in range(min(self.count, self.capacity)):
            ms = ctypes.c_float()
            if self._hip.hipEventElapsedTime(ctypes.byref(ms), self.events[2 * i], self.events[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            res.append((self.names[i].decode(), ms.value))
        return res

    def close(self):
        for i in range(2 * self.capacity):
            self._hip.hipEventDestroy(self.events[i])
        self.capacity = 0
