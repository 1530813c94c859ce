"""Seeded synthetic inputs and the workload shapes.

This module draws random numbers and describes shapes.  It holds none of the
path's arithmetic (no quantiser, no scoring, no selection, no attention), so
the test suite can feed the same inputs to the HIP library and to the CPU
checker.  Every tensor comes from a torch.Generator seeded from
(workload seed, layer, role); on a GPU device the draw uses that device's
generator, so a check on the CPU copies the drawn inputs to the host.

Value recipes (the pages' workloads are long-context decode/prefill of the
DeepSeek-V4.1-Flash CSA2 layers; no dataset is involved):
  * latent KV rows and window rows: float32 N(0, 1), d_qk channels;
  * indexer queries and keys: integers uniform in [-4, 4] stored as E4M3
    bytes (exact, via torch's float8_e4m3fn cast of small integers); MXFP4
    indexer keys are float32 N(0, 1) rows written by the library's MXFP4
    quantiser;
  * indexer head weights: float32 N(0, 1);
  * attention queries: float32 N(0, 1);
  * every sequence has the full context (ctx_len = N) and a full window.
"""

from dataclasses import dataclass, field

import torch

ROLE = {
    "kv": 1, "k_idx": 2, "q_idx": 3, "w": 4, "q": 5, "swa": 6, "sink": 7,
}


def _gen(seed, layer, role, device):
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) * 1_000_003 + int(layer) * 10_007 + ROLE[role]) & 0x7FFF_FFFF_FFFF)
    return g


def normal_f32(shape, seed, layer, role, device="cpu"):
    g = _gen(seed, layer, role, device)
    return torch.randn(*shape, generator=g, device=device, dtype=torch.float32)


def int_e4m3(shape, seed, layer, role, lo=-4, hi=4, device="cpu"):
    """E4M3 bytes of integers drawn uniformly from [lo, hi] (exactly representable)."""
    g = _gen(seed, layer, role, device)
    v = torch.randint(lo, hi + 1, shape, generator=g, device=device, dtype=torch.int32)
    return v.to(torch.float32).to(torch.float8_e4m3fn).view(torch.uint8)


@dataclass
class Workload:
    name: str
    seed: int
    B: int            # sequences
    N: int            # context tokens per sequence
    H: int            # attention query heads
    d_qk: int         # latent row width (nope + rope)
    d_v: int          # value width (first d_v channels of the row)
    H_I: int          # indexer heads
    D_I: int          # indexer head dim
    K: int            # Top-K
    W: int = 128      # sliding window
    Tq: int = 1       # query tokens per sequence
    layers: list = field(default_factory=lambda: ["full"])
    pool_block: int = 0
    pool_nblocks: int = 0
    softmax_scale: float = 0.0
    page_size: int = 0   # > 0: main rows in a page pool (random page order), window in a ring
    m: int = 1           # tokens per cache entry (2: the encoder layers' compressed entries); N counts entries
    mxfp4: bool = False  # indexer keys in the pages' MXFP4 format (float32 N(0,1) rows quantised), not E4M3 integers
    rope: bool = False   # fused RoPE around attention (the pages' K = V row: d_qk = d_v = 512)

    def __post_init__(self):
        if self.softmax_scale == 0.0:
            self.softmax_scale = 1.0 / (576.0 ** 0.5)


# The five measured/parity workloads.
WORKLOADS = {
    "tiny": Workload("tiny: B1 x 4096 ctx, Full, 16 heads, indexer 4x64, top-256", 0,
                     B=1, N=4096, H=16, d_qk=576, d_v=512, H_I=4, D_I=64, K=256),
    "decode64k": Workload("decode: B64 x 64K ctx, Full, 64 heads, indexer 8x128, top-2048", 1,
                          B=64, N=65536, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048),
    "group128k": Workload("group: B16 x 128K ctx, Full -> Reindex -> Reuse, top-2048", 2,
                          B=16, N=131072, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048,
                          layers=["full", "reindex", "reuse"]),
    "hier1m": Workload("hierarchical: B4 x 1M ctx, Full + 9 pool layers, pool 2048x8, top-2048", 3,
                       B=4, N=1 << 20, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048,
                       layers=["full"] + ["pool"] * 9, pool_block=8, pool_nblocks=2048),
    "prefill256k": Workload("prefill: B1, 4096 new tokens on 256K ctx, causal, top-2048", 4,
                            B=1, N=262144 + 4096, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048,
                            Tq=4096),
    # Multi-query decode (speculative verification): two query tokens per
    # sequence, scored in one pass over the key cache.
    "mq2_64k": Workload("multi-query decode: B64 x 64K ctx, 2 query tokens per sequence, Full, 64 heads, "
                        "indexer 8x128, top-2048", 6,
                        B=64, N=65536, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048, Tq=2),
    # Encoder-side CSA2: one cache entry per two tokens (128K tokens -> 64K
    # entries), a group of one Full layer and five Reuse layers.
    "enc128k": Workload("encoder group: B16 x 128K tokens (m=2: 64K entries), Full + 5 Reuse, 64 heads, "
                        "indexer 8x128, top-2048", 8,
                        B=16, N=65536, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048,
                        layers=["full"] + ["reuse"] * 5, m=2),
    # The decode64k step with the pages' MXFP4 indexer keys (64 code bytes +
    # 4 E8M0 scale bytes per token instead of 128 E4M3 bytes).
    "mxfp4_64k": Workload("MXFP4 indexer keys: B64 x 64K ctx, Full, 64 heads, indexer 8x128, top-2048", 9,
                          B=64, N=65536, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048, mxfp4=True),
    # The pages' decode step in their own formats: the 512-wide K = V row
    # (288 bytes), MXFP4 indexer keys of 32 heads x 128 (68 bytes), top-512,
    # and the fused RoPE around attention.
    "pages64k": Workload("pages' formats: B64 x 64K ctx, K=V 512 (288 B) + MXFP4 indexer 32x128 (68 B), "
                         "top-512, fused RoPE", 10,
                         B=64, N=65536, H=64, d_qk=512, d_v=512, H_I=32, D_I=128, K=512, mxfp4=True, rope=True,
                         softmax_scale=1.0 / (512.0 ** 0.5)),
    # Serving layout: the decode64k step with the main rows in a pool of
    # 64-token pages (random page order) and each window in a 128-row ring.
    "paged64k": Workload("paged decode: B64 x 64K ctx, 64-token pages, ring window, Full, 64 heads, "
                         "indexer 8x128, top-2048", 7,
                         B=64, N=65536, H=64, d_qk=576, d_v=512, H_I=8, D_I=128, K=2048, page_size=64),
    # The pages' own shapes: 512-wide K=V row, indexer 32 x 128, top-512.
    "pages512": Workload("pages' shape: B2 x 8192 ctx, d 512 (K=V), indexer 32x128, top-512", 5,
                         B=2, N=8192, H=64, d_qk=512, d_v=512, H_I=32, D_I=128, K=512,
                         softmax_scale=1.0 / (512.0 ** 0.5)),
}


def decode_layer_inputs(wl, layer, device="cpu", seqs=None):
    """Per-layer query-side inputs of a decode workload (fresh for every layer).

    Returns dict: q_idx [B][Tq][H_I][D_I] u8, w [B][Tq][H_I] f32,
    q [B][Tq][H][d_qk] f32, swa_x [B][W][d_qk] f32 (window rows before
    quantisation).  `seqs` restricts to a subset of sequences (same values as
    in the full draw).
    """
    B, Tq = wl.B, wl.Tq
    d = {
        "q_idx": int_e4m3((B, Tq, wl.H_I, wl.D_I), wl.seed, layer, "q_idx", device=device),
        "w": normal_f32((B, Tq, wl.H_I), wl.seed, layer, "w", device=device),
        "q": normal_f32((B, Tq, wl.H, wl.d_qk), wl.seed, layer, "q", device=device),
        "swa_x": normal_f32((B, wl.W + Tq - 1, wl.d_qk), wl.seed, layer, "swa", device=device),
    }
    if seqs is not None:
        d = {k: v[seqs] for k, v in d.items()}
    return d


def shared_cache_inputs(wl, device="cpu"):
    """Shared caches of a workload: kv_x [B][N][d_qk] f32 rows, k_idx [B][N][D_I] u8."""
    return {
        "kv_x": normal_f32((wl.B, wl.N, wl.d_qk), wl.seed, 0, "kv", device=device),
        "k_idx": int_e4m3((wl.B, wl.N, wl.D_I), wl.seed, 0, "k_idx", device=device),
    }


def random_index_lists(B, K, N, seed, layer=0, device="cpu", n_invalid=0):
    """Random Top-K-shaped index lists [B][K] int32: distinct ids < N, with the
    last n_invalid slots of each row replaced by -1 and out-of-range ids."""
    g = _gen(seed, layer, "q", device)
    out = torch.empty(B, K, dtype=torch.int32, device=device)
    for b in range(B):
        perm = torch.randperm(N, generator=g, device=device)[:K]
        out[b, : len(perm)] = perm.to(torch.int32)
        if len(perm) < K:
            out[b, len(perm):] = -1
    if n_invalid:
        bad = torch.full((B, n_invalid), -1, dtype=torch.int32, device=device)
        bad[:, ::2] = N + 7
        out[:, K - n_invalid:] = bad
    return out


def rope_angles(B, seed, device="cpu"):
    """Rotary angles of each row's query position for 32 channel pairs (uniform
    over many turns: the kernel only sees their cosines and sines)."""
    return normal_f32((B, 32), seed, 0, "sink", device=device) * 100.0


def idx_key_rows(shape, seed, device="cpu"):
    """float32 N(0, 1) indexer key rows (before the MXFP4 write)."""
    return normal_f32(shape, seed, 0, "k_idx", device=device)


def page_order(n_pages, n_used, seed, device="cpu"):
    """A random order of the pool's pages (the first n_used are handed out)."""
    g = _gen(seed, 0, "kv", device)
    return torch.randperm(n_pages, generator=g, device=device)[:n_used]


def kv_rows_seq(wl, b, device="cpu"):
    """float32 N(0, 1) latent rows [N][d_qk] of sequence b (drawn per sequence so
    that very long caches can be built and checked one sequence at a time)."""
    return normal_f32((wl.N, wl.d_qk), wl.seed * 7919 + b, 0, "kv", device=device)
