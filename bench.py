"""CSA2 hot-path benchmark on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

A step is one pass of the hot path over one batch of synthetic input with
every cache resident in HBM:
  decode64k   (default) one Full-mode decode layer: indexer scores + exact
              Top-K over all 64K tokens of 64 sequences, then sparse FP4 +
              FP8-window attention of 64 heads;
  tiny        the same at 1 x 4096 (a parity-sized case);
  group128k   Full -> Reindex -> Reuse layers over 16 x 128K;
  hier1m      Full layer with the 2048 x 8 candidate pool + 9 pool layers, 4 x 1M;
  prefill256k one causal chunk of 4096 queries on a 256K cache;
  enc128k     encoder group (one cache entry per two tokens): Full + 5 Reuse
              layers over 16 x 64K entries;
  paged64k    decode64k with the main rows in a page pool and ring windows;
  mxfp4_64k   decode64k with the pages' MXFP4 indexer keys (68 bytes per token);
  pages64k    the pages' own decode formats: 512-wide K = V rows, MXFP4 keys of
              32 indexer heads, top-512, RoPE fused around attention;
  mq2_64k     multi-query decode: 2 query tokens per sequence over 64 x 64K
              (one pass over the keys for both, then attention per token).
Every step is timed by its own pair of HIP events; ms_per_step is their
median, and between steps (outside the events) a 512 MB buffer is read so
that no step starts with its inputs in the 256 MB MALL (--no-flush keeps
the caches warm).  Prints one JSON line: decode queries/s, algorithmic HBM
GB/s, the roofline of the dominant kernel (HIP events carried by its
launches inside the timed region; no other launch is bracketed there), a
per-kernel breakdown from a separate traced pass, and the CPU oracle timed
on a bounded sample.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
FP8_PEAK_TFLOPS = 5000.0      # dense FP8 matrix-core peak of MI355X
METRIC = "CSA2 decode queries/s + achieved HBM GB/s (% peak), 64K–1M ctx"


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default="decode64k")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-sample", type=int, default=0, help="sequences timed for the CPU baseline (0 = auto)")
    p.add_argument("--copy-calibration", action="store_true",
                   help="run only a plain 1 GiB device copy (for counter calibration) and exit")
    p.add_argument("--no-flush", action="store_true",
                   help="do not read the 512 MB flush buffer between timed steps (MALL left warm)")
    p.add_argument("--stored-keys", action="store_true",
                   help="give the indexer its stored-key workspace (prefill chunks then store their score keys "
                        "and select in one scoring pass instead of by scoring passes)")
    return p.parse_args()


# ------------------------------------------------------------ step timer ---

class StepTimer:
    """Per-step HIP events on one stream, created without the system-scope
    fence (they only carry timestamps: with the fence every record wrote back
    the L2 and left gaps of several microseconds around it)."""

    FLAGS = 0x20000000   # hipEventDisableSystemFence

    def __init__(self, n, stream):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.stream = ctypes.c_void_p(stream.cuda_stream)
        self.ev = []
        for _ in range(2 * n):
            e = ctypes.c_void_p()
            if self.hip.hipEventCreateWithFlags(ctypes.byref(e), self.FLAGS) != 0:
                raise RuntimeError("hipEventCreateWithFlags failed")
            self.ev.append(e)

    def start(self, i):
        self.hip.hipEventRecord(self.ev[2 * i], self.stream)

    def stop(self, i):
        self.hip.hipEventRecord(self.ev[2 * i + 1], self.stream)

    def ms(self):
        out = []
        for i in range(len(self.ev) // 2):
            t = self.ct.c_float()
            if self.hip.hipEventElapsedTime(self.ct.byref(t), self.ev[2 * i], self.ev[2 * i + 1]) != 0:
                raise RuntimeError("hipEventElapsedTime failed")
            out.append(t.value)
        return out

    def close(self):
        for e in self.ev:
            self.hip.hipEventDestroy(e)
        self.ev = []


# ------------------------------------------------------- counter traffic ---

def counter_traffic(kernel, workload="decode64k", key="traffic_bytes_per_launch"):
    """HBM bytes per launch (or, key="traffic_bytes_per_step", per step) of
    `kernel` on `workload` from the committed FETCH_SIZE/WRITE_SIZE summary,
    or None when that summary is missing or the kernel's sources have changed
    since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.md")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ": " in line and not line.startswith(("|", "#", "`")):
            k, v = line.split(": ", 1)
            kv[k.strip()] = v.strip()
    try:
        h = hashlib.sha256()
        for f in kv["kernel_source_files"].split():
            with open(os.path.join(ROOT, "fp4_kv_cache_index_amd", "csrc", f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != kv["kernel_source_sha256"]:
            return None
        return int(kv[key])
    except (KeyError, OSError, ValueError):
        return None


# ------------------------------------------------------------ byte model ---

def layer_bytes(wl, kind, pool_cap=0):
    """Algorithmic HBM bytes per query row of one layer (what the method must move)."""
    d, K, W, H = wl.d_qk, wl.K, wl.W, wl.H
    row = d // 2 + d // 16            # FP4 main row: codes + E4M3 scales
    swa = d + d // 32                 # window row: E4M3 values + E8M0 scales
    attn = K * row + W * swa + 4 * H * d + 4 * H * wl.d_v
    if wl.page_size:
        attn += 4 * K                 # the block-table entry of every Top-K token
    idx_q = wl.H_I * wl.D_I + 4 * wl.H_I
    key = wl.D_I // 2 + wl.D_I // 32 if wl.mxfp4 else wl.D_I     # indexer key bytes per token
    if kind in ("full", "reindex"):
        b = key * wl.N + idx_q + 8 * K + attn
        if wl.pool_block:
            b += 4 * wl.pool_nblocks * wl.pool_block        # pool write
        return b
    if kind == "reuse":
        return 4 * K + attn
    if kind == "pool":
        return wl.D_I * pool_cap + 4 * pool_cap + idx_q + 8 * K + attn
    raise ValueError(kind)


# ------------------------------------------------------------- workloads ---

class Case:
    """Resident inputs and the step function of one workload."""

    def __init__(self, wl, dev, stored_keys=False):
        import torch
        import fp4_kv_cache_index_amd as csa2
        from fp4_kv_cache_index_amd import inputs
        self.wl, self.dev, self.csa2, self.torch = wl, dev, csa2, torch
        B, N, d = wl.B, wl.N, wl.d_qk
        # Shared caches: FP4 main rows in the pages' interleaved entry layout.
        self.cache = torch.empty(B, N, d // 2 + d // 16, dtype=torch.uint8, device=dev)
        self.codes, self.scales = self.cache[..., : d // 2], self.cache[..., d // 2:]
        for b in range(B):   # quantise one sequence at a time (bounded temporary)
            x = inputs.kv_rows_seq(wl, b, device=dev)
            csa2.kv_fp4_quantize(x, codes=self.codes[b], scales=self.scales[b])
            del x
        if wl.page_size:
            # Serving layout: the same rows in a pool of pages handed out in a
            # random order, and each window in a ring (row = position % W).
            P = wl.page_size
            npg = (N + P - 1) // P
            self.n_pages = B * npg + 64
            self.block_table = inputs.page_order(self.n_pages, B * npg, wl.seed, device=dev).view(B, npg).to(
                torch.int32).contiguous()
            self.pool = torch.empty(self.n_pages * P, self.cache.shape[-1], dtype=torch.uint8, device=dev)
            j = torch.arange(N, device=dev)
            for b in range(B):
                self.pool.index_copy_(0, self.block_table[b, j // P].to(torch.int64) * P + j % P, self.cache[b])
            del self.cache, self.codes, self.scales
            self.pool_codes, self.pool_scales = self.pool[:, : d // 2], self.pool[:, d // 2:]
            self.swa_end = torch.full((B,), N, dtype=torch.int32, device=dev)
        if wl.mxfp4:   # the pages' indexer K: E2M1 codes + E8M0 scale per 32 channels, two arrays
            self.k_codes = torch.empty(B, N, wl.D_I // 2, dtype=torch.uint8, device=dev)
            self.k_scales = torch.empty(B, N, wl.D_I // 32, dtype=torch.uint8, device=dev)
            for b in range(B):
                x = inputs.idx_key_rows((N, wl.D_I), wl.seed * 7919 + b, device=dev)
                csa2.idx_mxfp4_quantize(x, codes=self.k_codes[b], scales=self.k_scales[b])
                del x
            self.k_idx = None
        else:
            self.k_idx = inputs.int_e4m3((B, N, wl.D_I), wl.seed, 0, "k_idx", device=dev)
        self.ctx = torch.full((B,), N, dtype=torch.int32, device=dev)
        if wl.rope:   # (cos, sin) of each row's query position for the 32 rotary channel pairs
            th = inputs.rope_angles(B, wl.seed, device=dev)
            self.rope_cs = torch.stack([torch.cos(th), torch.sin(th)], dim=-1).reshape(B, 64).contiguous()
        self.swa_len = torch.full((B,), wl.W, dtype=torch.int32, device=dev)
        self.layers = []
        for li, kind in enumerate(wl.layers):
            lay = inputs.decode_layer_inputs(wl, li, device=dev)
            sv, ss = csa2.swa_fp8_quantize(lay["swa_x"])
            if wl.page_size:   # window rows of positions N-W .. N-1 into their ring rows
                ring = (torch.arange(wl.W, device=dev) + N - wl.W) % wl.W
                sv = torch.empty_like(sv).index_copy_(1, ring, sv)
                ss = torch.empty_like(ss).index_copy_(1, ring, ss)
            ent = {"kind": kind, "q_idx": lay["q_idx"], "w": lay["w"], "sv": sv, "ss": ss,
                   "q": lay["q"] if wl.Tq > 1 else lay["q"][:, 0].contiguous()}
            self.layers.append(ent)
        if wl.Tq > 1:
            base = N - wl.Tq
            self.q_pos = (torch.arange(wl.Tq, dtype=torch.int32, device=dev) + base).repeat(B, 1).contiguous()
            self.swa_pos0 = torch.full((B,), base - wl.W + 1, dtype=torch.int32, device=dev)
        else:
            self.q_pos = None
        # Workspaces and outputs, allocated once.
        rows = B * wl.Tq
        pb, nb = (wl.pool_block, wl.pool_nblocks) if wl.pool_block else (0, 0)
        ws_size = (csa2.csa2_index_score_topk_workspace_size_stored if stored_keys else
                   csa2.csa2_index_score_topk_workspace_size)
        self.ws_idx = self._ws(ws_size(B, wl.Tq, N, wl.K, pb, nb))
        self.ws_idx_bytes = self.ws_idx.numel()
        self.ws_attn = self._ws(csa2.csa2_sparse_attn_prefill_workspace_size(B, wl.Tq, wl.H, wl.d_v, wl.K, wl.W)
                                if wl.Tq > 1 or wl.page_size else csa2.csa2_sparse_attn_decode_workspace_size(B, wl.H, wl.d_v, wl.K,
                                                                                            wl.W))
        self.pool_cap = nb * pb
        self.ws_pool = self._ws(csa2.csa2_hier_pool_topk_workspace_size(B, 1, self.pool_cap, wl.K)) if pb else None
        self.topk = [torch.empty(B, wl.Tq, wl.K, dtype=torch.int32, device=dev) for _ in wl.layers]
        self.out = torch.empty(rows * wl.H * wl.d_v, dtype=torch.float32, device=dev)
        if pb:
            self.pool_idx = torch.empty(B, 1, self.pool_cap, dtype=torch.int32, device=dev)
            self.pool_len = torch.empty(B, 1, dtype=torch.int32, device=dev)
        torch.cuda.synchronize()

    def _ws(self, n):
        t = self.torch.empty(int(n) + 256, dtype=self.torch.uint8, device=self.dev)
        off = (-t.data_ptr()) % 256
        return t[off:off + int(n)]

    def step(self):
        wl, csa2 = self.wl, self.csa2
        prev = None
        for li, L in enumerate(self.layers):
            kind = L["kind"]
            if kind in ("full", "reindex"):
                extra = {}
                if wl.pool_block and li == 0:
                    extra = dict(pool_block=wl.pool_block, pool_nblocks=wl.pool_nblocks,
                                 out={"topk_idx": self.topk[li], "pool_idx": self.pool_idx, "pool_len": self.pool_len})
                else:
                    extra = dict(out={"topk_idx": self.topk[li]})
                if wl.mxfp4:
                    csa2.csa2_index_score_topk_mxfp4(L["q_idx"], L["w"], self.k_codes, self.k_scales, self.ctx,
                                                     wl.K, q_pos=self.q_pos, workspace=self.ws_idx, **extra)
                else:
                    csa2.csa2_index_score_topk(L["q_idx"], L["w"], self.k_idx, self.ctx, wl.K, q_pos=self.q_pos,
                                               workspace=self.ws_idx, **extra)
                idx = self.topk[li]
            elif kind == "pool":
                csa2.csa2_hier_pool_topk(L["q_idx"], L["w"], self.k_idx, self.pool_idx, self.pool_len, wl.K,
                                         ctx_len=self.ctx, workspace=self.ws_pool, out={"topk_idx": self.topk[li]})
                idx = self.topk[li]
            elif kind == "reuse":
                idx = prev
            else:
                raise ValueError(kind)
            if wl.page_size:
                out = self.out.view(wl.B, wl.Tq, wl.H, wl.d_v)
                q4 = L["q"] if wl.Tq > 1 else L["q"].view(wl.B, 1, wl.H, wl.d_qk)
                csa2.csa2_sparse_attn_paged(q4, self.pool_codes, self.pool_scales, self.block_table, wl.page_size, idx,
                                            self.ctx, self.q_pos, L["sv"], L["ss"], self.swa_end, wl.W,
                                            wl.softmax_scale, d_v=wl.d_v, workspace=self.ws_attn, out=out)
            elif wl.Tq > 1:
                out = self.out.view(wl.B, wl.Tq, wl.H, wl.d_v)
                csa2.csa2_sparse_attn_prefill(L["q"], self.codes, self.scales, idx, self.ctx, self.q_pos, L["sv"],
                                              L["ss"], self.swa_pos0, wl.W, wl.softmax_scale, d_v=wl.d_v,
                                              workspace=self.ws_attn, out=out)
            elif wl.rope:
                out = self.out.view(wl.B, wl.H, wl.d_v)
                csa2.csa2_sparse_attn_decode_rope(L["q"], self.codes, self.scales, idx[:, 0], self.ctx, L["sv"],
                                                  L["ss"], self.swa_len, wl.softmax_scale, self.rope_cs,
                                                  rotate_q=True, workspace=self.ws_attn, out=out)
            else:
                out = self.out.view(wl.B, wl.H, wl.d_v)
                csa2.csa2_sparse_attn_decode(L["q"], self.codes, self.scales, idx[:, 0], self.ctx, L["sv"], L["ss"],
                                             self.swa_len, wl.softmax_scale, d_v=wl.d_v, workspace=self.ws_attn,
                                             out=out)
            prev = idx

    def step_bytes(self):
        wl = self.wl
        per_row = sum(layer_bytes(wl, L["kind"], self.pool_cap) for L in self.layers)
        total = per_row * wl.B * wl.Tq
        if wl.Tq > 1:
            # A prefill chunk streams the key cache once for all its queries.
            n_scan = sum(1 for L in self.layers if L["kind"] in ("full", "reindex"))
            total -= n_scan * (wl.D_I // 2 + wl.D_I // 32 if wl.mxfp4 else wl.D_I) * wl.N * wl.B * (wl.Tq - 1)
        return total


# ----------------------------------------------------------- CPU oracle ---

def cpu_baseline(case, n_seq, budget_s=10.0):
    """Time the oracle's step (scores + Top-K + attention) on at least n_seq
    sequences of the first layer, continuing while less than budget_s seconds
    of oracle work have accumulated (bounded by the batch); cache quantisation
    of the rows it reads is set-up and not timed."""
    import numpy as np
    from oracle import attention as A
    from oracle import indexer as I
    from oracle import quant as Q
    from oracle.topk import topk_select
    from fp4_kv_cache_index_amd import inputs
    wl = case.wl
    L = case.layers[0]
    h = lambda t: t.detach().cpu().numpy()
    t_tot = 0.0
    rows = 0
    swa_all = h(inputs.decode_layer_inputs(wl, 0, device=case.dev)["swa_x"])
    for b in range(wl.B):
        if b >= n_seq and t_tot >= budget_s:
            break
        k_idx = None if wl.mxfp4 else h(case.k_idx[b])
        kcb = h(case.k_codes[b]) if wl.mxfp4 else None
        ksb = h(case.k_scales[b]) if wl.mxfp4 else None
        kv_x = h(inputs.kv_rows_seq(wl, b, device=case.dev))
        qi, w, q = h(L["q_idx"][b]), h(L["w"][b]), h(L["q"][b])
        swa_x = swa_all[b]
        for t in range(wl.Tq if wl.Tq == 1 else 1):
            t0 = time.perf_counter()
            s = (I.index_scores_mxfp4(qi[t], w[t], kcb, ksb, wl.N) if wl.mxfp4
                 else I.index_scores(qi[t], w[t], k_idx, wl.N))
            idx, _ = topk_select(s, wl.N, wl.K)
            t1 = time.perf_counter()
            # set-up: the oracle's own cache rows for the selected ids and the window
            sel = idx[idx >= 0]
            codes = np.zeros((wl.N, wl.d_qk // 2), np.uint8)
            scales = np.zeros((wl.N, wl.d_qk // 16), np.uint8)
            codes[sel], scales[sel] = Q.fp4_quantize(kv_x[sel])
            v8, s8 = Q.mxfp8_quantize(swa_x[: wl.W])
            t2 = time.perf_counter()
            A.sparse_attn_decode_row(q if q.ndim == 2 else q[t], codes, scales, idx, wl.N, v8, s8, wl.W, wl.d_qk,
                                     wl.d_v, wl.softmax_scale)
            t3 = time.perf_counter()
            t_tot += (t1 - t0) + (t3 - t2)
            rows += 1
    try:
        from threadpoolctl import threadpool_info
        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        blas = 1
    return {"value": rows / t_tot, "unit": "queries/s", "cores": int(blas), "kind": "oracle",
            "sample": f"{rows} query row(s) of layer 0 of {wl.name} (scores + Top-K + attention, "
                      f"{t_tot:.1f} s of oracle work; "
                      f"host has {os.cpu_count()} logical CPUs, BLAS threads {blas})",
            "seconds": round(t_tot, 3)}


# ------------------------------------------------------------------ main ---

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); this build has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import fp4_kv_cache_index_amd as csa2
    from fp4_kv_cache_index_amd import inputs
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 3}))
        return
    wl = inputs.WORKLOADS[args.workload]
    print(f"[bench] building inputs for {wl.name}", file=sys.stderr, flush=True)
    case = Case(wl, dev, args.stored_keys)
    print("[bench] warmup", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        case.step()
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # Between timed steps (outside their events) a 512 MB buffer is read, so
    # that no step finds its inputs in the 256 MB MALL (or the L2) left by
    # the previous one.  A read leaves no dirty lines behind (a written flush
    # buffer made the next step pay for its write-back).
    flush = None
    if not args.no_flush:
        flush = torch.ones(64 << 20, dtype=torch.int64, device=dev)
        flush_out = torch.empty((), dtype=torch.int64, device=dev)
    timer = StepTimer(args.steps, stream)
    # Dominant kernel: the indexer scan over the key cache (decode) or the
    # dense FP8 scoring product (prefill chunk).  Inside the timed region only
    # its launches are bracketed by HIP events, so the step time carries two
    # event records per scoring launch and nothing else.
    prefill = wl.Tq >= 16         # (2..15 query rows per sequence: the multi-query scan)
    dom = "index_prefill" if prefill else "index_score"
    n_scan_layers = sum(1 for L in case.layers if L["kind"] in ("full", "reindex"))
    # (the bounded prefill selection scores in up to 8 passes per block of
    # query rows: 64 launches per step leave room for them)
    per_step = 64 if prefill else 4
    with csa2.KernelTrace(capacity=per_step * args.steps * max(1, len(wl.layers)), only=dom) as tr:
        torch.cuda.synchronize()
        e0.record(stream)
        for i in range(args.steps):
            if flush is not None:
                torch.amax(flush, dim=0, out=flush_out)
            timer.start(i)
            case.step()
            timer.stop(i)
        e1.record(stream)
        torch.cuda.synchronize()
    step_ms = sorted(timer.ms())
    timer.close()
    region_ms = e0.elapsed_time(e1)
    ms = step_ms[len(step_ms) // 2] if len(step_ms) % 2 else 0.5 * (step_ms[len(step_ms) // 2 - 1] +
                                                                   step_ms[len(step_ms) // 2])
    mean_ms = sum(step_ms) / len(step_ms)
    if tr.count > tr.capacity:
        raise RuntimeError(f"kernel trace holds {tr.capacity} launches, the timed steps made {tr.count}")
    dom_launches = [t for name, t in tr.durations_ms() if name == dom]
    tr.close()
    dom_ms = sum(dom_launches) / len(dom_launches) if dom_launches else float("nan")
    # Per-kernel breakdown from a separate traced pass (every launch bracketed).
    n_bd = min(args.steps, 5)
    with csa2.KernelTrace(capacity=(256 if prefill else 64) * n_bd * max(1, len(wl.layers))) as tr:
        for _ in range(n_bd):
            case.step()
        torch.cuda.synchronize()
    if tr.count > tr.capacity:
        raise RuntimeError(f"kernel trace holds {tr.capacity} launches, the traced steps made {tr.count}")
    per_kernel = {}
    for name, t in tr.durations_ms():
        s = per_kernel.setdefault(name, [0.0, 0])
        s[0] += t
        s[1] += 1
    tr.close()
    qps = wl.B * wl.Tq / (ms * 1e-3)
    step_bytes = case.step_bytes()
    gbps = step_bytes / (ms * 1e-3) / 1e9
    if prefill:
        # The chunk's scoring is one product over its causal (query, key)
        # pairs, run as one launch with stored keys or as the selection
        # passes (two sampled, one full, and short ones for rows still open)
        # with the bounded workspace: its time is the sum of the step's
        # launches, its work the product counted once.
        base = wl.N - wl.Tq
        pairs = wl.B * (wl.Tq * base + wl.Tq * (wl.Tq + 1) // 2)     # causal (query, key) pairs
        flops = 2 * wl.H_I * wl.D_I * pairs
        dom_step_ms = sum(dom_launches) / args.steps if dom_launches else float("nan")
        achieved = flops / (dom_step_ms * 1e-3) / 1e12
        wkey = "stored" if args.stored_keys else "passes"
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": FP8_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / FP8_PEAK_TFLOPS, 4),
                "traffic": counter_traffic(dom, f"{args.workload}_{wkey}", "traffic_bytes_per_step"),
                "kernel": dom, "kernel_ms": round(dom_step_ms, 5),
                "launches_per_step": round(len(dom_launches) / args.steps, 2), "selection": wkey}
    else:
        # one pass over the keys serves every query row of a sequence
        key = wl.D_I // 2 + wl.D_I // 32 if wl.mxfp4 else wl.D_I
        scan_bytes = (key * wl.N + wl.Tq * (wl.H_I * wl.D_I + 4 * wl.H_I)) * wl.B
        achieved = scan_bytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": counter_traffic(dom, args.workload), "kernel": dom,
                "kernel_ms": round(dom_ms, 5), "launches_per_step": n_scan_layers}
    cpu = None
    if not args.no_cpu_baseline:
        n_seq = args.cpu_sample or (1 if wl.N >= (1 << 20) else 2)
        print(f"[bench] CPU oracle on {n_seq} sequence(s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(case, n_seq)
    line = {
        "metric": METRIC, "value": round(qps, 1), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8+fp16 (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": wl.name, "global_batch": wl.B, "seq_len": wl.N, "query_tokens": wl.Tq,
                   "heads": wl.H, "indexer": f"{wl.H_I}x{wl.D_I}", "top_k": wl.K, "window": wl.W,
                   "layers": wl.layers, "tokens_per_entry": wl.m,
                   "indexer_keys": "MXFP4 (E2M1 + E8M0/32)" if wl.mxfp4 else "E4M3 integers",
                   "indexer_workspace_bytes": case.ws_idx_bytes, "parallelism": "single GPU"},
        "hbm_gbps": round(gbps, 1), "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "step_bytes": step_bytes,
        "step_stats": {"median_ms": round(ms, 5), "mean_ms": round(mean_ms, 5), "min_ms": round(step_ms[0], 5),
                       "max_ms": round(step_ms[-1], 5), "timed_region_ms": round(region_ms, 3),
                       "mall_flush_between_steps": flush is not None},
        "kernels_ms_per_step": {k: round(v[0] / n_bd, 5) for k, v in per_kernel.items()},
        "roofline": roof, "cpu_baseline": cpu,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
