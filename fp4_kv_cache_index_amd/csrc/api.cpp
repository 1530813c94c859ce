// C ABI of the CSA2 hot path: host-side validation, workspace layout and the
// launch sequence of each operation.  Every operation enqueues its kernels on
// the caller's stream and returns; nothing here allocates or synchronises.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <cstring>

#include "../../include/csa2.h"
#include "internal.h"

namespace csa2 {

Trace& thread_trace() {
  static thread_local Trace t;
  return t;
}

bool trace_launch(const char* name, hipEvent_t* start, hipEvent_t* stop) {
  Trace& t = thread_trace();
  if (!t.active) return false;
  if (t.only[0] != 0 && std::strcmp(name, t.only) != 0) return false;
  const int c = t.count++;
  if (c >= t.capacity) return false;   // counted, not timed
  *start = t.events[2 * c];
  *stop = t.events[2 * c + 1];
  if (t.names) t.names[c] = name;
  return true;
}

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int v = cache[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

static inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }
static inline bool aligned4(const void* p) { return ((uintptr_t)p & 3u) == 0; }
static inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// ----------------------------------------------------- index score topk ---

struct ScoreLayout {
  int64_t rows, n_stride, nb_max, nb_stride;
  int64_t th_stride;   // per-tile histograms per row (one-workgroup select), or 0
  size_t off_keys, off_nvalid, off_tok, off_bkeys, off_nbvalid, off_blk, off_th, total;
};

static ScoreLayout score_layout(int64_t B, int64_t Tq, int64_t n_max, int32_t pool_block) {
  ScoreLayout L{};
  L.rows = B * Tq;
  L.n_stride = round_up(n_max > 0 ? n_max : 1, 64);
  size_t o = 0;
  L.off_keys = o; o += al256(sizeof(uint32_t) * L.rows * L.n_stride);
  L.off_nvalid = o; o += al256(sizeof(int32_t) * L.rows);
  L.off_tok = o; o += al256(select_ws_bytes(L.rows, n_max));
  if (pool_block > 0) {
    L.nb_max = (n_max + pool_block - 1) / pool_block;
    L.nb_stride = round_up(L.nb_max > 0 ? L.nb_max : 1, 64);
    L.off_bkeys = o; o += al256(sizeof(uint32_t) * L.rows * L.nb_stride);
    L.off_nbvalid = o; o += al256(sizeof(int32_t) * L.rows);
    L.off_blk = o; o += al256(select_ws_bytes(L.rows, L.nb_max));
  } else if (n_max <= kLocalSel) {
    L.th_stride = index_score_tiles_bound(n_max);
    L.off_th = o; o += al256(sizeof(uint32_t) * 2048 * L.rows * L.th_stride);
  }
  L.total = o;
  return L;
}

static bool pool_block_ok(int32_t pb) { return pb == 1 || pb == 2 || pb == 4 || pb == 8 || pb == 16; }
static bool d_idx_ok(int32_t D_I) { return D_I == 32 || D_I == 64 || D_I == 128 || D_I == 256; }

// ------------------------------------------------------------ attention ---

static int attn_common_check(const float* q, const uint8_t* kv_codes, int64_t c_bstride, int64_t c_rstride,
                             const uint8_t* kv_scales, int64_t s_bstride, int64_t s_rstride,
                             const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len,
                             const uint8_t* swa_vals, int64_t sv_bstride, int64_t sv_rstride,
                             const uint8_t* swa_scales, int64_t ss_bstride, int64_t ss_rstride, int32_t W,
                             int32_t B, int32_t H, int32_t d_qk, int32_t d_v, float* out) {
  if (!q || !kv_codes || !kv_scales || !topk_idx || !ctx_len || !out) return CSA2_EINVAL;
  if (B < 0 || k_top < 0 || W < 0 || H <= 0 || d_qk <= 0 || d_v <= 0) return CSA2_EINVAL;
  if (d_qk % 16 != 0 || d_v > d_qk || d_v % 16 != 0) return CSA2_EINVAL;
  // Code rows are read as 32-bit words; scale bytes are read one at a time.
  if (!aligned4(kv_codes) || !aligned4(q)) return CSA2_EINVAL;
  if ((c_bstride | c_rstride) & 3) return CSA2_EINVAL;
  if (c_rstride < d_qk / 2 || s_rstride < d_qk / 16 || c_bstride < 0 || s_bstride < 0) return CSA2_EINVAL;
  if (W > 0) {
    if (!swa_vals || !swa_scales) return CSA2_EINVAL;
    if (!aligned4(swa_vals) || ((sv_bstride | sv_rstride) & 3)) return CSA2_EINVAL;
    if (sv_rstride < d_qk || ss_rstride < d_qk / 32 || sv_bstride < 0 || ss_bstride < 0) return CSA2_EINVAL;
    if (d_qk % 32 != 0) return CSA2_EINVAL;
  }
  if (!((d_qk == 576 && d_v == 512) || (d_qk == 512 && d_v == 512))) return CSA2_EUNSUPPORTED;
  if (H % 16 != 0 || H > 64) return CSA2_EUNSUPPORTED;
  return CSA2_OK;
}

}  // namespace csa2

using namespace csa2;

extern "C" {

const char* csa2_status_string(int status) {
  switch (status) {
    case CSA2_OK: return "ok";
    case CSA2_EINVAL: return "invalid argument (null pointer, shape, stride or alignment)";
    case CSA2_EUNSUPPORTED: return "valid arguments outside the supported shape set";
    case CSA2_EWORKSPACE: return "workspace smaller than the required size";
    case CSA2_EHIP: return "HIP launch error";
    default: return "unknown status";
  }
}

const char* csa2_version(void) { return "0.1.0"; }

int kv_fp4_quantize(const float* x, int64_t n_rows, int32_t d, int64_t x_row_stride, uint8_t* codes,
                    int64_t codes_row_stride, uint8_t* scales, int64_t scales_row_stride, void* stream) {
  if (n_rows < 0 || d <= 0 || d % 16 != 0) return CSA2_EINVAL;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !codes || !scales) return CSA2_EINVAL;
  if (x_row_stride < d || codes_row_stride < d / 2 || scales_row_stride < d / 16) return CSA2_EINVAL;
  if (!aligned4(x) || !aligned4(codes) || (codes_row_stride & 3)) return CSA2_EINVAL;
  hipError_t e = launch_kv_fp4_quantize(x, n_rows, d, x_row_stride, codes, codes_row_stride, scales,
                                        scales_row_stride, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

int swa_fp8_quantize(const float* x, int64_t n_rows, int32_t d, int64_t x_row_stride, uint8_t* vals,
                     int64_t vals_row_stride, uint8_t* scales, int64_t scales_row_stride, void* stream) {
  if (n_rows < 0 || d <= 0 || d % 32 != 0) return CSA2_EINVAL;
  if (n_rows == 0) return CSA2_OK;
  if (!x || !vals || !scales) return CSA2_EINVAL;
  if (x_row_stride < d || vals_row_stride < d || scales_row_stride < d / 32) return CSA2_EINVAL;
  if (!aligned4(x) || !aligned4(vals) || (vals_row_stride & 3)) return CSA2_EINVAL;
  hipError_t e = launch_swa_fp8_quantize(x, n_rows, d, x_row_stride, vals, vals_row_stride, scales,
                                         scales_row_stride, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

size_t csa2_index_score_topk_workspace_size(int32_t B, int32_t Tq, int64_t n_max, int32_t k_top,
                                            int32_t pool_block, int32_t pool_nblocks) {
  (void)k_top;
  (void)pool_nblocks;
  if (B < 0 || Tq < 0 || n_max < 0) return 0;
  return score_layout(B, Tq, n_max, pool_block > 0 ? pool_block : 0).total;
}

int csa2_index_score_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_batch_stride,
                          int64_t k_row_stride, const int32_t* ctx_len, const int32_t* q_pos, int32_t B, int32_t Tq,
                          int32_t H_I, int32_t D_I, int64_t n_max, int32_t k_top, int32_t* topk_idx,
                          float* topk_score, int32_t pool_block, int32_t pool_nblocks, int32_t* pool_idx,
                          int32_t* pool_len, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || Tq < 0 || n_max < 0 || k_top <= 0 || H_I <= 0 || D_I <= 0) return CSA2_EINVAL;
  if (B == 0 || Tq == 0) return CSA2_OK;
  if (!q_idx || !w || !k_idx || !ctx_len || !topk_idx || !ws) return CSA2_EINVAL;
  if (D_I % 32 != 0 || k_row_stride < D_I || k_batch_stride < 0) return CSA2_EINVAL;
  if (!aligned4(k_idx) || (k_row_stride & 3) || (k_batch_stride & 3) || !aligned4(q_idx)) return CSA2_EINVAL;
  if (((uintptr_t)ws & 255u) != 0) return CSA2_EINVAL;
  const bool pool = pool_idx != nullptr;
  if (pool) {
    if (!pool_len || pool_nblocks <= 0 || !pool_block_ok(pool_block)) return CSA2_EINVAL;
  }
  if (!d_idx_ok(D_I) || H_I > 32) return CSA2_EUNSUPPORTED;
  if (n_max > (int64_t)kSelTile * kMaxSelTiles || (int64_t)B * Tq > 65535) return CSA2_EUNSUPPORTED;
  if (D_I >= 128 && (k_row_stride & 15)) return CSA2_EINVAL;  // 16-byte slices per lane
  if ((k_row_stride & 7) || (k_batch_stride & 7)) return CSA2_EINVAL;
  if (k_row_stride >= (int64_t)1 << 22) return CSA2_EUNSUPPORTED;   // 32-bit row offsets in the scan
  ScoreLayout L = score_layout(B, Tq, n_max, pool ? pool_block : 0);
  if (ws_bytes < L.total) return CSA2_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  uint32_t* keys = (uint32_t*)(base + L.off_keys);
  int32_t* n_valid = (int32_t*)(base + L.off_nvalid);
  SelectWs tok = select_ws_carve(base + L.off_tok, L.rows, n_max);
  SelectWs blk{};
  uint32_t* bkeys = nullptr;
  int32_t* nb_valid = nullptr;
  if (pool) {
    bkeys = (uint32_t*)(base + L.off_bkeys);
    nb_valid = (int32_t*)(base + L.off_nbvalid);
    blk = select_ws_carve(base + L.off_blk, L.rows, L.nb_max);
  }
  ScoreArgs a{q_idx, w, k_idx, k_batch_stride, k_row_stride, ctx_len, q_pos, B, Tq, H_I, D_I, n_max, k_top,
              pool ? pool_block : 0, pool ? pool_nblocks : 0};
  const SelectOut tout{topk_idx, topk_score, nullptr, 0, 0, nullptr, nullptr};
  if (!pool && n_max <= kLocalSel) {
    // Rows of at most 64K positions: one workgroup per row selects, with the
    // first digit from the scan's per-tile histograms (the dense prefill
    // path writes none: there the select builds it).
    const int64_t tiles = index_score_tiles(a);
    SelectWs th = tok;
    th.hist1 = nullptr;
    th.tile_hist = tiles > 0 ? (uint32_t*)(base + L.off_th) : nullptr;
    th.th_stride = L.th_stride;
    hipError_t e = launch_index_score(a, keys, L.n_stride, n_valid, th, nullptr, 0, nullptr, nullptr, s);
    if (e == hipSuccess)
      e = select_local(keys, L.n_stride, n_valid, L.rows, k_top, n_max, th.tile_hist, L.th_stride, tiles, tout, s);
    return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
  }
  hipError_t e = select_clear(tok, L.rows, s);
  if (e == hipSuccess && pool) e = select_clear(blk, L.rows, s);
  if (e == hipSuccess)
    e = launch_index_score(a, keys, L.n_stride, n_valid, tok, bkeys, L.nb_stride, nb_valid, pool ? &blk : nullptr, s);
  if (e == hipSuccess) e = select_finish(tok, keys, L.n_stride, n_valid, L.rows, k_top, tout, s);
  if (e == hipSuccess && pool) {
    SelectOut out{pool_idx, nullptr, nullptr, 0, pool_block, n_valid, pool_len};
    e = select_finish(blk, bkeys, L.nb_stride, nb_valid, L.rows, pool_nblocks, out, s);
  }
  return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

size_t csa2_hier_pool_topk_workspace_size(int32_t B, int32_t Tq, int32_t pool_cap, int32_t k_top) {
  (void)k_top;
  if (B < 0 || Tq < 0 || pool_cap < 0) return 0;
  int64_t rows = (int64_t)B * Tq;
  return al256(sizeof(uint32_t) * rows * round_up(pool_cap > 0 ? pool_cap : 1, 64)) + al256(sizeof(int32_t) * rows) +
         al256(select_ws_bytes(rows, pool_cap));
}

int csa2_hier_pool_topk(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_batch_stride,
                        int64_t k_row_stride, const int32_t* pool_idx, const int32_t* pool_len, int32_t pool_cap,
                        int32_t B, int32_t Tq, int32_t H_I, int32_t D_I, int32_t k_top, int32_t* topk_idx,
                        float* topk_score, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || Tq < 0 || pool_cap < 0 || k_top <= 0 || H_I <= 0 || D_I <= 0) return CSA2_EINVAL;
  if (B == 0 || Tq == 0) return CSA2_OK;
  if (!q_idx || !w || !k_idx || !pool_idx || !pool_len || !topk_idx || !ws) return CSA2_EINVAL;
  if (D_I % 32 != 0 || k_row_stride < D_I || k_batch_stride < 0) return CSA2_EINVAL;
  if (!aligned4(k_idx) || !aligned4(q_idx) || (k_row_stride & 7) || (k_batch_stride & 7)) return CSA2_EINVAL;
  if (((uintptr_t)ws & 255u) != 0) return CSA2_EINVAL;
  if (!d_idx_ok(D_I) || H_I > 32) return CSA2_EUNSUPPORTED;
  if (D_I >= 128 && (k_row_stride & 15)) return CSA2_EINVAL;
  if ((int64_t)B * Tq > 65535 || pool_cap > kSelTile * kMaxSelTiles) return CSA2_EUNSUPPORTED;
  size_t need = csa2_hier_pool_topk_workspace_size(B, Tq, pool_cap, k_top);
  if (ws_bytes < need) return CSA2_EWORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  int64_t rows = (int64_t)B * Tq;
  int64_t cap = round_up(pool_cap > 0 ? pool_cap : 1, 64);   // key row stride
  char* base = (char*)ws;
  uint32_t* keys = (uint32_t*)base;
  base += al256(sizeof(uint32_t) * rows * cap);
  int32_t* n_valid = (int32_t*)base;
  base += al256(sizeof(int32_t) * rows);
  SelectWs sw = select_ws_carve(base, rows, pool_cap);
  const SelectOut out{topk_idx, topk_score, pool_idx, pool_cap, 0, nullptr, nullptr};
  if (pool_cap <= kLocalSelMap) {
    // Pools that fit one workgroup: the select builds the first digit itself
    // (the pool scan's small tiles would leave many per-tile histograms to
    // add up).
    SelectWs none = sw;
    none.hist1 = nullptr;
    hipError_t e = launch_pool_score(q_idx, w, k_idx, k_batch_stride, k_row_stride, pool_idx, pool_len, pool_cap, B,
                                     Tq, H_I, D_I, k_top, keys, cap, n_valid, none, s);
    if (e == hipSuccess) e = select_local(keys, cap, n_valid, rows, k_top, pool_cap, nullptr, 0, 0, out, s);
    return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
  }
  hipError_t e = select_clear(sw, rows, s);
  if (e == hipSuccess)
    e = launch_pool_score(q_idx, w, k_idx, k_batch_stride, k_row_stride, pool_idx, pool_len, pool_cap, B, Tq, H_I,
                          D_I, k_top, keys, cap, n_valid, sw, s);
  if (e == hipSuccess) e = select_finish(sw, keys, cap, n_valid, rows, k_top, out, s);
  return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

size_t csa2_sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t d_v, int32_t k_top, int32_t W) {
  if (B < 0 || H <= 0 || d_v <= 0 || k_top < 0 || W < 0) return 0;
  int splits = attn_num_splits(B, k_top, W);
  return attn_ws_bytes(B, H, d_v, splits);
}

int csa2_sparse_attn_decode(const float* q, const uint8_t* kv_codes, int64_t c_batch_stride, int64_t c_row_stride,
                            const uint8_t* kv_scales, int64_t s_batch_stride, int64_t s_row_stride,
                            const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len,
                            const uint8_t* swa_vals, int64_t sv_batch_stride, int64_t sv_row_stride,
                            const uint8_t* swa_scales, int64_t ss_batch_stride, int64_t ss_row_stride,
                            const int32_t* swa_len, int32_t W, const float* sink, int32_t B, int32_t H, int32_t d_qk,
                            int32_t d_v, float softmax_scale, float* out, float* lse, void* ws, size_t ws_bytes,
                            void* stream) {
  if (B == 0) return CSA2_OK;
  int st = attn_common_check(q, kv_codes, c_batch_stride, c_row_stride, kv_scales, s_batch_stride, s_row_stride,
                             topk_idx, k_top, ctx_len, swa_vals, sv_batch_stride, sv_row_stride, swa_scales,
                             ss_batch_stride, ss_row_stride, W, B, H, d_qk, d_v, out);
  if (st != CSA2_OK) return st;
  if (W > 0 && !swa_len) return CSA2_EINVAL;
  if (k_top + W == 0) return CSA2_EINVAL;
  if (B > 65535) return CSA2_EUNSUPPORTED;
  if (!ws || ((uintptr_t)ws & 255u)) return CSA2_EINVAL;
  if (ws_bytes < csa2_sparse_attn_decode_workspace_size(B, H, d_v, k_top, W)) return CSA2_EWORKSPACE;
  AttnArgs a{q, kv_codes, c_batch_stride, c_row_stride, kv_scales, s_batch_stride, s_row_stride, topk_idx, k_top,
             ctx_len, nullptr, swa_vals, sv_batch_stride, sv_row_stride, swa_scales, ss_batch_stride, ss_row_stride,
             swa_len, nullptr, 0, W, sink, B, 1, H, d_qk, d_v, softmax_scale, out, lse};
  hipError_t e = launch_sparse_attn(a, false, ws, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

size_t csa2_sparse_attn_prefill_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d_v, int32_t k_top,
                                               int32_t W) {
  if (B < 0 || Tq < 0 || H <= 0 || d_v <= 0 || k_top < 0 || W < 0) return 0;
  int64_t rows = (int64_t)B * Tq;
  int splits = attn_num_splits(rows, k_top, W);
  return attn_ws_bytes(rows, H, d_v, splits);
}

int csa2_sparse_attn_prefill(const float* q, const uint8_t* kv_codes, int64_t c_batch_stride, int64_t c_row_stride,
                             const uint8_t* kv_scales, int64_t s_batch_stride, int64_t s_row_stride,
                             const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len, const int32_t* q_pos,
                             const uint8_t* swa_vals, int64_t sv_batch_stride, int64_t sv_row_stride,
                             const uint8_t* swa_scales, int64_t ss_batch_stride, int64_t ss_row_stride,
                             const int32_t* swa_pos0, int32_t swa_rows, int32_t W, const float* sink, int32_t B,
                             int32_t Tq, int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale, float* out,
                             float* lse, void* ws, size_t ws_bytes, void* stream) {
  if (B == 0 || Tq == 0) return CSA2_OK;
  if (B < 0 || Tq < 0) return CSA2_EINVAL;
  int st = attn_common_check(q, kv_codes, c_batch_stride, c_row_stride, kv_scales, s_batch_stride, s_row_stride,
                             topk_idx, k_top, ctx_len, swa_vals, sv_batch_stride, sv_row_stride, swa_scales,
                             ss_batch_stride, ss_row_stride, W, B, H, d_qk, d_v, out);
  if (st != CSA2_OK) return st;
  if (!q_pos) return CSA2_EINVAL;
  if (W > 0 && (!swa_pos0 || swa_rows < 0)) return CSA2_EINVAL;
  if (k_top + W == 0) return CSA2_EINVAL;
  if ((int64_t)B * Tq > 65535) return CSA2_EUNSUPPORTED;
  if (!ws || ((uintptr_t)ws & 255u)) return CSA2_EINVAL;
  if (ws_bytes < csa2_sparse_attn_prefill_workspace_size(B, Tq, H, d_v, k_top, W)) return CSA2_EWORKSPACE;
  AttnArgs a{q, kv_codes, c_batch_stride, c_row_stride, kv_scales, s_batch_stride, s_row_stride, topk_idx, k_top,
             ctx_len, q_pos, swa_vals, sv_batch_stride, sv_row_stride, swa_scales, ss_batch_stride, ss_row_stride,
             nullptr, swa_pos0, W > 0 ? swa_rows : 0, W, sink, B, Tq, H, d_qk, d_v, softmax_scale, out, lse};
  hipError_t e = launch_sparse_attn(a, true, ws, (hipStream_t)stream);
  return e == hipSuccess ? CSA2_OK : CSA2_EHIP;
}

int csa2_trace_attach(void** events, const char** names, int32_t capacity) {
  if (capacity < 0 || (capacity > 0 && !events)) return CSA2_EINVAL;
  Trace& t = thread_trace();
  t.events = (hipEvent_t*)events;
  t.names = names;
  t.capacity = capacity;
  t.count = 0;
  t.active = true;
  return CSA2_OK;
}

int csa2_trace_only(const char* kernel_name) {
  Trace& t = thread_trace();
  if (!t.active) return CSA2_EINVAL;
  if (kernel_name && std::strlen(kernel_name) >= sizeof(t.only)) return CSA2_EINVAL;
  std::memset(t.only, 0, sizeof(t.only));
  if (kernel_name) std::strcpy(t.only, kernel_name);
  return CSA2_OK;
}

int csa2_trace_detach(int32_t* n_launches) {
  Trace& t = thread_trace();
  if (n_launches) *n_launches = t.count;
  t = Trace{};
  return CSA2_OK;
}

}  // extern "C"
