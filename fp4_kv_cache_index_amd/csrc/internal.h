// Internal (host-side) interface between the C ABI and the kernel files.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace csa2 {

// Kernel launch with the optional per-thread trace: a traced launch carries
// its start and stop events in the dispatch itself (hipExtLaunchKernelGGL),
// so tracing puts no marker between kernels on the stream.
struct Trace {
  hipEvent_t* events = nullptr;
  const char** names = nullptr;
  int capacity = 0;
  int count = 0;
  bool active = false;
  char only[64] = {0};      // non-empty: trace only launches of this kernel name
};
Trace& thread_trace();

// True when the calling thread traces this launch; then *start and *stop are
// the events to attach to it.
bool trace_launch(const char* name, hipEvent_t* start, hipEvent_t* stop);

#define CSA2_LAUNCH(name, kernel, grid, block, shmem, stream, ...)                                       \
  do {                                                                                                   \
    hipEvent_t ev_start__ = nullptr, ev_stop__ = nullptr;                                                \
    if (::csa2::trace_launch((name), &ev_start__, &ev_stop__))                                           \
      hipExtLaunchKernelGGL(kernel, (grid), (block), (shmem), (stream), ev_start__, ev_stop__, 0u,       \
                            __VA_ARGS__);                                                                \
    else                                                                                                 \
      hipLaunchKernelGGL(kernel, (grid), (block), (shmem), (stream), __VA_ARGS__);                       \
  } while (0)

// Number of compute units of the current device (cached per device).
int device_cu_count();

// ----------------------------------------------------------- quantisers ---
hipError_t launch_kv_fp4_quantize(const float* x, int64_t n_rows, int d, int64_t x_stride,
                                  uint8_t* codes, int64_t c_stride, uint8_t* scales, int64_t s_stride,
                                  hipStream_t s);
hipError_t launch_idx_mxfp4_quantize(const float* x, int64_t n_rows, int d, int64_t x_stride,
                                     uint8_t* codes, int64_t c_stride, uint8_t* scales, int64_t s_stride,
                                     hipStream_t s);
hipError_t launch_swa_fp8_quantize(const float* x, int64_t n_rows, int d, int64_t x_stride,
                                   uint8_t* vals, int64_t v_stride, uint8_t* scales, int64_t s_stride,
                                   hipStream_t s);

// --------------------------------------------------------- radix select ---
// Per-row exact Top-K over u32 keys (larger is better, key 0 = absent) of
// the first n_valid[row] positions, ties to the lower position, emitted in
// ascending position order.  The producer of the keys also builds `hist1`,
// the per-row histogram of the top 12 key bits (after select_clear).
constexpr int kSelTile = 4096;       // positions per workgroup in the select passes
constexpr int kMaxSelTiles = 1024;   // positions per row <= kSelTile * kMaxSelTiles

struct SelectRowCtl {                // per-row control block (64 bytes)
  uint32_t cand_count;               // candidates appended by the collect pass
  uint32_t thr;                      // final threshold key T
  uint32_t need_eq;                  // ties at T to take (lowest positions)
  uint32_t total;                    // number of positions emitted
  uint32_t l1_total, l1_mode, l1_d, l1_above, l1_cnt;   // first-digit state (collect pass)
  uint32_t pad[7];
};

constexpr int kTileList = 512;       // positions listed per tile by the collect pass

struct SelectWs {
  SelectRowCtl* ctl;                 // [rows]
  uint32_t* hist1;                   // [rows][4096]
  uint32_t* cand;                    // [rows][cand_cap] of (key, position)
  uint32_t* tile_gt;                 // [rows][tiles] keys above the threshold bucket
  uint32_t* tile_off;                // [rows][tiles] output offset of the tile
  uint32_t* tile_eqb;                // [rows][tiles] threshold ties before the tile
  uint32_t* tile_cnt;                // [rows][tiles] listed positions, or ~0u when they did not fit
  uint16_t* tlist;                   // [rows][tiles][kTileList] in-tile offsets at or above the bucket
  int64_t cand_cap, tiles;
  // Used by the scoring kernels only when hist1 is null: when set, each
  // scoring workgroup stores its own top-12-bit histogram (2048 words, two
  // 16-bit bins per word, bin 2i in the low half of word i) at
  // tile_hist[(row * th_stride + tile) * 2048].
  uint32_t* tile_hist = nullptr;
  int64_t th_stride = 0;
};
size_t select_ws_bytes(int64_t rows, int64_t n_max);
SelectWs select_ws_carve(void* base, int64_t rows, int64_t n_max);

// Output modes of the emit pass.
struct SelectOut {
  int32_t* idx;                      // [rows][k] (row stride k)
  float* score;                      // nullable [rows][k]
  const int32_t* map;                // nullable [rows][map_stride]: emitted id = map[pos]
  int64_t map_stride;
  // Pool expansion: when expand > 0 each selected position c (a block)
  // expands to ids c*expand + u (u < expand, id < expand_limit[row]) at
  // output slots slot*expand + u; pool_len[row] receives the valid count.
  int expand;
  const int32_t* expand_limit;       // [rows] visible token count
  int32_t* pool_len;                 // [rows]
};

// Clears the control blocks and first-digit histograms of `rows` rows.
hipError_t select_clear(const SelectWs& ws, int64_t rows, hipStream_t s, const SelectWs* ws2 = nullptr);
// Rows of at most kLocalSel positions (kLocalSelMap with a map): one
// workgroup per row does the whole selection from the keys, taking the
// first radix digit from the producer's per-tile histograms when tile_hist
// is given (`tiles` of them per row, th_stride apart) and building it itself
// otherwise.  No clear pass is needed.  n_max bounds n_valid.  Not for pool
// expansion.
constexpr int kLocalSel = 65536;
constexpr int kLocalSelMap = 32768;
hipError_t select_local(const uint32_t* keys, int64_t key_stride, const int32_t* n_valid, int64_t rows, int k,
                        int64_t n_max, const uint32_t* tile_hist, int64_t th_stride, int64_t tiles,
                        const SelectOut& out, hipStream_t s);
// collect + finalize + emit, after the producer has written keys and hist1.
hipError_t select_finish(const SelectWs& ws, const uint32_t* keys, int64_t key_stride, const int32_t* n_valid,
                         int64_t rows, int k, const SelectOut& out, hipStream_t s);

// ------------------------------------------------ prefill chunk selection ---
// A dense prefill chunk (many query rows of one sequence against the same
// keys) selects without storing its [rows][n] score keys: the scoring
// product runs again in a few passes over the chunk's keys, each query row
// steered by a PfRow.
//   Pass 0 histograms the top 12 key bits of a 1/kPfSample sample of the
//   keys; from it each row finds the buckets that hold its threshold with a
//   margin of four standard deviations of the sample count, and pass 1
//   histograms the same sample again at a finer grain (4096 bins over those
//   buckets), which narrows the window to a few fine bins.  Pass 2 scores
//   every key, emits those above the window and appends those inside it as
//   candidates; the step kernel checks the
//   counts (emitted at most k_top, emitted + candidates at least k_top,
//   candidates at most kPfCap) and takes the rest from the sorted
//   candidates.  A row whose check fails starts over with the exact search:
//   a pass emits the keys that are selected for certain (above the threshold
//   bucket found so far: their positions go straight to the row's output,
//   unordered) and either histograms the next radix digit (12, 12, then 8
//   bits) of the keys still undecided, appends them as candidates (when at
//   most kPfCap of them remain), or, once the threshold key itself is known
//   and ties at it outnumber kPfCap, counts the ties per key tile and then
//   emits the lowest-position ones.
// A step kernel after each pass resolves the digit and picks the next mode;
// a last kernel sorts each row's positions.
constexpr int kPfCap = 4096;            // candidates kept per row
constexpr int kPfMaxK = 8192;           // largest k_top of this path (LDS sort)
constexpr int kPfRowsPerBlock = 1920;   // query rows per block of passes (workspace bound)
constexpr int kPfSample = 8;            // pass 0 scores one 16-key chunk in kPfSample
// two sample passes, the guess pass, then (rows whose guess failed) the exact
// search: digit levels 12 + 12 + 8, tie count, tie emission
constexpr int kPfPasses = 8;

enum PfMode : uint32_t {
  PF_DONE = 0, PF_HIST = 1, PF_CAND = 2, PF_EMIT = 3, PF_TIECOUNT = 4, PF_TIEEMIT = 5,
  PF_GUESS = 6   // emit keys >= g_emit, append keys in [g_cand, g_emit) as candidates
};

struct PfRow {                          // 80 bytes per query row
  uint32_t mode;
  // Keys selected for certain in the next pass: e_on, key in the previous
  // bucket (e_ps >= 32: every key; else key >> e_ps == e_pfx) and above the
  // current bucket (key >> n_ps > n_pfx), or inside it when e_incl.
  uint32_t e_on, e_ps, e_pfx, e_incl;
  // The undecided bucket: keys with key >> n_ps == n_pfx (n_ps >= 32: all).
  uint32_t n_ps, n_pfx;
  uint32_t need;                        // keys still to take from the bucket
  uint32_t bcnt;                        // keys in the bucket
  uint32_t out_cnt;                     // positions emitted so far (atomic)
  uint32_t cand_cnt;                    // candidates appended (atomic)
  // The histogram counts the sample: 1 coarse (pass 0), 2 fine (pass 1).
  uint32_t sampled;
  // PF_GUESS: keys >= g_emit are emitted (none when g_emit_none), keys in
  // [g_cand, g_emit) become candidates.
  uint32_t g_emit, g_cand, g_emit_none;
  // Sample passes: bin min((key - h_base) >> h_shift, 4095) of keys >=
  // h_base; s_total = sampled visible keys.
  uint32_t h_base, h_shift, s_total;
  uint32_t pad;
};

struct PfArgs {
  PfRow* rows;                          // [block rows]
  uint32_t* hist;                       // [block rows][4096]: digit histogram, or ties per key tile
  uint64_t* cand;                       // [block rows][kPfCap]: (key << 32) | ~position
  int32_t* out_idx;                     // the caller's topk_idx [rows][k_top]
  uint32_t* out_key;                    // nullable: the caller's topk_score [rows][k_top] (key bits until the end)
  const int32_t* n_valid;               // [rows]: visible keys per query row (written by every pass)
  uint32_t* active;                     // [kPfPasses]: 1 when a row of the block is not done after a step
  int64_t row_base;                     // first (global) query row of the block
  int k_top;
  int pass;                             // the pass a kernel runs (set per launch)
};
size_t pf_ws_bytes(int64_t block_rows);
PfArgs pf_ws_carve(void* base, int64_t block_rows);
// Initial state of every row of the block (level-1 histogram, zeroed counts).
hipError_t pf_clear(const PfArgs& pf, int64_t block_rows, hipStream_t s);
// After pass `pass`: resolve a digit / select candidates / prefix the tie
// counts.
hipError_t pf_step(const PfArgs& pf, int64_t block_rows, int pass, hipStream_t s);
// Sort each row's positions ascending, pad with -1 (scores: -inf).
hipError_t pf_final(const PfArgs& pf, int64_t block_rows, float* topk_score, hipStream_t s);

// ------------------------------------------------------------- scoring ---
struct ScoreArgs {
  const uint8_t* q_idx; const float* w;
  const uint8_t* k_idx; int64_t k_bstride, k_rstride;    // E4M3 key rows, or MXFP4 code rows
  const int32_t* ctx_len; const int32_t* q_pos;
  int B, Tq, H_I, D_I; int64_t n_max; int k_top;
  int pool_block, pool_nblocks;
  // MXFP4 keys (k_scales != null): E2M1 codes at k_idx, one E8M0 byte per 32
  // channels at k_scales + b * ks_bstride + j * ks_rstride.
  const uint8_t* k_scales = nullptr; int64_t ks_bstride = 0, ks_rstride = 0;
};
hipError_t launch_index_score(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                              const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                              const SelectWs* blk, hipStream_t s);
// Workgroups per row of the flat scan (0 when the dense prefill path
// scores instead, which writes no per-tile histograms), and an upper bound
// of it for any device.
int64_t index_score_tiles(const ScoreArgs& a);
int64_t index_score_tiles_bound(int64_t n_max);
// Dense prefill chunks: whether the matrix-core product scores this call,
// its query rows per workgroup (blocks of passes align with them), and one
// selection pass over the query tiles [y0, y0 + ny) (flattened (sequence,
// tile) index) steered by pf.
bool prefill_gemm_applies(const ScoreArgs& a);
int prefill_rows_per_tile(const ScoreArgs& a);
hipError_t launch_prefill_pass(const ScoreArgs& a, const PfArgs& pf, int pass, int64_t y0, int64_t ny,
                               int32_t* n_valid, hipStream_t s);
// Pool layers: a.q_idx / a.w / keys / ctx_len / B / Tq / H_I / D_I / k_top
// (and the MXFP4 scales) as in ScoreArgs.
hipError_t launch_pool_score(const ScoreArgs& a, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                             uint32_t* keys, int64_t key_stride, int32_t* n_valid, const SelectWs& ws, hipStream_t s);

// ----------------------------------------------------------- attention ---
struct AttnArgs {
  const float* q;
  const uint8_t* kv_codes; int64_t c_bstride, c_rstride;
  const uint8_t* kv_scales; int64_t s_bstride, s_rstride;
  const int32_t* topk_idx; int k_top; const int32_t* ctx_len;
  const int32_t* q_pos;                                  // prefill only (nullable)
  const uint8_t* swa_vals; int64_t sv_bstride, sv_rstride;
  const uint8_t* swa_scales; int64_t ss_bstride, ss_rstride;
  const int32_t* swa_len;                                // decode only
  const int32_t* swa_pos0; int swa_rows;                 // prefill only
  int W; const float* sink;
  int B, Tq, H, d_qk, d_v; float softmax_scale;
  float* out; float* lse;
  // Paged main rows (block_table != null): pool row of token j of sequence b
  // = block_table[b * bt_stride + (j >> page_shift)] << page_shift | (j & mask).
  const int32_t* block_table = nullptr; int64_t bt_stride = 0; int page_shift = 0; int n_pages = 0;
  // Ring window (swa_ring > 0): position x at row x % swa_ring; swa_end[b]
  // is one past the newest position written.
  int swa_ring = 0; const int32_t* swa_end = nullptr;
  // Rotary handling (rope_cs != null): per query row rope_dim floats, (cos,
  // sin) of each channel pair of the last rope_dim channels; q's rotary
  // channels rotated forward when rope_q, the output's rotated back.
  const float* rope_cs = nullptr; int rope_dim = 0; int rope_q = 0;
};
int attn_num_splits(int64_t rows, int k_top, int W);
size_t attn_ws_bytes(int64_t rows, int H, int d_v, int splits);
hipError_t launch_sparse_attn(const AttnArgs& a, bool prefill, void* ws, hipStream_t s);

}  // namespace csa2
