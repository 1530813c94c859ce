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
hipError_t select_clear(const SelectWs& ws, int64_t rows, hipStream_t s);
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

// ------------------------------------------------------------- scoring ---
struct ScoreArgs {
  const uint8_t* q_idx; const float* w;
  const uint8_t* k_idx; int64_t k_bstride, k_rstride;
  const int32_t* ctx_len; const int32_t* q_pos;
  int B, Tq, H_I, D_I; int64_t n_max; int k_top;
  int pool_block, pool_nblocks;
};
hipError_t launch_index_score(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                              const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                              const SelectWs* blk, hipStream_t s);
// Workgroups per row of the flat scan (0 when the dense prefill path
// scores instead, which writes no per-tile histograms), and an upper bound
// of it for any device.
int64_t index_score_tiles(const ScoreArgs& a);
int64_t index_score_tiles_bound(int64_t n_max);
hipError_t launch_pool_score(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                             int64_t k_rstride, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                             int B, int Tq, int H_I, int D_I, int k_top, uint32_t* keys, int64_t key_stride,
                             int32_t* n_valid, const SelectWs& ws, hipStream_t s);

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
};
int attn_num_splits(int64_t rows, int k_top, int W);
size_t attn_ws_bytes(int64_t rows, int H, int d_v, int splits);
hipError_t launch_sparse_attn(const AttnArgs& a, bool prefill, void* ws, hipStream_t s);

}  // namespace csa2
