// Exact per-row Top-K by radix select over order-preserving u32 keys.
//
// Selection rule (the indexer keeps its top-k tokens -- techniques map,
// "Checked in its code", indexer-selected sparse attention; the tie rule and
// output order are this library's): order positions by (key desc, position
// asc), keep the first k, emit them in ascending position order.
//
// With T the k-th largest key and need_eq the number of keys equal to T that
// belong to the selection, the selection is {key > T} plus the need_eq
// lowest positions with key == T.  The producer (the scoring kernel) writes
// the keys and a histogram of their top 12 bits.  Then:
//   collect  -- every workgroup resolves the threshold bucket from the
//               histogram itself, counts its tile's keys above the bucket,
//               appends the bucket's keys as (key, position) candidates and
//               lists, in position order, the tile's positions at or above
//               the bucket (when at most kTileList of them); the row's
//               first workgroup also records the resolved first digit;
//   finalize -- one workgroup per row finds T and need_eq among the
//               candidates (two more radix digits, in LDS), every tile's
//               output offset, the -1 padding and the pool length;
//   emit     -- every tile writes its selected positions in ascending order,
//               from its list (or from all its keys when the list overflowed).
// No workgroup waits for or elects another; kernel boundaries order the
// passes.  The key array is read once in full after it is written.
#include "common.h"
#include "internal.h"
#include "select_dev.h"

namespace csa2 {

static __host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

static int64_t sel_tiles(int64_t n_max) {
  int64_t t = (n_max + kSelTile - 1) / kSelTile;
  return t < 1 ? 1 : t;
}
static int64_t sel_cap(int64_t n_max) { return ((n_max > 0 ? n_max : 1) + 63) / 64 * 64; }

size_t select_ws_bytes(int64_t rows, int64_t n_max) {
  const int64_t tiles = sel_tiles(n_max), cap = sel_cap(n_max);
  size_t b = 0;
  b += align256(sizeof(SelectRowCtl) * rows);
  b += align256(sizeof(uint32_t) * 4096 * rows);
  b += align256(sizeof(uint32_t) * 2 * cap * rows);
  b += 4 * align256(sizeof(uint32_t) * tiles * rows);
  b += align256(sizeof(uint16_t) * kTileList * tiles * rows);
  return b;
}

SelectWs select_ws_carve(void* base, int64_t rows, int64_t n_max) {
  const int64_t tiles = sel_tiles(n_max), cap = sel_cap(n_max);
  char* p = (char*)base;
  SelectWs w;
  w.ctl = (SelectRowCtl*)p; p += align256(sizeof(SelectRowCtl) * rows);
  w.hist1 = (uint32_t*)p; p += align256(sizeof(uint32_t) * 4096 * rows);
  w.cand = (uint32_t*)p; p += align256(sizeof(uint32_t) * 2 * cap * rows);
  w.tile_gt = (uint32_t*)p; p += align256(sizeof(uint32_t) * tiles * rows);
  w.tile_off = (uint32_t*)p; p += align256(sizeof(uint32_t) * tiles * rows);
  w.tile_eqb = (uint32_t*)p; p += align256(sizeof(uint32_t) * tiles * rows);
  w.tile_cnt = (uint32_t*)p; p += align256(sizeof(uint32_t) * tiles * rows);
  w.tlist = (uint16_t*)p;
  w.cand_cap = cap;
  w.tiles = tiles;
  return w;
}

// ------------------------------------------------------------- kernels ---

__global__ void select_clear_kernel(uint32_t* p, int64_t n_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// The 16 keys a thread handles: positions base + 1024*i + 4*tid + j
// (i, j = 0..3), loaded as four 16-byte vectors (coalesced across the
// workgroup) before any of them is used.  Positions at or past nv read as 0
// (absent); rows are padded to a multiple of 64 keys, so a vector that starts
// below nv stays inside the row.  Ordering by (i, tid, j) is position order.
__device__ __forceinline__ void load_tile_keys(const uint32_t* kr, int64_t base, int64_t nv, uint32_t (&k)[16]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t p = base + 4 * ((int64_t)threadIdx.x + 256 * i);
    v4u v = {0u, 0u, 0u, 0u};
    if (p < nv) v = *reinterpret_cast<const v4u*>(kr + p);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[4 * i + j] = (p + j < nv) ? v[j] : 0u;
  }
}

// collect: counts above the threshold bucket per tile; appends the bucket;
// lists the tile's positions at or above the bucket in position order.
__global__ void __launch_bounds__(256)
select_collect_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                      const int32_t* __restrict__ n_valid, int k) {
  __shared__ uint32_t red[4], res[4];
  __shared__ uint32_t slot0, ltot[2];
  const int64_t row = blockIdx.y;
  const int64_t nv = n_valid[row];
  const int64_t base = (int64_t)blockIdx.x * kSelTile;
  uint32_t kk[16];
  load_tile_keys(keys + row * key_stride, base, nv, kk);   // in flight during the resolution
  const Level1 L = resolve_level1(ws.hist1 + row * 4096, (uint32_t)k, red, res);
  if (blockIdx.x == 0 && threadIdx.x == 0) {   // published for the finalize pass
    SelectRowCtl& c = ws.ctl[row];
    c.l1_total = L.total; c.l1_mode = L.mode; c.l1_d = L.d; c.l1_above = L.above; c.l1_cnt = L.cnt;
  }
  uint32_t gt = 0, nc = 0;
  uint32_t nl[4] = {0u, 0u, 0u, 0u};   // listed keys per round i
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool valid = kk[i] != 0u;
    const uint32_t bkt = kk[i] >> 20;
    if (L.mode == 1u) gt += valid;
    else if (L.mode == 2u) gt += valid && bkt >= L.d;
    else {
      gt += valid && bkt > L.d;
      nc += valid && bkt == L.d;
    }
    nl[i >> 2] += valid && (L.mode == 1u || bkt >= L.d);
  }
  const int64_t tix = row * ws.tiles + blockIdx.x;
  const uint32_t g_incl = block_prefix_sum_256(gt, red);
  if (threadIdx.x == 255) ws.tile_gt[tix] = g_incl;
  // Per-round prefix sums, two rounds per word (16-bit fields; a round holds
  // at most 1024 keys).
  const uint32_t w01 = nl[0] | (nl[1] << 16), w23 = nl[2] | (nl[3] << 16);
  const uint32_t i01 = block_prefix_sum_256(w01, red);
  const uint32_t i23 = block_prefix_sum_256(w23, red);
  if (threadIdx.x == 255) { ltot[0] = i01; ltot[1] = i23; }
  __syncthreads();
  const uint32_t t0 = ltot[0] & 0xFFFFu, t1 = ltot[0] >> 16, t2 = ltot[1] & 0xFFFFu, t3 = ltot[1] >> 16;
  const uint32_t count = t0 + t1 + t2 + t3;
  if (threadIdx.x == 0) ws.tile_cnt[tix] = count <= (uint32_t)kTileList ? count : ~0u;
  if (count <= (uint32_t)kTileList) {
    const uint32_t ex01 = i01 - w01, ex23 = i23 - w23;
    const uint32_t start[4] = {ex01 & 0xFFFFu, t0 + (ex01 >> 16), t0 + t1 + (ex23 & 0xFFFFu),
                               t0 + t1 + t2 + (ex23 >> 16)};
    uint16_t* lst = ws.tlist + tix * kTileList;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t at = start[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t key = kk[4 * i + j];
        if (key != 0u && (L.mode == 1u || (key >> 20) >= L.d))
          lst[at++] = (uint16_t)(1024 * i + 4 * threadIdx.x + j);
      }
    }
  }
  if (L.mode != 0u) return;
  const uint32_t c_incl = block_prefix_sum_256(nc, red);
  if (threadIdx.x == 255) slot0 = c_incl ? atomicAdd(&ws.ctl[row].cand_count, c_incl) : 0u;
  __syncthreads();
  if (nc == 0u) return;
  uint32_t slot = slot0 + c_incl - nc;
  uint32_t* cr = ws.cand + row * 2 * ws.cand_cap;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (kk[i] != 0u && (kk[i] >> 20) == L.d) {
      cr[2 * slot] = kk[i];
      cr[2 * slot + 1] = (uint32_t)(base + 4 * ((int64_t)threadIdx.x + 256 * (i >> 2)) + (i & 3));
      ++slot;
    }
  }
}

__device__ __forceinline__ uint32_t block_sum_256(uint32_t v, uint32_t* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  const uint32_t t = red[0] + red[1] + red[2] + red[3];
  __syncthreads();
  return t;
}

constexpr int kCandLds = 4096;   // candidates staged in LDS by the finalize pass

// finalize (one workgroup per row): the exact threshold T and tie count from
// the candidates (staged in LDS when they fit), every tile's output offset
// and the ties before it, the -1 padding and the pool length.
__global__ void __launch_bounds__(256)
select_finalize_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                       const int32_t* __restrict__ n_valid, int k, SelectOut out) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t ck[kCandLds], cp[kCandLds];
  __shared__ uint32_t tsel[kMaxSelTiles], teq[kMaxSelTiles];
  __shared__ uint32_t red[4], res[4];
  __shared__ uint32_t carry[2];
  const int64_t row = blockIdx.x;
  const int64_t tiles = ws.tiles;
  // The first 256 tiles' counts are loaded up front (their latency overlaps
  // the candidate staging and the digit passes).
  const uint32_t gt_pre = threadIdx.x < tiles ? ws.tile_gt[row * tiles + threadIdx.x] : 0u;
  const int64_t nv = n_valid[row];
  // First-digit state as the collect pass resolved it from the histogram.
  const SelectRowCtl& c0 = ws.ctl[row];
  const Level1 L{c0.l1_total, c0.l1_mode, c0.l1_d, c0.l1_above, c0.l1_cnt};
  const uint32_t nc = L.mode == 0u ? c0.cand_count : 0u;
  const uint32_t* cr = ws.cand + row * 2 * ws.cand_cap;
  const bool in_lds = nc <= (uint32_t)kCandLds;
  if (in_lds) {
    for (uint32_t c = threadIdx.x; c < nc; c += 256) {
      ck[c] = cr[2 * c];
      cp[c] = cr[2 * c + 1];
    }
  }
  for (int64_t t = threadIdx.x; t < tiles; t += 256) {
    tsel[t] = 0u;
    teq[t] = 0u;
  }
  __syncthreads();
  auto cand_key = [&](uint32_t c) { return in_lds ? ck[c] : cr[2 * c]; };
  auto cand_pos = [&](uint32_t c) { return in_lds ? cp[c] : cr[2 * c + 1]; };
  uint32_t thr, need_eq, total;
  if (L.mode == 1u) {
    thr = 0u; need_eq = 0u; total = L.total;
  } else if (L.mode == 2u) {
    thr = (L.d << 20) - 1u; need_eq = 0u; total = (uint32_t)k;
  } else {
    total = (uint32_t)k;
    const uint32_t need = (uint32_t)k - L.above;
    for (int i = threadIdx.x; i < 4096; i += 256) hist[i] = 0u;
    __syncthreads();
    for (uint32_t c = threadIdx.x; c < nc; c += 256) atomicAdd(&hist[(cand_key(c) >> 8) & 0xFFFu], 1u);
    __syncthreads();
    const Digit A = resolve_digit<4096>(hist, need, red, res);
    const uint32_t need2 = need - A.above;
    if (need2 == A.cnt) {
      thr = (((L.d << 12) | A.d) << 8) - 1u;
      need_eq = 0u;
    } else {
      for (int i = threadIdx.x; i < 256; i += 256) hist[i] = 0u;
      __syncthreads();
      for (uint32_t c = threadIdx.x; c < nc; c += 256) {
        const uint32_t key = cand_key(c);
        if (((key >> 8) & 0xFFFu) == A.d) atomicAdd(&hist[key & 0xFFu], 1u);
      }
      __syncthreads();
      const Digit Bd = resolve_digit<256>(hist, need2, red, res);
      thr = (L.d << 20) | (A.d << 8) | Bd.d;
      need_eq = need2 - Bd.above;
    }
  }
  // Selected candidates and ties per tile.
  uint32_t eq_all = 0;
  for (uint32_t c = threadIdx.x; c < nc; c += 256) {
    const uint32_t key = cand_key(c), tile = cand_pos(c) / kSelTile;
    if (key > thr) atomicAdd(&tsel[tile], 1u);
    else if (key == thr) {
      atomicAdd(&teq[tile], 1u);
      ++eq_all;
    }
  }
  if (threadIdx.x == 0) { carry[0] = 0u; carry[1] = 0u; }
  eq_all = block_sum_256(eq_all, red);
  // Exclusive scan over tiles, 256 at a time with a running carry.
  for (int64_t t0 = 0; t0 < tiles; t0 += 256) {
    const int64_t t = t0 + threadIdx.x;
    uint32_t g = 0, e = 0;
    if (t < tiles) {
      g = (t0 == 0 ? gt_pre : ws.tile_gt[row * tiles + t]) + tsel[t];
      e = teq[t];
    }
    const uint32_t c_out = carry[0], c_eq = carry[1];
    const uint32_t e_incl = block_prefix_sum_256(e, red);
    const uint32_t eq_before = c_eq + e_incl - e;
    uint32_t take = 0;
    if (need_eq > eq_before) take = (need_eq - eq_before) < e ? (need_eq - eq_before) : e;
    const uint32_t sel = g + take;
    const uint32_t s_incl = block_prefix_sum_256(sel, red);
    if (t < tiles) {
      ws.tile_off[row * tiles + t] = c_out + s_incl - sel;
      ws.tile_eqb[row * tiles + t] = eq_before;
    }
    __syncthreads();
    if (threadIdx.x == 255) { carry[0] = c_out + s_incl; carry[1] = c_eq + e_incl; }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    ws.ctl[row].thr = thr;
    ws.ctl[row].need_eq = need_eq;
    ws.ctl[row].total = total;
  }
  // Padding.
  if (out.expand == 0) {
    int32_t* oi = out.idx + row * (int64_t)k;
    float* os = out.score ? out.score + row * (int64_t)k : nullptr;
    for (int64_t i = total + threadIdx.x; i < k; i += 256) {
      oi[i] = -1;
      if (os) os[i] = -__builtin_inff();
    }
  } else {
    const int64_t cap = (int64_t)k * out.expand;
    int32_t* oi = out.idx + row * cap;
    for (int64_t i = (int64_t)total * out.expand + threadIdx.x; i < cap; i += 256) oi[i] = -1;
    if (threadIdx.x == 0) {
      // Only the last block of the row can be partial; it is selected when
      // it is above T, or at T with every tie taken (it is the last tie).
      int32_t len = (int32_t)(total * out.expand);
      if (nv > 0) {
        const uint32_t klast = keys[row * key_stride + nv - 1];
        const bool sel_last = L.mode == 1u || klast > thr || (klast == thr && eq_all <= need_eq);
        if (sel_last) len -= (int32_t)(nv * out.expand - out.expand_limit[row]);
      }
      out.pool_len[row] = len;
    }
  }
}

// emit: the selected positions of each tile, in ascending order.
__global__ void __launch_bounds__(256)
select_emit_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                   const int32_t* __restrict__ n_valid, int k, SelectOut out) {
  constexpr int PER = kSelTile / 256;  // consecutive positions per thread
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.y;
  const int64_t tiles = ws.tiles;
  const int64_t nv = n_valid[row];
  const int64_t base = (int64_t)blockIdx.x * kSelTile;
  if (base >= nv) return;
  const uint32_t* kr = keys + row * key_stride;
  const int64_t tix = row * tiles + blockIdx.x;
  const uint32_t cnt = ws.tile_cnt[tix];
  if (cnt != ~0u) {
    // The tile's positions at or above the threshold bucket, in position
    // order: thread t takes list entries 2t and 2t+1.
    const uint16_t* lst = ws.tlist + tix * kTileList;
    const uint32_t thr = ws.ctl[row].thr, need_eq = ws.ctl[row].need_eq;
    const uint32_t off0 = ws.tile_off[tix];
    const uint32_t eqb0 = ws.tile_eqb[tix];
    uint32_t lk[2];
    int64_t lp[2];
    bool lh[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t c = 2 * threadIdx.x + q;
      lh[q] = c < cnt;
      lp[q] = base + (lh[q] ? lst[c] : 0);
      lk[q] = lh[q] ? kr[lp[q]] : 0u;
    }
    uint32_t n_eq = 0, n_gt = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      n_gt += lh[q] && lk[q] > thr;
      n_eq += lh[q] && lk[q] == thr;
    }
    const uint32_t eq_incl = block_prefix_sum_256(n_eq, red);
    const uint32_t eq_rank = eqb0 + eq_incl - n_eq;
    uint32_t my_take = 0;
    if (need_eq > eq_rank) my_take = (need_eq - eq_rank) < n_eq ? (need_eq - eq_rank) : n_eq;
    const uint32_t sel = n_gt + my_take;
    const uint32_t sel_incl = block_prefix_sum_256(sel, red);
    uint32_t slot = off0 + sel_incl - sel;
    uint32_t taken_eq = 0;
    const int32_t* map = out.map ? out.map + row * out.map_stride : nullptr;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      if (!lh[q]) break;
      bool take = lk[q] > thr;
      if (!take && lk[q] == thr) {
        take = taken_eq < my_take;
        ++taken_eq;
      }
      if (!take) continue;
      if (slot >= (uint32_t)k) break;
      if (out.expand == 0) {
        const int32_t id = map ? map[lp[q]] : (int32_t)lp[q];
        out.idx[row * (int64_t)k + slot] = id;
        if (out.score) out.score[row * (int64_t)k + slot] = key_score(lk[q]);
      } else {
        const int64_t cap = (int64_t)k * out.expand;
        const int32_t lim = out.expand_limit[row];
        for (int u = 0; u < out.expand; ++u) {
          const int64_t id = lp[q] * out.expand + u;
          out.idx[row * cap + (int64_t)slot * out.expand + u] = id < lim ? (int32_t)id : -1;
        }
      }
      ++slot;
    }
    return;
  }
  const int64_t p0 = base + (int64_t)threadIdx.x * PER;
  uint32_t kk[PER];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    v4u v = {0u, 0u, 0u, 0u};
    if (p0 + 4 * i < nv) v = *reinterpret_cast<const v4u*>(kr + p0 + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) kk[4 * i + j] = (p0 + 4 * i + j < nv) ? v[j] : 0u;
  }
  const uint32_t thr = ws.ctl[row].thr, need_eq = ws.ctl[row].need_eq;
  const uint32_t off0 = ws.tile_off[tix];
  const uint32_t eqb0 = ws.tile_eqb[tix];
  uint32_t n_eq = 0, n_gt = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    bool valid = p0 + i < nv;
    n_gt += valid && kk[i] > thr;
    n_eq += valid && kk[i] == thr;
  }
  uint32_t eq_incl = block_prefix_sum_256(n_eq, red);
  uint32_t eq_rank = eqb0 + eq_incl - n_eq;          // global tie rank of my first tie
  uint32_t my_take = 0;
  if (need_eq > eq_rank) my_take = (need_eq - eq_rank) < n_eq ? (need_eq - eq_rank) : n_eq;
  uint32_t sel = n_gt + my_take;
  uint32_t sel_incl = block_prefix_sum_256(sel, red);
  uint32_t slot = off0 + sel_incl - sel;
  uint32_t taken_eq = 0;
  const int32_t* map = out.map ? out.map + row * out.map_stride : nullptr;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    int64_t pos = p0 + i;
    if (pos >= nv) break;
    bool take = kk[i] > thr;
    if (!take && kk[i] == thr) {
      take = taken_eq < my_take;
      ++taken_eq;
    }
    if (!take) continue;
    if (slot >= (uint32_t)k) break;   // never write past the row (cannot happen when counts agree)
    if (out.expand == 0) {
      int32_t id = map ? map[pos] : (int32_t)pos;
      out.idx[row * (int64_t)k + slot] = id;
      if (out.score) out.score[row * (int64_t)k + slot] = key_score(kk[i]);
    } else {
      const int64_t cap = (int64_t)k * out.expand;
      const int32_t lim = out.expand_limit[row];
      for (int u = 0; u < out.expand; ++u) {
        int64_t id = pos * out.expand + u;
        out.idx[row * cap + (int64_t)slot * out.expand + u] = id < lim ? (int32_t)id : -1;
      }
    }
    ++slot;
  }
}

// small: the whole selection of a row in one 1024-thread workgroup when the
// row has at most kSmallSel positions (pool layers, short contexts).  The
// row is cut into 4 groups of 4096 positions; thread t holds positions
// 4t .. 4t+3 of every group (and their map entries) in registers, so each
// load instruction of a wave reads 1 KB of consecutive keys.  Three radix
// digits (12, 12, 8 bits) over the row's keys give T and the ties to take,
// with one LDS histogram per level cleared together at the start.  The
// output offsets follow position order, (group, thread, element): one
// prefix sum over threads of four packed (above T, equal to T) counts, one
// per group, plus the totals of the earlier groups.  No global histogram,
// no clear pass.
constexpr int kSmallThreads = 1024;
constexpr int kSmallGroups = 4;
static_assert(kSmallSel == 4 * kSmallGroups * kSmallThreads, "4 positions per thread and group");

// Digit of a BINS-bin LDS histogram (4096 or 256) at which the count from
// the top reaches `need`, as (d, count above d, count at d); `total` gets the
// histogram's sum (the digit is meaningless when need > total).  Thread t
// reads bins 4g .. 4g+3 of group g = BINS/4 - 1 - t, so a prefix sum over
// threads counts from the top.
template <int BINS>
__device__ Digit small_digit(const uint32_t* hist, uint32_t need, uint32_t* red, uint32_t* res, uint32_t& total) {
  constexpr int G = BINS / 4;
  static_assert(G == kSmallThreads || G == 64, "one group per thread or per lane of the first wave");
  if (G == kSmallThreads || threadIdx.x < 64) {
    const int g = G - 1 - threadIdx.x;
    const v4u h = reinterpret_cast<const v4u*>(hist)[g];
    const uint32_t sum = h[0] + h[1] + h[2] + h[3];
    const uint32_t incl = G == kSmallThreads ? block_scan<kSmallThreads>(sum, red) : wave_prefix_sum(sum);
    if (threadIdx.x == G - 1) res[4] = incl;
    uint32_t run = incl - sum;
    if (run < need && need <= incl) {
#pragma unroll
      for (int j = 3; j >= 0; --j) {
        if (run < need && need <= run + h[j]) {
          res[0] = 4 * g + j;
          res[1] = run;
          res[2] = h[j];
        }
        run += h[j];
      }
    }
  }
  __syncthreads();
  total = res[4];
  return Digit{res[0], res[1], res[2]};
}

__global__ void __launch_bounds__(kSmallThreads)
select_small_kernel(const uint32_t* __restrict__ keys, int64_t key_stride, const int32_t* __restrict__ n_valid, int k,
                    SelectOut out) {
  constexpr int NT = kSmallThreads, NG = kSmallGroups, GS = 4 * NT, PT = 4 * NG;
  constexpr int NWV = NT / 64;
  __shared__ __align__(16) uint32_t hist0[4096];
  __shared__ __align__(16) uint32_t hist1[4096];
  __shared__ __align__(16) uint32_t hist2[256];
  __shared__ __align__(16) uint32_t red[NG * NWV];
  __shared__ uint32_t res[5];
  const int64_t row = blockIdx.x;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 1024; i += NT) {
    reinterpret_cast<v4u*>(hist0)[i] = v4u{0u, 0u, 0u, 0u};
    reinterpret_cast<v4u*>(hist1)[i] = v4u{0u, 0u, 0u, 0u};
  }
  if (threadIdx.x < 64) reinterpret_cast<v4u*>(hist2)[threadIdx.x] = v4u{0u, 0u, 0u, 0u};
  int64_t nv = n_valid[row];
  if (nv > kSmallSel) nv = kSmallSel;   // (the host guarantees it)
  const uint32_t* kr = keys + row * key_stride;
  const int32_t* map = out.map ? out.map + row * out.map_stride : nullptr;
  // kk[4g + j] is position g*GS + 4t + j.
  uint32_t kk[PT];
  int32_t mp[PT];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int p = g * GS + 4 * threadIdx.x;
    // rows are padded to a multiple of 64 keys: a vector starting below nv
    // stays inside the row
    v4u v = {0u, 0u, 0u, 0u};
    if (p < nv) v = *reinterpret_cast<const v4u*>(kr + p);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      kk[4 * g + j] = p + j < nv ? v[j] : 0u;
      mp[4 * g + j] = p + j;
    }
  }
  if (map) {
    if (((uintptr_t)map & 15u) == 0) {
      // the map row holds at least nv entries, but not a whole last vector
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int p = g * GS + 4 * threadIdx.x;
        if (p + 3 < nv) {
          const v4u m = *reinterpret_cast<const v4u*>(map + p);
#pragma unroll
          for (int j = 0; j < 4; ++j) mp[4 * g + j] = (int32_t)m[j];
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (p + j < nv) mp[4 * g + j] = map[p + j];
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < PT; ++e) {
        const int p = (e >> 2) * GS + 4 * threadIdx.x + (e & 3);
        if (p < nv) mp[e] = map[p];
      }
    }
  }
  __syncthreads();   // histograms cleared
  // Threshold T and ties to take; every visible position (key != 0) when
  // there are at most k of them.
  bool take_all = nv <= k;
  uint32_t thr = 0u, need_eq = 0u;
  if (!take_all) {
#pragma unroll
    for (int e = 0; e < PT; ++e)
      if (kk[e]) atomicAdd(&hist0[kk[e] >> 20], 1u);
    __syncthreads();
    uint32_t total;
    const Digit D0 = small_digit<4096>(hist0, (uint32_t)k, red, res, total);
    if (total <= (uint32_t)k) {
      take_all = true;
    } else {
      uint32_t need = (uint32_t)k - D0.above, prefix = D0.d;
      if (need == D0.cnt) {   // the whole bucket is taken
        thr = prefix ? (prefix << 20) - 1u : 0u;
      } else {
#pragma unroll
        for (int e = 0; e < PT; ++e)
          if (kk[e] != 0u && (kk[e] >> 20) == prefix) atomicAdd(&hist1[(kk[e] >> 8) & 0xFFFu], 1u);
        __syncthreads();
        const Digit D1 = small_digit<4096>(hist1, need, red, res, total);
        need -= D1.above;
        prefix = (prefix << 12) | D1.d;
        if (need == D1.cnt) {
          thr = prefix ? (prefix << 8) - 1u : 0u;
        } else {
#pragma unroll
          for (int e = 0; e < PT; ++e)
            if (kk[e] != 0u && (kk[e] >> 8) == prefix) atomicAdd(&hist2[kk[e] & 0xFFu], 1u);
          __syncthreads();
          const Digit D2 = small_digit<256>(hist2, need, red, res, total);
          thr = (prefix << 8) | D2.d;
          need_eq = need - D2.above;
        }
      }
    }
  }
  // Emission: ties at T go to the lowest positions.  Per group, the counts
  // above T and at T are packed in one word (each total is at most 4096).
  uint32_t cnt[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = kk[4 * g + j];
      gt += x != 0u && (take_all || x > thr);
      eq += !take_all && x != 0u && x == thr;
    }
    cnt[g] = (gt << 16) | eq;
  }
  uint32_t incl[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) incl[g] = wave_prefix_sum(cnt[g]);
  if (lane == 63) {
#pragma unroll
    for (int g = 0; g < NG; ++g) red[g * NWV + wv] = incl[g];
  }
  __syncthreads();
  uint32_t base = 0;   // packed totals of the earlier groups
  uint32_t before[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    uint32_t waves_before = 0, group_total = 0;
#pragma unroll
    for (int q = 0; q < NWV / 4; ++q) {
      const v4u r = reinterpret_cast<const v4u*>(red + g * NWV)[q];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        waves_before += 4 * q + j < wv ? r[j] : 0u;
        group_total += r[j];
      }
    }
    before[g] = base + waves_before + incl[g] - cnt[g];
    base += group_total;
  }
  int32_t* oi = out.idx + row * (int64_t)k;
  float* os = out.score ? out.score + row * (int64_t)k : nullptr;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const uint32_t eq_before = before[g] & 0xFFFFu;
    uint32_t slot = (before[g] >> 16) + (eq_before < need_eq ? eq_before : need_eq);
    const uint32_t eq = cnt[g] & 0xFFFFu;
    uint32_t take = 0;
    if (need_eq > eq_before) take = need_eq - eq_before < eq ? need_eq - eq_before : eq;
    uint32_t taken = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t x = kk[4 * g + j];
      if (x == 0u) continue;
      bool pick = take_all || x > thr;
      if (!pick && x == thr && taken < take) {
        pick = true;
        ++taken;
      }
      if (pick && slot < (uint32_t)k) {
        oi[slot] = mp[4 * g + j];
        if (os) os[slot] = key_score(x);
        ++slot;
      }
    }
  }
  // Exactly k are selected unless every visible position is.
  if (take_all) {
    for (int64_t i = (base >> 16) + threadIdx.x; i < k; i += NT) {
      oi[i] = -1;
      if (os) os[i] = -__builtin_inff();
    }
  }
}

// ---------------------------------------------------------------- host ---

hipError_t select_small(const uint32_t* keys, int64_t key_stride, const int32_t* n_valid, int64_t rows, int k,
                        const SelectOut& out, hipStream_t s) {
  if (out.expand != 0) return hipErrorInvalidValue;
  CSA2_LAUNCH("select_small", select_small_kernel, dim3((unsigned)rows), dim3(kSmallThreads), 0, s, keys, key_stride,
              n_valid, k, out);
  return hipGetLastError();
}

hipError_t select_clear(const SelectWs& ws, int64_t rows, hipStream_t s) {
  // ctl and hist1 are carved contiguously.
  int64_t words = (int64_t)((char*)(ws.hist1 + 4096 * rows) - (char*)ws.ctl) / 4;
  int64_t grid = (words + 1023) / 1024;
  if (grid > 2048) grid = 2048;
  CSA2_LAUNCH("select_clear", select_clear_kernel, dim3((unsigned)grid), dim3(256), 0, s, (uint32_t*)ws.ctl,
              words);
  return hipGetLastError();
}

hipError_t select_finish(const SelectWs& ws, const uint32_t* keys, int64_t key_stride, const int32_t* n_valid,
                         int64_t rows, int k, const SelectOut& out, hipStream_t s) {
  dim3 grid((unsigned)ws.tiles, (unsigned)rows);
  CSA2_LAUNCH("select_collect", select_collect_kernel, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid, k);
  CSA2_LAUNCH("select_finalize", select_finalize_kernel, dim3((unsigned)rows), dim3(256), 0, s, ws, keys, key_stride,
              n_valid, k, out);
  CSA2_LAUNCH("select_emit", select_emit_kernel, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid, k, out);
  return hipGetLastError();
}

}  // namespace csa2
