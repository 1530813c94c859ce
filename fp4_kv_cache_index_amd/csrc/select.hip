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
//   level1   -- (many tiles) one workgroup per row resolves the threshold
//               bucket (the first digit) from the histogram and records it;
//               with few tiles every collect workgroup resolves it itself;
//   collect  -- every workgroup counts its tile's keys above the bucket,
//               appends the bucket's keys as (key, position) candidates and
//               lists, in position order, the tile's positions at or above
//               the bucket (when at most kTileList of them);
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

// Zeroes n0 words at p0, then n1 words at p1 (a second region in the same
// launch: the token and block states of a pool scan).
__global__ void select_clear_kernel(uint32_t* p0, int64_t n0, uint32_t* p1, int64_t n1) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n0 + n1;
       i += (int64_t)gridDim.x * blockDim.x) {
    if (i < n0) p0[i] = 0u;
    else p1[i - n0] = 0u;
  }
}

// The 16 keys a thread handles: positions base + 1024*i + 4*tid + j
// (i, j = 0..3), loaded as four 16-byte vectors (coalesced across the
// workgroup) before any of them is used.  The loads go through a buffer
// descriptor whose range ends at nv rounded up to a whole vector (rows are
// padded to a multiple of 64 keys, so that stays inside the row): every lane
// issues the same four loads with no branch, hence no wait between them, and
// vectors past the range read 0.  Positions at or past nv are then cleared.
// Ordering by (i, tid, j) is position order.
__device__ __forceinline__ void load_tile_keys(const uint32_t* kr, int64_t base, int64_t nv, uint32_t (&k)[16]) {
  const int64_t rem = nv - base;
  const int bytes = rem <= 0 ? 0 : (rem >= kSelTile ? 4 * kSelTile : 4 * (int)((rem + 3) & ~3LL));
  const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kr + base), (short)0, bytes, 0x00020000);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = 4 * ((int)threadIdx.x + 256 * i);
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * q, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) k[4 * i + j] = (base + q + j < nv) ? v[j] : 0u;
  }
}

// level 1: one workgroup per row resolves the first digit from the row's
// histogram and records it for the collect and finalize passes (rows with
// many tiles: each collect workgroup would read the 16 KB histogram, as many
// bytes as its keys).
constexpr int64_t kLevel1Pass = 16384;   // collect workgroups from which the pass pays
__global__ void __launch_bounds__(256) select_level1_kernel(SelectWs ws, int k) {
  __shared__ uint32_t red[4], res[4];
  const int64_t row = blockIdx.x;
  const Level1 L = resolve_level1(ws.hist1 + row * 4096, (uint32_t)k, red, res);
  if (threadIdx.x == 0) {
    SelectRowCtl& c = ws.ctl[row];
    c.l1_total = L.total; c.l1_mode = L.mode; c.l1_d = L.d; c.l1_above = L.above; c.l1_cnt = L.cnt;
  }
}

// collect: counts above the threshold bucket per tile; appends the bucket;
// lists the tile's positions at or above the bucket in position order.
// With PRE the level-1 pass has recorded the first digit; otherwise every
// workgroup resolves it from the histogram (cheaper when the row has few
// tiles than one more launch) and the row's first one records it.
template <bool PRE>
__global__ void __launch_bounds__(256)
select_collect_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                      const int32_t* __restrict__ n_valid, int k) {
  __shared__ uint32_t red[4], res[PRE ? 1 : 4];
  __shared__ uint32_t slot0, ltot[2];
  const int64_t row = blockIdx.y;
  const int64_t nv = n_valid[row];
  const int64_t base = (int64_t)blockIdx.x * kSelTile;
  uint32_t kk[16];
  load_tile_keys(keys + row * key_stride, base, nv, kk);   // in flight during the resolution
  Level1 L;
  if constexpr (PRE) {
    const SelectRowCtl& c = ws.ctl[row];
    L = Level1{c.l1_total, c.l1_mode, c.l1_d, c.l1_above, c.l1_cnt};
  } else {
    L = resolve_level1(ws.hist1 + row * 4096, (uint32_t)k, red, res);
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      SelectRowCtl& c = ws.ctl[row];
      c.l1_total = L.total; c.l1_mode = L.mode; c.l1_d = L.d; c.l1_above = L.above; c.l1_cnt = L.cnt;
    }
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
      // it is above T, or at T when ties are taken at all and every one of
      // them is (it is the last tie).  With need_eq == 0, T is the key just
      // below the selection (a whole bucket or sub-bucket taken), and a
      // block whose key equals it is not selected.
      int32_t len = (int32_t)(total * out.expand);
      if (nv > 0) {
        const uint32_t klast = keys[row * key_stride + nv - 1];
        const bool sel_last =
            L.mode == 1u || klast > thr || (klast == thr && need_eq > 0u && eq_all <= need_eq);
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
  // The pass's control words, all requested at once.
  const uint32_t cnt = ws.tile_cnt[tix];
  const uint32_t thr = ws.ctl[row].thr, need_eq = ws.ctl[row].need_eq;
  const uint32_t off0 = ws.tile_off[tix];
  const uint32_t eqb0 = ws.tile_eqb[tix];
  if (cnt != ~0u) {
    // The tile's positions at or above the threshold bucket, in position
    // order: thread t takes list entries 2t and 2t+1.
    const uint16_t* lst = ws.tlist + tix * kTileList;
    uint32_t lk[2];
    int64_t lp[2];
    bool lh[2];
    // Both list entries first (their slots always exist), then both keys
    // from selected addresses: two round trips, with no branch between loads.
    static_assert(2 * 256 == kTileList, "two list slots per thread");
    uint32_t le[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) le[q] = lst[2 * threadIdx.x + q];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      lh[q] = 2 * threadIdx.x + q < cnt;
      lp[q] = base + (lh[q] ? le[q] : 0u);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q) lk[q] = kr[lp[q]];
#pragma unroll
    for (int q = 0; q < 2; ++q) lk[q] = lh[q] ? lk[q] : 0u;
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
  {
    // (as in load_tile_keys: a descriptor ending at nv rounded up to a
    // vector, unconditional loads, positions past nv cleared)
    const int64_t rem = nv - base;
    const int bytes = rem >= kSelTile ? 4 * kSelTile : 4 * (int)((rem + 3) & ~3LL);
    const auto rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(kr + base), (short)0, bytes, 0x00020000);
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) {
      const v4u v = __builtin_amdgcn_raw_buffer_load_b128(rs, 4 * (PER * (int)threadIdx.x + 4 * i), 0, 0);
#pragma unroll
      for (int j = 0; j < 4; ++j) kk[4 * i + j] = (p0 + 4 * i + j < nv) ? v[j] : 0u;
    }
  }
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

// local: the whole selection of a row in one 1024-thread workgroup when the
// row has at most kLocalSel positions.  Wave w owns the NS*64 consecutive
// positions from w*NS*64, element s of its lane l being position
// w*NS*64 + 64s + l: each load instruction of a wave reads 256 consecutive
// bytes, and the order (wave, s, lane) is position order.
//   level 0    -- the top-12-bit histogram, summed from the producer's
//                 per-tile histograms or built here in LDS, gives the
//                 threshold bucket;
//   candidates -- when the bucket and everything above it fit in LDS
//                 (kLocalCand entries), those keys are packed there in
//                 position order, and levels 1-2 and the emission run over
//                 them; otherwise over the registers.
// Packing in position order: a wave counts its selected elements (a ballot
// and a population count per element, in scalar registers), the wave
// totals give every wave its base, and a second pass writes each selected
// element at its wave's running count plus its mbcnt rank.
constexpr int kLocalThreads = 1024;
constexpr int kLocalCand = 8192;
static_assert(kLocalSel == 64 * kLocalThreads && kLocalSelMap == 32 * kLocalThreads, "64 or 32 elements per thread");

// Inclusive prefix sum over the workgroup, plus the workgroup total.
__device__ __forceinline__ uint32_t local_scan(uint32_t v, uint32_t* red, uint32_t& total) {
  constexpr int NWV = kLocalThreads / 64;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  v = wave_prefix_sum(v);
  if (lane == 63) red[wv] = v;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int g = 0; g < NWV / 4; ++g) {
    const v4u r = reinterpret_cast<const v4u*>(red)[g];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      add += 4 * g + j < wv ? r[j] : 0u;
      tot += r[j];
    }
  }
  total = tot;
  return v + add;
}

// Digit of a 4096-bin histogram at which the count from the top reaches
// `need`, from the bins 4g .. 4g+3 (g = 1023 - thread) that each thread
// holds: (d, count above d, count at d); `total` gets the histogram's sum
// (the digit is meaningless when need > total).  `red` and `res` are LDS.
__device__ Digit local_digit_regs(const uint32_t (&h)[4], uint32_t need, uint32_t* red, uint32_t* res,
                                  uint32_t& total) {
  const int g = kLocalThreads - 1 - threadIdx.x;
  const uint32_t sum = h[0] + h[1] + h[2] + h[3];
  uint32_t tot;
  const uint32_t incl = local_scan(sum, red, tot);
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
  __syncthreads();
  total = tot;
  return Digit{res[0], res[1], res[2]};
}

// The same for an LDS histogram of 4096 or 256 bins (the latter on the
// first wave only).
template <int BINS>
__device__ Digit local_digit(const uint32_t* hist, uint32_t need, uint32_t* red, uint32_t* res) {
  if constexpr (BINS == 4096) {
    const v4u v = reinterpret_cast<const v4u*>(hist)[kLocalThreads - 1 - threadIdx.x];
    const uint32_t h[4] = {v[0], v[1], v[2], v[3]};
    uint32_t total;
    return local_digit_regs(h, need, red, res, total);
  } else {
    static_assert(BINS == 256, "4096 or 256 bins");
    if (threadIdx.x < 64) {
      const int g = 63 - threadIdx.x;
      const v4u h = reinterpret_cast<const v4u*>(hist)[g];
      const uint32_t sum = h[0] + h[1] + h[2] + h[3];
      const uint32_t incl = wave_prefix_sum(sum);
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
    return Digit{res[0], res[1], res[2]};
  }
}

__device__ __forceinline__ uint32_t lane_rank(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Base of this wave and total over the workgroup of the per-wave counts
// `cnt` (wave-uniform).  `wtot` is LDS of 16 words, read after the call.
__device__ __forceinline__ uint32_t wave_base(uint32_t cnt, uint32_t* wtot, uint32_t& total) {
  constexpr int NWV = kLocalThreads / 64;
  const int lane = threadIdx.x & 63, wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  if (lane == 0) wtot[wv] = cnt;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int g = 0; g < NWV / 4; ++g) {
    const v4u r = reinterpret_cast<const v4u*>(wtot)[g];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      base += 4 * g + j < wv ? r[j] : 0u;
      tot += r[j];
    }
  }
  total = tot;
  return base;
}

template <int NS, bool MAP, bool TH>
__global__ void __launch_bounds__(kLocalThreads)
select_local_kernel(const uint32_t* __restrict__ keys, int64_t key_stride, const int32_t* __restrict__ n_valid, int k,
                    const uint32_t* __restrict__ tile_hist, int64_t th_stride, int tiles, SelectOut out) {
  constexpr int NT = kLocalThreads, NWV = NT / 64, WS = 64 * NS;   // WS: positions per wave
  __shared__ __align__(16) uint32_t hist0[TH ? 4 : 4096];
  __shared__ __align__(16) uint32_t hist1[4096];
  __shared__ __align__(16) uint32_t hist2[256];
  __shared__ __align__(16) uint32_t red[NWV];
  __shared__ __align__(16) uint32_t wtot[2][NWV];
  // (keys and ids apart: a 64-bit pair store would tie every key register
  // to a free neighbour)
  __shared__ __align__(16) uint32_t cand_key[kLocalCand];
  __shared__ __align__(16) int32_t cand_id[kLocalCand];
  __shared__ uint32_t res[4];
  const int64_t row = blockIdx.x;
  const int t = threadIdx.x, lane = t & 63, wv = __builtin_amdgcn_readfirstlane(t >> 6);
  for (int i = t; i < 1024; i += NT) {
    if (!TH) reinterpret_cast<v4u*>(hist0)[i] = v4u{0u, 0u, 0u, 0u};
    reinterpret_cast<v4u*>(hist1)[i] = v4u{0u, 0u, 0u, 0u};
  }
  if (t < 64) reinterpret_cast<v4u*>(hist2)[t] = v4u{0u, 0u, 0u, 0u};
  int64_t nv64 = n_valid[row];
  if (nv64 > NS * NT) nv64 = NS * NT;   // (the host guarantees it)
  const int nv = (int)(nv64 < 0 ? 0 : nv64);
  const int wbase = wv * WS;            // first position of this wave
  // The first tiles' histogram words are requested before the keys, so that
  // the first digit can be resolved while the keys stream in.
  constexpr int TP = 8;
  uint2 thv[TH ? TP : 1];
  const uint2* th = TH ? reinterpret_cast<const uint2*>(tile_hist + row * th_stride * 2048) + (NT - 1 - t) : nullptr;
  if constexpr (TH) {
#pragma unroll
    for (int i = 0; i < TP; ++i) thv[i] = i < tiles && nv > k ? th[i * 1024] : uint2{0u, 0u};
  }
  // Loads through buffer descriptors, one per 1024 positions of the wave,
  // whose range ends at nv: positions at or past nv read as 0 without a
  // memory access, every lane issues the same loads (no branch, so no wait
  // between them), and the 256-byte step of s fits the instruction offset.
  auto rsrc = [&](const void* base, int q) {
    const int64_t rem = (int64_t)nv - (wbase + 1024 * q);
    const int bytes = rem <= 0 ? 0 : (rem >= 1024 ? 4096 : (int)rem * 4);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
  };
  const uint32_t* kr = keys + row * key_stride + wbase;
  uint32_t kk[NS];
#pragma unroll
  for (int q = 0; q < NS / 16; ++q) {
    const auto rk = rsrc(kr + 1024 * q, q);
#pragma unroll
    for (int s = 0; s < 16; ++s) kk[16 * q + s] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane + 256 * s, 0, 0);
  }
  int32_t mp[MAP ? NS : 1];
  if constexpr (MAP) {
    const int32_t* mr = out.map + row * out.map_stride + wbase;
#pragma unroll
    for (int q = 0; q < NS / 16; ++q) {
      const auto rm = rsrc(mr + 1024 * q, q);
#pragma unroll
      for (int s = 0; s < 16; ++s)
        mp[16 * q + s] = (int32_t)__builtin_amdgcn_raw_buffer_load_b32(rm, 4 * lane + 256 * s, 0, 0);
    }
  }
  // Output ids are recomputed from an opaque copy of the lane position, so
  // that the load addresses are not kept alive for them.
  int p_id = wbase + lane;
  asm volatile("" : "+v"(p_id));
  auto id_of = [&](int s) -> int32_t { if constexpr (MAP) return mp[s]; else return p_id + 64 * s; };
  int32_t* oi = out.idx + row * (int64_t)k;
  float* os = out.score ? out.score + row * (int64_t)k : nullptr;

  // Level 0.  When every visible position is taken (at most k of them),
  // keys above T = 0 are selected.
  bool take_all = nv <= k;
  Digit D0{0u, 0u, 0u};
  if (!take_all) {
    uint32_t h[4] = {0u, 0u, 0u, 0u};
    if constexpr (TH) {
      auto add = [&](uint2 v) {
        h[0] += v.x & 0xFFFFu;
        h[1] += v.x >> 16;
        h[2] += v.y & 0xFFFFu;
        h[3] += v.y >> 16;
      };
#pragma unroll
      for (int i = 0; i < TP; ++i) add(thv[i]);
      int i = TP;
      for (; i + 8 <= tiles; i += 8) {   // eight loads in flight
        uint2 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = th[(i + u) * 1024];
#pragma unroll
        for (int u = 0; u < 8; ++u) add(v[u]);
      }
      for (; i < tiles; ++i) add(th[i * 1024]);
      __syncthreads();   // (LDS clears)
    } else {
      __syncthreads();   // histograms cleared
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if (kk[s]) atomicAdd(&hist0[kk[s] >> 20], 1u);
      __syncthreads();
      const v4u v = reinterpret_cast<const v4u*>(hist0)[NT - 1 - t];
      h[0] = v[0]; h[1] = v[1]; h[2] = v[2]; h[3] = v[3];
    }
    uint32_t total;
    D0 = local_digit_regs(h, (uint32_t)k, red, res, total);
    take_all = total <= (uint32_t)k;
  }
  if (take_all) {
    uint32_t cnt = 0;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      cnt += (uint32_t)__popcll(__ballot(kk[s] != 0u));
      if (s % 8 == 7) __builtin_amdgcn_sched_barrier(0);   // a few masks live at a time
    }
    uint32_t n;
    uint32_t run = wave_base(cnt, wtot[0], n);
    // The writes test the elements again: an opaque bound keeps the compiler
    // from holding one condition per element across the barrier.
    uint32_t z = 0u;
    asm volatile("" : "+v"(z));
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint64_t m = __ballot(kk[s] > z);
      if (kk[s] > z) {
        const uint32_t slot = run + lane_rank(m);
        if (slot < (uint32_t)k) {
          oi[slot] = id_of(s);
          if (os) os[slot] = key_score(kk[s]);
        }
      }
      run += (uint32_t)__popcll(m);
      if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    for (int64_t i = n + t; i < k; i += NT) {
      oi[i] = -1;
      if (os) os[i] = -__builtin_inff();
    }
    return;
  }
  // T = the k-th largest key: in bucket D0.d; need1 of the bucket's keys are
  // taken.  Key 0 (absent) can lie in bucket 0 only: lo excludes it.
  const uint32_t need1 = (uint32_t)k - D0.above;
  const uint32_t lo = D0.d ? D0.d << 20 : 1u;
  uint32_t thr, need_eq = 0u;
  // Candidates: keys >= lo (D0.above + D0.cnt of them).  Counted per wave
  // first; when they fit in LDS they are packed there in position order as
  // (key, id).
  uint32_t cnt = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    cnt += (uint32_t)__popcll(__ballot(kk[s] >= lo));
    if (s % 8 == 7) __builtin_amdgcn_sched_barrier(0);   // a few masks live at a time
  }
  uint32_t ncand;
  const uint32_t base = wave_base(cnt, wtot[0], ncand);
  if (ncand <= (uint32_t)kLocalCand) {
    uint32_t lo2 = lo;   // (opaque, as above)
    asm volatile("" : "+v"(lo2));
    uint32_t run = base;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const uint64_t m = __ballot(kk[s] >= lo2);
      if (kk[s] >= lo2) {
        const uint32_t slot = run + lane_rank(m);   // < ncand
        cand_key[slot] = kk[s];
        cand_id[slot] = id_of(s);
      }
      run += (uint32_t)__popcll(m);
      if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
    __syncthreads();
    if (need1 == D0.cnt) {   // the whole bucket is taken: every candidate
      thr = lo - 1u;
    } else {
      for (uint32_t i = t; i < ncand; i += NT) {
        const uint32_t x = cand_key[i];
        if ((x >> 20) == D0.d) atomicAdd(&hist1[(x >> 8) & 0xFFFu], 1u);
      }
      __syncthreads();
      const Digit D1 = local_digit<4096>(hist1, need1, red, res);
      const uint32_t need2 = need1 - D1.above;
      const uint32_t p24 = (D0.d << 12) | D1.d;
      if (need2 == D1.cnt) {
        thr = p24 ? (p24 << 8) - 1u : 0u;
      } else {
        for (uint32_t i = t; i < ncand; i += NT) {
          const uint32_t x = cand_key[i];
          if ((x >> 8) == p24) atomicAdd(&hist2[x & 0xFFu], 1u);
        }
        __syncthreads();
        const Digit D2 = local_digit<256>(hist2, need2, red, res);
        thr = (p24 << 8) | D2.d;   // a visible key: not 0
        need_eq = need2 - D2.above;
      }
    }
    // Emission from the candidates: thread t takes a run of P consecutive
    // ones; counts above T and at T are packed (each at most kLocalCand).
    const uint32_t P = (ncand + NT - 1) / NT;
    const uint32_t c0 = t * P, c1 = c0 + P < ncand ? c0 + P : ncand;
    uint32_t gt = 0, eq = 0;
    for (uint32_t i = c0; i < c1; ++i) {
      const uint32_t x = cand_key[i];
      gt += x > thr;
      eq += x == thr;
    }
    const uint32_t c = (gt << 16) | eq;
    uint32_t tot;
    const uint32_t excl = local_scan(c, red, tot) - c;
    const uint32_t eq_before = excl & 0xFFFFu;
    uint32_t slot = (excl >> 16) + (eq_before < need_eq ? eq_before : need_eq);
    uint32_t take = need_eq > eq_before ? (need_eq - eq_before < eq ? need_eq - eq_before : eq) : 0u;
    for (uint32_t i = c0; i < c1; ++i) {
      const uint32_t x = cand_key[i];
      bool pick = x > thr;
      if (!pick && x == thr && take > 0) {
        pick = true;
        --take;
      }
      if (pick && slot < (uint32_t)k) {
        oi[slot] = cand_id[i];
        if (os) os[slot] = key_score(x);
        ++slot;
      }
    }
    return;
  }
  // Too many candidates for LDS (a crowded bucket): levels 1-2 and the
  // emission over the registers.
  {
#pragma unroll
    for (int s = 0; s < NS; ++s)
      if ((kk[s] >> 20) == D0.d && kk[s] >= lo) atomicAdd(&hist1[(kk[s] >> 8) & 0xFFFu], 1u);
    __syncthreads();
    const Digit D1 = local_digit<4096>(hist1, need1, red, res);
    const uint32_t need2 = need1 - D1.above;
    const uint32_t p24 = (D0.d << 12) | D1.d;
    if (need2 == D1.cnt) {
      thr = p24 ? (p24 << 8) - 1u : 0u;
    } else {
#pragma unroll
      for (int s = 0; s < NS; ++s)
        if ((kk[s] >> 8) == p24 && kk[s] >= lo) atomicAdd(&hist2[kk[s] & 0xFFu], 1u);
      __syncthreads();
      const Digit D2 = local_digit<256>(hist2, need2, red, res);
      thr = (p24 << 8) | D2.d;
      need_eq = need2 - D2.above;
    }
  }
  // The selection: keys above T, then the need_eq lowest positions at T.
  uint32_t cg = 0, ce = 0;
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    cg += (uint32_t)__popcll(__ballot(kk[s] > thr));
    ce += (uint32_t)__popcll(__ballot(kk[s] == thr));
    if (s % 8 == 7) __builtin_amdgcn_sched_barrier(0);
  }
  uint32_t ng, ne;
  uint32_t run_g = wave_base(cg, wtot[0], ng);
  uint32_t run_e = wave_base(ce, wtot[1], ne);
  uint32_t thr2 = thr;   // (opaque, as above)
  asm volatile("" : "+v"(thr2));
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const uint64_t mg = __ballot(kk[s] > thr2);
    const uint64_t me = __ballot(kk[s] == thr2);
    const uint32_t eb = run_e + lane_rank(me);   // ties before this element
    const bool pick = kk[s] > thr2 || (kk[s] == thr2 && eb < need_eq);
    if (pick) {
      const uint32_t slot = run_g + lane_rank(mg) + (eb < need_eq ? eb : need_eq);
      if (slot < (uint32_t)k) {
        oi[slot] = id_of(s);
        if (os) os[slot] = key_score(kk[s]);
      }
    }
    run_g += (uint32_t)__popcll(mg);
    run_e += (uint32_t)__popcll(me);
    if (s % 4 == 3) __builtin_amdgcn_sched_barrier(0);
  }
}

// ---------------------------------------------------------------- host ---

hipError_t select_local(const uint32_t* keys, int64_t key_stride, const int32_t* n_valid, int64_t rows, int k,
                        int64_t n_max, const uint32_t* tile_hist, int64_t th_stride, int64_t tiles,
                        const SelectOut& out, hipStream_t s) {
  if (out.expand != 0 || n_max > kLocalSel || (out.map && n_max > kLocalSelMap)) return hipErrorInvalidValue;
  if (tile_hist && (tiles < 1 || tiles > th_stride)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)rows), block(kLocalThreads);
  const int nt = (int)tiles;
#define CSA2_LOCAL(NS, MAP, TH)                                                                                    \
  CSA2_LAUNCH("select_local", (select_local_kernel<NS, MAP, TH>), grid, block, 0, s, keys, key_stride, n_valid, k, \
              tile_hist, th_stride, nt, out)
  const bool th = tile_hist != nullptr;
  if (n_max <= 16 * kLocalThreads) {
    if (out.map) {
      if (th) CSA2_LOCAL(16, true, true); else CSA2_LOCAL(16, true, false);
    } else {
      if (th) CSA2_LOCAL(16, false, true); else CSA2_LOCAL(16, false, false);
    }
  } else if (n_max <= 32 * kLocalThreads) {
    if (out.map) {
      if (th) CSA2_LOCAL(32, true, true); else CSA2_LOCAL(32, true, false);
    } else {
      if (th) CSA2_LOCAL(32, false, true); else CSA2_LOCAL(32, false, false);
    }
  } else {
    if (th) CSA2_LOCAL(64, false, true); else CSA2_LOCAL(64, false, false);
  }
#undef CSA2_LOCAL
  return hipGetLastError();
}

hipError_t select_clear(const SelectWs& ws, int64_t rows, hipStream_t s, const SelectWs* ws2) {
  // ctl and hist1 are carved contiguously.
  auto words = [&](const SelectWs& w) { return (int64_t)((char*)(w.hist1 + 4096 * rows) - (char*)w.ctl) / 4; };
  const int64_t n0 = words(ws), n1 = ws2 ? words(*ws2) : 0;
  int64_t grid = (n0 + n1 + 1023) / 1024;
  if (grid > 2048) grid = 2048;
  CSA2_LAUNCH("select_clear", select_clear_kernel, dim3((unsigned)grid), dim3(256), 0, s, (uint32_t*)ws.ctl, n0,
              ws2 ? (uint32_t*)ws2->ctl : (uint32_t*)nullptr, n1);
  return hipGetLastError();
}

hipError_t select_finish(const SelectWs& ws, const uint32_t* keys, int64_t key_stride, const int32_t* n_valid,
                         int64_t rows, int k, const SelectOut& out, hipStream_t s) {
  dim3 grid((unsigned)ws.tiles, (unsigned)rows);
  if (ws.tiles * rows >= kLevel1Pass) {
    CSA2_LAUNCH("select_level1", select_level1_kernel, dim3((unsigned)rows), dim3(256), 0, s, ws, k);
    CSA2_LAUNCH("select_collect", select_collect_kernel<true>, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid,
                k);
  } else {
    CSA2_LAUNCH("select_collect", select_collect_kernel<false>, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid,
                k);
  }
  CSA2_LAUNCH("select_finalize", select_finalize_kernel, dim3((unsigned)rows), dim3(256), 0, s, ws, keys, key_stride,
              n_valid, k, out);
  CSA2_LAUNCH("select_emit", select_emit_kernel, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid, k, out);
  return hipGetLastError();
}


// ----------------------------------------------- prefill chunk selection ---
// The states and buffers of a block of query rows (see PfRow): per row its
// state, a 4096-word histogram (or key-tile tie counts), kPfCap candidates.
static inline size_t pf_al256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t pf_ws_bytes(int64_t block_rows) {
  return pf_al256(sizeof(PfRow) * block_rows) + pf_al256(sizeof(uint32_t) * 4096 * block_rows) +
         pf_al256(sizeof(uint64_t) * kPfCap * block_rows) + pf_al256(sizeof(uint32_t) * kPfPasses);
}

PfArgs pf_ws_carve(void* base, int64_t block_rows) {
  char* p = (char*)base;
  PfArgs a{};
  a.rows = (PfRow*)p;
  p += pf_al256(sizeof(PfRow) * block_rows);
  a.hist = (uint32_t*)p;
  p += pf_al256(sizeof(uint32_t) * 4096 * block_rows);
  a.cand = (uint64_t*)p;
  p += pf_al256(sizeof(uint64_t) * kPfCap * block_rows);
  a.active = (uint32_t*)p;
  return a;
}

__global__ void __launch_bounds__(256) pf_clear_kernel(PfArgs pf) {
  const int64_t lr = blockIdx.x;
  if (threadIdx.x == 0) {
    PfRow r{};
    r.mode = PF_HIST;
    r.e_ps = 32u;
    r.n_ps = 32u;
    r.need = (uint32_t)pf.k_top;
    r.sampled = 1u;
    r.h_base = 0u;
    r.h_shift = 20u;   // (the top 12 bits)
    pf.rows[lr] = r;
    if (lr == 0)
      for (int i = 0; i < kPfPasses; ++i) pf.active[i] = 0u;
  }
  v4u* h = reinterpret_cast<v4u*>(pf.hist + lr * 4096);
  for (int i = threadIdx.x; i < 1024; i += 256) h[i] = v4u{0u, 0u, 0u, 0u};
}

// Bitonic sort of P (a power of two) 64-bit values in LDS by NT threads.
template <int NT>
__device__ void pf_bitonic(uint64_t* a, int P, bool descending) {
  for (int k = 2; k <= P; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < P; i += NT) {
        const int l = i ^ j;
        if (l > i) {
          const uint64_t x = a[i], y = a[l];
          const bool up = ((i & k) == 0) != descending;
          if ((x > y) == up) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
}

// Ascending bitonic sort of 2048 u64 values held 8 per thread (thread t:
// elements 8t .. 8t+7) by 256 threads.  Each thread keeps its own elements
// and takes the min or the max of every compare-exchange itself: partners
// inside the thread in registers, partners in another lane of the wave
// (distances 8 .. 256) by lane shuffles, partners in another wave
// (distances 512 and 1024) through LDS (`lds`: 2048 words of 64 bits).
__device__ __forceinline__ uint64_t pf_shfl_xor64(uint64_t x, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)x, m, 64);
  const uint32_t hi = (uint32_t)__shfl_xor((int)(uint32_t)(x >> 32), m, 64);
  return ((uint64_t)hi << 32) | lo;
}
template <int J>
__device__ __forceinline__ void pf_sort_inthread(uint64_t (&v)[8], int k, int t) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    if (e & J) continue;
    const uint64_t a = v[e], b = v[e | J];
    const bool up = ((8 * t + e) & k) == 0;
    const uint64_t lo = a < b ? a : b, hi = a < b ? b : a;
    v[e] = up ? lo : hi;
    v[e | J] = up ? hi : lo;
  }
}
__device__ void pf_sort2048(uint64_t (&v)[8], uint64_t* lds) {
  const int t = threadIdx.x;
  for (int k = 2; k <= 2048; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      if (j >= 512) {
#pragma unroll
        for (int e = 0; e < 8; ++e) lds[8 * t + e] = v[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * t + e;
          const uint64_t o = lds[i ^ j];
          const bool keep_min = (((i & k) == 0) == ((i & j) == 0));
          v[e] = keep_min ? (v[e] < o ? v[e] : o) : (v[e] < o ? o : v[e]);
        }
        __syncthreads();
      } else if (j >= 8) {
        const int m = j >> 3;
        const bool lower = (t & m) == 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint64_t o = pf_shfl_xor64(v[e], m);
          const bool keep_min = ((((8 * t + e) & k) == 0) == lower);
          v[e] = keep_min ? (v[e] < o ? v[e] : o) : (v[e] < o ? o : v[e]);
        }
      } else if (j == 4) {
        pf_sort_inthread<4>(v, k, t);
      } else if (j == 2) {
        pf_sort_inthread<2>(v, k, t);
      } else {
        pf_sort_inthread<1>(v, k, t);
      }
    }
  }
}

// After a pass, per row: resolve the digit of a histogram pass, pick the
// next mode; select the candidates of a candidate pass; prefix the tie
// counts of a tie-count pass.
__device__ __forceinline__ void pf_step_row(const PfArgs& pf, int pass) {
  __shared__ uint32_t red[4];
  __shared__ uint32_t res[4];
  // (32 KB: four workgroups per compute unit; with 16 KB and eight the
  // candidate step measured 1.6 times slower)
  __shared__ __align__(16) uint64_t sbuf[kPfCap];
  const int64_t lr = blockIdx.x;
  PfRow* st = pf.rows + lr;
  const uint32_t mode = st->mode;
  if (mode == PF_DONE) return;
  uint32_t* h = pf.hist + lr * 4096;
  const int64_t grow = pf.row_base + lr;
  const uint32_t K = (uint32_t)pf.k_top;
  // The exact search from its start (every count cleared; the histogram
  // zeroed by the caller).
  auto restart = [&]() {
    if (threadIdx.x == 0) {
      st->e_on = 0u; st->e_ps = 32u; st->e_pfx = 0u; st->e_incl = 0u;
      st->n_ps = 32u; st->n_pfx = 0u; st->need = K; st->bcnt = 0u;
      st->out_cnt = 0u; st->cand_cnt = 0u; st->sampled = 0u;
      st->mode = PF_HIST;
    }
  };
  auto zero_hist = [&]() {
    v4u* h4 = reinterpret_cast<v4u*>(h);
    for (int i = threadIdx.x; i < 1024; i += 256) h4[i] = v4u{0u, 0u, 0u, 0u};
  };
  if (pass == 1 && st->sampled == 0u) {
    // Pass 1 histograms the sample again: rows already outside it (taking
    // every key, or searching exactly) wait for the next pass.
    if (mode == PF_HIST) zero_hist();
    return;
  }
  if (mode == PF_HIST) {
    uint32_t need = st->need;
    const uint32_t n_ps = st->n_ps, n_pfx = st->n_pfx;
    if (n_ps >= 32u) {
      // level 1: every visible key was counted, or (sampled) one chunk in
      // kPfSample.  (The row's fields are read before the first barrier:
      // thread 0 rewrites them at the end.)
      const uint32_t stage = st->sampled, prev_total = st->s_total;
      const uint64_t hb = st->h_base, hs = st->h_shift;
      uint32_t sum = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) sum += h[threadIdx.x * 16 + i];
      const uint32_t incl = block_suffix_sum_256(sum, red);
      if (threadIdx.x == 0) res[3] = incl;
      __syncthreads();
      const bool sampled = stage != 0u;
      const uint32_t total = sampled ? (uint32_t)pf.n_valid[grow] : res[3];
      const uint32_t total_s = res[3];
      __syncthreads();
      if (sampled && total > K) {
        const uint32_t s_total = stage == 1u ? total_s : prev_total;
        if (s_total == 0u) {   // (no sampled key visible: search exactly)
          restart();
          zero_hist();
          return;
        }
        // With ks the sample's share of k_top and m four standard deviations
        // of the sample count (plus four), the window runs from the bin
        // where ks - m sampled keys are reached from the top (exclusive: the
        // keys above it are emitted) down to the bin where ks + m are.
        const float ks = (float)K * (float)s_total / (float)total;
        const float m = 4.0f * __builtin_sqrtf(ks) + 4.0f;
        const uint32_t need_e = ks - m >= 1.0f ? (uint32_t)(ks - m) + 1u : 1u;
        const float fl = __builtin_ceilf(ks + m);
        const uint32_t need_l = fl > (float)total_s ? total_s + 1u : (uint32_t)fl;
        // (total_s: the sampled keys inside this histogram's range)
        Digit de{4095u, 0u, 0u}, dl{0u, 0u, 0u};
        if (need_e <= total_s) de = resolve_digit<4096>(h, need_e, red, res);
        const bool has_lo = need_l <= total_s;
        if (has_lo) dl = resolve_digit<4096>(h, need_l, red, res);
        // key bounds of bins: bin d covers [hb + (d << hs), hb + ((d + 1) << hs))
        const uint64_t e_key = hb + ((uint64_t)(de.d + 1u) << hs);
        const uint64_t c_key = has_lo ? hb + ((uint64_t)dl.d << hs) : (stage == 1u ? 0ull : hb);
        if (stage == 1u) {
          // Coarse: histogram the window [c_key, e_key) again at a finer
          // grain: at most 4095 bins of 2^sh keys cover it, and the last of
          // the 4096 bins takes the keys above.
          const uint64_t span = e_key - c_key;
          uint32_t sh = 8u;
          while (sh < 20u && ((uint64_t)4095 << sh) < span) ++sh;
          __syncthreads();   // (every thread has read h)
          zero_hist();
          if (threadIdx.x == 0) {
            st->h_base = (uint32_t)c_key;
            st->h_shift = sh;
            st->s_total = s_total;
            st->sampled = 2u;
          }
          return;
        }
        // Fine: the guess, unless the window is unusable: its emission
        // bound in the last bin (which holds every key above the range), no
        // lower bound, or more candidates expected than kept (heavy ties):
        // then the row searches exactly from the next pass on.
        const float in_win = (float)(dl.above + dl.cnt - de.above) * (float)total / (float)s_total;
        if (de.d >= 4095u || !has_lo || in_win > 0.75f * (float)kPfCap) {
          restart();
          zero_hist();
          return;
        }
        if (threadIdx.x == 0) {
          st->g_emit_none = 0u;
          st->g_emit = (uint32_t)e_key;
          st->g_cand = (uint32_t)c_key;
          st->out_cnt = 0u; st->cand_cnt = 0u; st->sampled = 0u;
          st->mode = PF_GUESS;
        }
        return;
      }
      if (total <= K) {   // every visible key is selected: the first `total` positions
        if (!pf.out_key) {
          for (uint32_t i = threadIdx.x; i < total; i += 256) pf.out_idx[grow * K + i] = (int32_t)i;
          if (threadIdx.x == 0) {
            st->out_cnt = total;
            st->mode = PF_DONE;
          }
          return;
        }
        if (threadIdx.x == 0) {   // (their scores come from the next pass)
          st->e_on = 1u; st->e_ps = 32u; st->e_pfx = 0u; st->e_incl = 1u;
          st->n_ps = 0u; st->n_pfx = 0u; st->need = 0u; st->bcnt = 0u; st->sampled = 0u;
          st->mode = PF_EMIT;
        }
        return;
      }
      need = K;
    }
    const Digit d = resolve_digit<4096>(h, need, red, res);
    const uint32_t w = n_ps == 8u ? 8u : 12u;
    const uint32_t new_ps = (n_ps >= 32u ? 32u : n_ps) - w;
    const uint32_t new_pfx = (n_ps >= 32u ? 0u : (n_pfx << w)) | d.d;
    const uint32_t need2 = need - d.above;
    uint32_t nm;
    if (need2 == d.cnt) nm = PF_EMIT;                 // the whole bucket is taken
    else if (d.cnt <= (uint32_t)kPfCap) nm = PF_CAND;
    else nm = new_ps > 0u ? PF_HIST : PF_TIECOUNT;
    if (threadIdx.x == 0) {
      st->e_on = 1u; st->e_ps = n_ps; st->e_pfx = n_pfx; st->e_incl = nm == PF_EMIT ? 1u : 0u;
      st->n_ps = new_ps; st->n_pfx = new_pfx; st->need = need2; st->bcnt = d.cnt; st->cand_cnt = 0u;
      st->mode = nm;
    }
    if (nm == PF_HIST || nm == PF_TIECOUNT) zero_hist();   // (resolve_digit has read h and synchronised)
  } else if (mode == PF_CAND || mode == PF_GUESS) {
    // The bucket's keys as (key << 32 | ~position): descending order is
    // (score desc, position asc); the first `need` are taken.
    uint32_t n = st->cand_cnt;
    const uint32_t base = st->out_cnt;
    uint32_t need = st->need;
    if (mode == PF_GUESS) {
      // The guess holds when the keys above the window are at most k_top,
      // with the window's keys at least k_top, and every candidate was kept.
      if (base > K || base + n < K || n > (uint32_t)kPfCap) {
        restart();
        zero_hist();
        return;
      }
      need = K - base;
    }
    if (n > (uint32_t)kPfCap) n = kPfCap;
    if (need > n) need = n;
    auto take = [&](uint32_t i, uint64_t v) {   // i-th largest candidate
      const uint32_t slot = base + i;
      if (i < need && slot < K) {
        pf.out_idx[grow * K + slot] = (int32_t)(0xFFFFFFFFu - (uint32_t)v);
        if (pf.out_key) pf.out_key[grow * K + slot] = (uint32_t)(v >> 32);
      }
    };
    if (n <= 2048u) {
      // complements sorted ascending: the largest candidates first (padding
      // ~0 last); loaded in any order (coalesced), sorted into thread order
      uint64_t v[8];
      const uint64_t* cp = pf.cand + lr * kPfCap + threadIdx.x;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = threadIdx.x + 256u * e < n ? ~cp[256 * e] : ~0ull;
      pf_sort2048(v, sbuf);
#pragma unroll
      for (int e = 0; e < 8; ++e) take(8u * threadIdx.x + e, ~v[e]);
    } else {
      int P = 1;
      while (P < (int)n) P <<= 1;
      for (int i = threadIdx.x; i < P; i += 256) sbuf[i] = i < (int)n ? pf.cand[lr * kPfCap + i] : 0ull;
      __syncthreads();
      pf_bitonic<256>(sbuf, P, true);
      for (uint32_t i = threadIdx.x; i < need; i += 256) take(i, sbuf[i]);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      st->out_cnt = base + need;
      st->mode = PF_DONE;
    }
  } else if (mode == PF_TIECOUNT) {
    // exclusive prefix of the ties per key tile, in place
    uint32_t v[16];
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] = h[threadIdx.x * 16 + i];
      sum += v[i];
    }
    uint32_t run = block_prefix_sum_256(sum, red) - sum;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      h[threadIdx.x * 16 + i] = run;
      run += v[i];
    }
    if (threadIdx.x == 0) {
      st->e_on = 0u;
      st->mode = PF_TIEEMIT;
    }
  } else {   // PF_EMIT, PF_TIEEMIT: the pass has emitted the rest
    if (threadIdx.x == 0) st->mode = PF_DONE;
  }
}

// A step flags whether it leaves a row undone (plain stores of 1: same-address
// atomics from every workgroup cost more): the next pass and step return at
// once when none is.
__global__ void __launch_bounds__(256) pf_step_kernel(PfArgs pf, int pass) {
  if (pass > 0 && pf.active[pass - 1] == 0u) return;   // (uniform)
  pf_step_row(pf, pass);
  if (threadIdx.x == 0 && pf.rows[blockIdx.x].mode != PF_DONE) pf.active[pass] = 1u;
}

// Rows of up to 32 * kRankWords positions with k_top <= 2048 take their
// slots by rank in a position bitmap: every position sets its bit, a block
// scan gives each 32-bit word the number of set bits before it, and a
// position's slot is that count plus the set bits below it in its word
// (positions are unique and below the row's visible count).  Thread t owns
// words t*kRankWpt .. +kRankWpt-1 (odd: a wave's threads hit distinct banks).
constexpr int kRankWpt = 41;
constexpr int kRankWords = 256 * kRankWpt;   // 10,496 words: 335,872 positions

__device__ void pf_final_rank(const PfArgs& pf, int64_t lr, int64_t grow, uint32_t n, int nw, uint32_t* bits,
                              uint16_t* pre, uint32_t* wtot, float* __restrict__ topk_score) {
  constexpr int NT = 256, EPT = 2048 / NT;
  const int K = pf.k_top;
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int w0 = t * kRankWpt;
  const bool own = w0 < nw;   // (words past nw in an owned range are zeroed too)
  if (own) {
#pragma unroll
    for (int i = 0; i < kRankWpt; ++i) bits[w0 + i] = 0u;
  }
  const int32_t* oi = pf.out_idx + grow * K;
  const uint32_t* ok = pf.out_key ? pf.out_key + grow * K : nullptr;
  uint32_t pos[EPT], key[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) {   // (all read before any slot is written below)
    const uint32_t i = (uint32_t)t + NT * e;
    pos[e] = i < n ? (uint32_t)oi[i] : ~0u;
    key[e] = i < n && ok ? ok[i] : 0u;
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < EPT; ++e)
    if (pos[e] != ~0u) atomicOr(&bits[pos[e] >> 5], 1u << (pos[e] & 31u));
  __syncthreads();
  uint32_t tot = 0;
  if (own) {
#pragma unroll
    for (int i = 0; i < kRankWpt; ++i) tot += (uint32_t)__builtin_popcount(bits[w0 + i]);
  }
  const uint32_t incl = wave_prefix_sum(tot);
  if (lane == 63) wtot[wv] = incl;
  __syncthreads();
  uint32_t run = incl - tot;
  for (int j = 0; j < wv; ++j) run += wtot[j];
  if (own) {
#pragma unroll
    for (int i = 0; i < kRankWpt; ++i) {
      const uint32_t b = bits[w0 + i];
      pre[w0 + i] = (uint16_t)run;
      run += (uint32_t)__builtin_popcount(b);
    }
  }
  __syncthreads();
#pragma unroll
  for (int e = 0; e < EPT; ++e) {
    if (pos[e] == ~0u) continue;
    const uint32_t w = pos[e] >> 5;
    const uint32_t r = pre[w] + (uint32_t)__builtin_popcount(bits[w] & ((1u << (pos[e] & 31u)) - 1u));
    pf.out_idx[grow * K + r] = (int32_t)pos[e];
    if (topk_score) topk_score[grow * K + r] = key_score(key[e]);
  }
  for (int i = (int)n + t; i < K; i += NT) {
    pf.out_idx[grow * K + i] = -1;
    if (topk_score) topk_score[grow * K + i] = -__builtin_inff();
  }
}

// Each row's positions ascending (ids unique), scores from their keys, -1 /
// -inf padding.  PMAX >= k_top.
template <int PMAX, int NT>
__global__ void __launch_bounds__(NT) pf_final_kernel(PfArgs pf, float* __restrict__ topk_score) {
  constexpr bool RANK = PMAX == 2048 && NT == 256;
  // (the rank path's bitmap and counts, or the sort's values)
  __shared__ __align__(16) uint32_t lds[RANK ? kRankWords + kRankWords / 2 + 4 : 2 * PMAX];
  uint64_t* sbuf = reinterpret_cast<uint64_t*>(lds);
  const int64_t lr = blockIdx.x;
  const int64_t grow = pf.row_base + lr;
  const int K = pf.k_top;
  uint32_t n = pf.rows[lr].out_cnt;
  if (n > (uint32_t)K) n = K;
  if constexpr (RANK) {
    int64_t nv = pf.n_valid[grow];
    nv = nv < 0 ? 0 : nv;
    if (nv <= 32LL * kRankWords) {   // (uniform)
      pf_final_rank(pf, lr, grow, n, (int)((nv + 31) >> 5), lds, reinterpret_cast<uint16_t*>(lds + kRankWords),
                    lds + kRankWords + kRankWords / 2, topk_score);
      return;
    }
    // (position << 32 | key) sorted in registers; padding ~0 last
    const int32_t* oi = pf.out_idx + grow * K;
    const uint32_t* ok = pf.out_key ? pf.out_key + grow * K : nullptr;
    uint64_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {   // (any order in: coalesced loads)
      const uint32_t i = threadIdx.x + 256u * e;
      v[e] = i < n ? ((uint64_t)(uint32_t)oi[i] << 32) | (ok ? ok[i] : 0u) : ~0ull;
    }
    pf_sort2048(v, sbuf);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int i = 8 * (int)threadIdx.x + e;
      if (i >= K) continue;
      const bool val = i < (int)n;
      pf.out_idx[grow * K + i] = val ? (int32_t)(v[e] >> 32) : -1;
      if (topk_score) topk_score[grow * K + i] = val ? key_score((uint32_t)v[e]) : -__builtin_inff();
    }
    return;
  }
  int P = 1;
  while (P < (int)n) P <<= 1;
  const int32_t* oi = pf.out_idx + grow * K;
  const uint32_t* ok = pf.out_key ? pf.out_key + grow * K : nullptr;
  for (int i = threadIdx.x; i < P; i += NT)
    sbuf[i] = i < (int)n ? ((uint64_t)(uint32_t)oi[i] << 32) | (ok ? ok[i] : 0u) : ~0ull;
  __syncthreads();
  pf_bitonic<NT>(sbuf, P, false);
  for (int i = threadIdx.x; i < K; i += NT) {
    const bool v = i < (int)n;
    pf.out_idx[grow * K + i] = v ? (int32_t)(sbuf[i] >> 32) : -1;
    if (topk_score) topk_score[grow * K + i] = v ? key_score((uint32_t)sbuf[i]) : -__builtin_inff();
  }
}

hipError_t pf_clear(const PfArgs& pf, int64_t block_rows, hipStream_t s) {
  CSA2_LAUNCH("pf_clear", pf_clear_kernel, dim3((unsigned)block_rows), dim3(256), 0, s, pf);
  return hipGetLastError();
}

hipError_t pf_step(const PfArgs& pf, int64_t block_rows, int pass, hipStream_t s) {
  CSA2_LAUNCH("pf_step", pf_step_kernel, dim3((unsigned)block_rows), dim3(256), 0, s, pf, pass);
  return hipGetLastError();
}

hipError_t pf_final(const PfArgs& pf, int64_t block_rows, float* topk_score, hipStream_t s) {
  if (pf.k_top <= 2048)
    CSA2_LAUNCH("pf_final", (pf_final_kernel<2048, 256>), dim3((unsigned)block_rows), dim3(256), 0, s, pf, topk_score);
  else
    CSA2_LAUNCH("pf_final", (pf_final_kernel<kPfMaxK, 512>), dim3((unsigned)block_rows), dim3(512), 0, s, pf,
                topk_score);
  return hipGetLastError();
}

}  // namespace csa2
