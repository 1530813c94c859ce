// Exact per-row Top-K by radix select over order-preserving u32 keys.
//
// Selection rule (the indexer keeps its top-k tokens -- techniques map,
// "Checked in its code", indexer-selected sparse attention; the tie rule and
// output order are this library's): order positions by (key desc, position
// asc), keep the first k, emit them in ascending position order.
//
// With T the k-th largest key and need_eq the number of keys equal to T that
// belong to the selection, the selection is {key > T} plus the need_eq
// lowest positions with key == T.  T is found digit by digit (12 + 12 + 8
// bits) from histograms; each pass is a grid of workgroups over fixed tiles
// of a row, and the last workgroup of a row to finish (counter election, no
// waiting) resolves the digit for that row.  A final count pass gives every
// tile its output offset, and the emit pass writes indices in order.  Rows
// whose visible count is <= k, or whose threshold bucket is taken whole,
// skip the remaining digit passes.
#include "common.h"
#include "internal.h"
#include "select_dev.h"

namespace csa2 {

static __host__ __device__ inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

size_t select_ws_bytes(int64_t rows, int64_t tiles) {
  size_t b = 0;
  b += align256(sizeof(SelectRowCtl) * rows);
  b += align256(sizeof(uint32_t) * 4096 * rows);
  b += align256(sizeof(uint32_t) * 4096 * rows);
  b += align256(sizeof(uint32_t) * 256 * rows);
  b += align256(sizeof(uint32_t) * tiles * rows);
  b += align256(sizeof(uint32_t) * tiles * rows);
  return b;
}

SelectWs select_ws_carve(void* base, int64_t rows, int64_t tiles) {
  char* p = (char*)base;
  SelectWs w;
  w.ctl = (SelectRowCtl*)p; p += align256(sizeof(SelectRowCtl) * rows);
  w.hist1 = (uint32_t*)p; p += align256(sizeof(uint32_t) * 4096 * rows);
  w.hist2 = (uint32_t*)p; p += align256(sizeof(uint32_t) * 4096 * rows);
  w.hist3 = (uint32_t*)p; p += align256(sizeof(uint32_t) * 256 * rows);
  w.tile_gt = (uint32_t*)p; p += align256(sizeof(uint32_t) * tiles * rows);
  w.tile_eq = (uint32_t*)p;
  return w;
}

// The 16 keys a thread handles in the unordered passes: positions
// base + 4*(tid + 256*i) + (0..3), i = 0..3, loaded as four 16-byte vectors
// (coalesced across the workgroup) before any of them is used.  Positions at
// or past nv read as 0 (absent).  Rows are padded to a multiple of 64 keys, so
// a vector that starts below nv stays inside the row.
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

// ------------------------------------------------------------- kernels ---

__global__ void select_clear_kernel(uint32_t* p, int64_t n_words) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
       i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// Pass 1 over stored keys: histogram of the top 12 bits.
__global__ void __launch_bounds__(256)
select_hist1_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                    const int32_t* __restrict__ n_valid, int k) {
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t flag;
  const int64_t row = blockIdx.y;
  const int64_t base = (int64_t)blockIdx.x * kSelTile;
  const int64_t nv = n_valid[row];
  for (int i = threadIdx.x; i < 4096; i += 256) hist[i] = 0u;
  __syncthreads();
  uint32_t kk[16];
  load_tile_keys(keys + row * key_stride, base, nv, kk);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (kk[i]) atomicAdd(&hist[kk[i] >> 20], 1u);
  __syncthreads();
  uint32_t* gh = ws.hist1 + row * 4096;
  for (int i = threadIdx.x; i < 4096; i += 256)
    if (hist[i]) atomic_add_agent(gh + i, hist[i]);
  if (arrive_last(&ws.ctl[row].arrive[0], gridDim.x, &flag)) select_resolve1(&ws.ctl[row], gh, (uint32_t)k);
}

// Pass 2 (DIGIT = 2) and pass 3 (DIGIT = 3): refine the threshold.
template <int DIGIT>
__global__ void __launch_bounds__(256)
select_refine_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                     const int32_t* __restrict__ n_valid) {
  constexpr int BINS = DIGIT == 2 ? 4096 : 256;
  constexpr int SHIFT = DIGIT == 2 ? 20 : 8;         // prefix = key >> SHIFT
  constexpr int DSHIFT = DIGIT == 2 ? 8 : 0;         // digit = (key >> DSHIFT) & (BINS-1)
  __shared__ uint32_t hist[BINS];
  __shared__ uint32_t flag;
  __shared__ uint32_t red[4];
  __shared__ uint32_t res[3];
  const int64_t row = blockIdx.y;
  SelectRowCtl* ctl = &ws.ctl[row];
  const uint32_t mode = ctl->mode;
  uint32_t* gh = (DIGIT == 2 ? ws.hist2 + row * 4096 : ws.hist3 + row * 256);
  if (mode == 0u) {
    const uint32_t prefix = ctl->prefix;
    const int64_t base = (int64_t)blockIdx.x * kSelTile;
    const int64_t nv = n_valid[row];
    for (int i = threadIdx.x; i < BINS; i += 256) hist[i] = 0u;
    __syncthreads();
    uint32_t kk[16];
    load_tile_keys(keys + row * key_stride, base, nv, kk);
#pragma unroll
    for (int i = 0; i < 16; ++i)
      if (kk[i] && (kk[i] >> SHIFT) == prefix) atomicAdd(&hist[(kk[i] >> DSHIFT) & (BINS - 1)], 1u);
    __syncthreads();
    for (int i = threadIdx.x; i < BINS; i += 256)
      if (hist[i]) atomic_add_agent(gh + i, hist[i]);
  }
  if (!arrive_last(&ctl->arrive[DIGIT - 1], gridDim.x, &flag)) return;
  if (mode != 0u) return;
  const uint32_t need = ctl->need;
  resolve_digit<BINS>(gh, need, red, res);
  if (threadIdx.x == 0) {
    uint32_t d = res[0], above = res[1], cnt = res[2];
    uint32_t prefix = (ctl->prefix << (DIGIT == 2 ? 12 : 8)) | d;
    uint32_t n2 = need - above;
    if (DIGIT == 3) {
      ctl->thr = prefix;
      ctl->need_eq = n2;
      ctl->mode = 2u;
    } else if (n2 == cnt) {
      ctl->thr = (prefix << 8) - 1u;
      ctl->need_eq = 0u;
      ctl->mode = 2u;
    } else {
      ctl->prefix = prefix;
      ctl->need = n2;
    }
  }
}

// Pass 4: per-tile counts of keys above and at the threshold; the last
// workgroup turns them into output offsets and writes the -1 padding.
__global__ void __launch_bounds__(256)
select_count_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                    const int32_t* __restrict__ n_valid, int k, SelectOut out) {
  __shared__ uint32_t flag;
  __shared__ uint32_t red[4];
  __shared__ uint32_t carry[2];
  const int64_t row = blockIdx.y;
  const int64_t tiles = gridDim.x;
  SelectRowCtl* ctl = &ws.ctl[row];
  const uint32_t thr = ctl->thr;
  const int64_t base = (int64_t)blockIdx.x * kSelTile;
  const int64_t nv = n_valid[row];
  uint32_t kk[16];
  load_tile_keys(keys + row * key_stride, base, nv, kk);
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    gt += kk[i] != 0u && kk[i] > thr;
    eq += kk[i] != 0u && kk[i] == thr;
  }
  // workgroup sums
  for (int off = 32; off > 0; off >>= 1) {
    gt += __shfl_xor(gt, off, 64);
    eq += __shfl_xor(eq, off, 64);
  }
  __shared__ uint32_t sgt[4], seq[4];
  if ((threadIdx.x & 63) == 0) { sgt[threadIdx.x >> 6] = gt; seq[threadIdx.x >> 6] = eq; }
  __syncthreads();
  if (threadIdx.x == 0) {
    store_agent(ws.tile_gt + row * tiles + blockIdx.x, sgt[0] + sgt[1] + sgt[2] + sgt[3]);
    store_agent(ws.tile_eq + row * tiles + blockIdx.x, seq[0] + seq[1] + seq[2] + seq[3]);
  }
  if (!arrive_last(&ctl->arrive[3], (uint32_t)tiles, &flag)) return;
  // Exclusive scan over tiles, 256 at a time with a running carry.
  const uint32_t need_eq = ctl->need_eq;
  if (threadIdx.x == 0) { carry[0] = 0u; carry[1] = 0u; }
  __syncthreads();
  for (int64_t t0 = 0; t0 < tiles; t0 += 256) {
    int64_t t = t0 + threadIdx.x;
    uint32_t g = 0, e = 0;
    if (t < tiles) {
      g = load_agent(ws.tile_gt + row * tiles + t);
      e = load_agent(ws.tile_eq + row * tiles + t);
    }
    uint32_t c_out = carry[0], c_eq = carry[1];
    uint32_t e_incl = block_prefix_sum_256(e, red);
    uint32_t eq_before = c_eq + e_incl - e;
    uint32_t take = 0;
    if (need_eq > eq_before) take = (need_eq - eq_before) < e ? (need_eq - eq_before) : e;
    uint32_t sel = g + take;
    uint32_t s_incl = block_prefix_sum_256(sel, red);
    if (t < tiles) {
      ws.tile_gt[row * tiles + t] = c_out + s_incl - sel;   // output offset of this tile
      ws.tile_eq[row * tiles + t] = eq_before;              // ties before this tile
    }
    __syncthreads();
    if (threadIdx.x == 255) { carry[0] = c_out + s_incl; carry[1] = c_eq + e_incl; }
    __syncthreads();
  }
  const uint32_t total = carry[0];
  if (threadIdx.x == 0) ctl->total = total;
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
    if (threadIdx.x == 0) out.pool_len[row] = (int32_t)(total * out.expand);
  }
}

// Pass 5: emit the selected positions of each tile in ascending order.
__global__ void __launch_bounds__(256)
select_emit_kernel(SelectWs ws, const uint32_t* __restrict__ keys, int64_t key_stride,
                   const int32_t* __restrict__ n_valid, int k, SelectOut out) {
  constexpr int PER = kSelTile / 256;  // consecutive positions per thread
  __shared__ uint32_t red[4];
  const int64_t row = blockIdx.y;
  const int64_t tiles = gridDim.x;
  const SelectRowCtl* ctl = &ws.ctl[row];
  const uint32_t thr = ctl->thr, need_eq = ctl->need_eq;
  const uint32_t off0 = ws.tile_gt[row * tiles + blockIdx.x];
  const uint32_t eqb0 = ws.tile_eq[row * tiles + blockIdx.x];
  const int64_t nv = n_valid[row];
  const int64_t base = (int64_t)blockIdx.x * kSelTile;
  if (base >= nv) return;
  const int64_t p0 = base + (int64_t)threadIdx.x * PER;
  const uint32_t* kr = keys + row * key_stride;
  uint32_t kk[PER];
#pragma unroll
  for (int i = 0; i < PER / 4; ++i) {
    v4u v = {0u, 0u, 0u, 0u};
    if (p0 + 4 * i < nv) v = *reinterpret_cast<const v4u*>(kr + p0 + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) kk[4 * i + j] = (p0 + 4 * i + j < nv) ? v[j] : 0u;
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
      int32_t invalid = 0;
      for (int u = 0; u < out.expand; ++u) {
        int64_t id = pos * out.expand + u;
        bool ok = id < lim;
        out.idx[row * cap + (int64_t)slot * out.expand + u] = ok ? (int32_t)id : -1;
        invalid += !ok;
      }
      if (invalid) atomicSub(&out.pool_len[row], invalid);
    }
    ++slot;
  }
}

// ---------------------------------------------------------------- host ---

hipError_t select_clear(const SelectWs& ws, int64_t rows, hipStream_t s) {
  // ctl, hist1, hist2 and hist3 are carved contiguously.
  int64_t words = (int64_t)((char*)(ws.hist3 + 256 * rows) - (char*)ws.ctl) / 4;
  int64_t grid = (words + 255) / 256;
  if (grid > 4096) grid = 4096;
  CSA2_LAUNCH("select_clear", select_clear_kernel, dim3((unsigned)grid), dim3(256), 0, s, (uint32_t*)ws.ctl,
              words);
  return hipGetLastError();
}

hipError_t select_hist1(const SelectWs& ws, const uint32_t* keys, int64_t key_stride, const int32_t* n_valid,
                        int64_t rows, int64_t n_max, int k, hipStream_t s) {
  int64_t tiles = (n_max + kSelTile - 1) / kSelTile;
  if (tiles < 1) tiles = 1;
  CSA2_LAUNCH("select_hist1", select_hist1_kernel, dim3((unsigned)tiles, (unsigned)rows), dim3(256), 0, s, ws,
              keys, key_stride, n_valid, k);
  return hipGetLastError();
}

hipError_t select_finish(const SelectWs& ws, const uint32_t* keys, int64_t key_stride, const int32_t* n_valid,
                         int64_t rows, int64_t n_max, int k, const SelectOut& out, hipStream_t s) {
  int64_t tiles = (n_max + kSelTile - 1) / kSelTile;
  if (tiles < 1) tiles = 1;
  dim3 grid((unsigned)tiles, (unsigned)rows);
  CSA2_LAUNCH("select_refine2", select_refine_kernel<2>, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid);
  CSA2_LAUNCH("select_refine3", select_refine_kernel<3>, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid);
  CSA2_LAUNCH("select_count", select_count_kernel, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid, k, out);
  CSA2_LAUNCH("select_emit", select_emit_kernel, grid, dim3(256), 0, s, ws, keys, key_stride, n_valid, k, out);
  return hipGetLastError();
}

}  // namespace csa2
