// Indexer scoring: the lightning-style indexer of the DeepSeek-V4.1-Flash
// techniques map ("Checked in its code", indexer-selected sparse attention):
// every indexer head h of the query scores each visible key row k_j, and the
// per-token score is  s_j = sum_h w_h * ReLU(q_h . k_j).  The key cache holds
// one row of index_head_dim per token (fact sheet, kv_groups: indexer K).
//
// gfx950 mapping.  The scan is an HBM stream of the key rows (D_I bytes per
// token).  The dots run on the FP8 matrix cores (v_mfma_f32_16x16x32_fp8_fp8):
// A = the query heads (16 rows, padded), B = 16 key rows, K = 32 bytes per
// instruction.  With integer-valued E4M3 inputs every product and partial sum
// is an integer below 2^24, so the fp32 accumulation is exact and the order
// inside the instruction does not matter.  Each lane loads one contiguous
// D_I/4-byte slice of a key row; the A operand uses the same slice of each
// query head, so the k-permutation is identical on both sides.  The 16x16
// results pass through LDS so that every lane owns one token, applies ReLU
// and the weights, and adds the heads in ascending order with float32
// roundings and no FMA.  The epilogue also builds the radix-select
// histogram of the top 12 key bits in LDS, writes the score keys, and (for
// the hierarchical pool) the per-block maxima and their histogram.
#include "common.h"
#include "internal.h"
#include "select_dev.h"

namespace csa2 {

#ifndef CSA2_SCAN_TILE
#define CSA2_SCAN_TILE 4096
#endif
constexpr int kScanTile = CSA2_SCAN_TILE;   // max tokens per workgroup of the flat scan
constexpr int kPoolTile = 512;        // pool positions per workgroup (later layers)
constexpr int kScanWaves = 4;
// 16-token MFMA groups per wave iteration (bytes in flight per wave =
// 2 * 16 * groups * D_I); fewer for 32 indexer heads to bound the LDS tile.
#ifndef CSA2_SCAN_GROUPS
#define CSA2_SCAN_GROUPS 4
#endif
template <int HB>
constexpr int kScanGroups = HB == 1 ? CSA2_SCAN_GROUPS : 4;

template <int CH>
struct Frag {
  uint32_t w[CH / 4];
};

// A lane's share of a DI-byte row: for DI >= 64, DI/64 chunks of 16 bytes,
// chunk j at byte 64*j + 16*g (so the four lane groups of one load
// instruction cover whole 64-byte segments of 16 rows); for DI = 32 one
// 8-byte piece at 8*g.  Piece i (8 bytes) of the fragment feeds MFMA k-step i;
// the query fragments use the same map, so products pair up.
template <int DI>
__device__ __forceinline__ const uint8_t* frag_base(const uint8_t* row, int g) {
  return row + (DI >= 64 ? 16 * g : 8 * g);
}

template <int CH, int DI>
__device__ __forceinline__ void load_frag(Frag<CH>& f, const uint8_t* p, bool ok) {
  if (!ok) {
#pragma unroll
    for (int i = 0; i < CH / 4; ++i) f.w[i] = 0u;
    return;
  }
  if constexpr (DI >= 64) {
#pragma unroll
    for (int j = 0; j < DI / 64; ++j) {
      v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(p + 64 * j));
      f.w[4 * j] = v[0]; f.w[4 * j + 1] = v[1]; f.w[4 * j + 2] = v[2]; f.w[4 * j + 3] = v[3];
    }
  } else {
    v2u v = __builtin_nontemporal_load(reinterpret_cast<const v2u*>(p));
    f.w[0] = v[0]; f.w[1] = v[1];
  }
}

__device__ __forceinline__ long as_long(uint32_t lo, uint32_t hi) {
  return (long)(((unsigned long)hi << 32) | lo);
}

// GATHER = false: tokens j = tile positions of the row (flat scan).
// GATHER = true : position p maps to token pool_idx[row][p] (pool layers).
template <int DI, int HB, bool GATHER, bool POOL>
__global__ void __launch_bounds__(256)
index_score_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                   const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                   const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                   const int32_t* __restrict__ pool_idx, const int32_t* __restrict__ pool_len, int pool_cap,
                   int Tq, int H_I, int64_t n_max, int k_top, int tile,
                   uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                   SelectWs tok,
                   int pool_block, int nblocks, uint32_t* __restrict__ bkeys, int64_t bkey_stride,
                   int32_t* __restrict__ nb_valid_out, SelectWs blk) {
  constexpr int CH = DI / 4;           // bytes of a key row per lane
  constexpr int KS = DI / 32;          // MFMA k-steps
  constexpr int HMAX = 16 * HB;
  __shared__ uint32_t hist[4096];
  __shared__ uint32_t bhist[POOL ? 4096 : 1];
  __shared__ __attribute__((aligned(16))) float dots[kScanWaves][16 * kScanGroups<HB> * HMAX];
  __shared__ float wsh[HMAX];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.y;
  const int64_t b = row / Tq;
  constexpr bool pool = POOL;

  int64_t nv;
  if (GATHER) {
    int64_t pl = pool_len[row];
    nv = pl < 0 ? 0 : (pl > pool_cap ? pool_cap : pl);
  } else {
    int64_t c = ctx_len[b];
    if (q_pos) {
      int64_t qp = (int64_t)q_pos[row] + 1;
      if (qp < c) c = qp;
    }
    nv = c < 0 ? 0 : (c > n_max ? n_max : c);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    n_valid_out[row] = (int32_t)nv;
    if (pool) nb_valid_out[row] = (int32_t)((nv + pool_block - 1) / pool_block);
  }

  for (int i = threadIdx.x; i < 4096; i += 256) {
    hist[i] = 0u;
    if (pool) bhist[i] = 0u;
  }
  if (threadIdx.x < HMAX) wsh[threadIdx.x] = threadIdx.x < H_I ? w[row * H_I + threadIdx.x] : 0.0f;
  __syncthreads();
  float wv[HMAX];   // head weights (0 past H_I), wave-uniform
#pragma unroll
  for (int h = 0; h < HMAX; ++h) wv[h] = wsh[h];

  // A operand: query head (lane & 15) + 16*hb, slice (lane >> 4) of the row.
  const int c16 = lane & 15, g = lane >> 4;
  long qa[HB][KS];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    int h = c16 + 16 * hb;
    Frag<CH> f;
    load_frag<CH, DI>(f, frag_base<DI>(q_idx + (row * H_I + h) * DI, g), h < H_I);
#pragma unroll
    for (int i = 0; i < KS; ++i) qa[hb][i] = as_long(f.w[2 * i], f.w[2 * i + 1]);
  }
  __syncthreads();

  const int64_t tile0 = (int64_t)blockIdx.x * tile;
  const int pitch = (H_I + 3) & ~3;
  float* my = dots[wave];
  const uint8_t* kb = k_idx + b * k_bstride;
  const int32_t* prow = GATHER ? pool_idx + row * (int64_t)pool_cap : nullptr;

  // Each wave owns tile/4 consecutive positions, SG*16 per iteration; the
  // next iteration's key rows are in flight while this one is scored.
  constexpr int SG = kScanGroups<HB>;
  constexpr int IT = 16 * SG;
  const int64_t wbase = tile0 + (int64_t)wave * (tile / kScanWaves);
  int64_t wend = wbase + tile / kScanWaves;
  if (wend > nv) wend = nv;

  auto frag_ptr = [&](int64_t pos, bool& ok) -> const uint8_t* {
    ok = pos < wend;
    int64_t tokid = pos;
    if (GATHER && ok) tokid = prow[pos];
    return frag_base<DI>(kb + (ok ? tokid : 0) * k_rstride, g);
  };

  // Two fragment buffers used in ping-pong: while one batch of IT tokens is
  // scored, the other batch's loads are in flight.
  Frag<CH> fa[SG], fb[SG];
  auto load_batch = [&](Frag<CH>(&f)[SG], int64_t base) {
#pragma unroll
    for (int s = 0; s < SG; ++s) {
      bool ok;
      const uint8_t* p = frag_ptr(base + 16 * s + c16, ok);
      load_frag<CH, DI>(f[s], p, ok);
    }
  };
  auto score_batch = [&](const Frag<CH>(&f)[SG], int64_t it) {
#pragma unroll
    for (int s = 0; s < SG; ++s) {
#pragma unroll
      for (int hb = 0; hb < HB; ++hb) {
        v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < KS; ++i)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qa[hb][i], as_long(f[s].w[2 * i], f[s].w[2 * i + 1]),
                                                           acc, 0, 0, 0);
        // acc[r] = dot(head 16*hb + 4*g + r, token 16*s + c16)
        int h0 = 16 * hb + 4 * g;
        if (h0 < H_I) *reinterpret_cast<v4f*>(my + (16 * s + c16) * pitch + h0) = acc;
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
#pragma unroll
    for (int u = 0; u < SG / 4; ++u) {
      // Lane owns token it + 64u + lane.
      const int64_t j = it + 64 * u + lane;
      const bool vis = j < wend;
      float sc = 0.0f;
      const float* src = my + (64 * u + lane) * pitch;
#pragma unroll
      for (int h4 = 0; h4 < HMAX; h4 += 4) {
        if (h4 < pitch) {
          const v4f d4 = *reinterpret_cast<const v4f*>(src + h4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // heads past H_I have weight 0: adding +0 leaves the sum unchanged
            float r = d4[e] > 0.0f ? d4[e] : 0.0f;
            sc = __fadd_rn(sc, __fmul_rn(wv[h4 + e], r));
          }
        }
      }
      uint32_t key = vis ? score_key(sc) : 0u;
      if (vis) {
        keys[row * key_stride + j] = key;
        atomicAdd(&hist[key >> 20], 1u);
      }
      if (pool) {
        uint32_t m = key;
        for (int off = 1; off < pool_block; off <<= 1) {
          uint32_t o = __shfl_xor(m, off, 64);
          m = m > o ? m : o;
        }
        if (vis && (j % pool_block) == 0) {
          bkeys[row * bkey_stride + j / pool_block] = m;
          atomicAdd(&bhist[m >> 20], 1u);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  if (wbase < wend) load_batch(fa, wbase);
  for (int64_t it = wbase; it < wend; it += 2 * IT) {
    const bool has_b = it + IT < wend;
    if (has_b) load_batch(fb, it + IT);
    score_batch(fa, it);
    if (it + 2 * IT < wend) load_batch(fa, it + 2 * IT);
    if (has_b) score_batch(fb, it + IT);
  }
  __syncthreads();
  uint32_t* gh = tok.hist1 + row * 4096;
  for (int i = threadIdx.x; i < 4096; i += 256)
    if (hist[i]) atomic_add_agent(gh + i, hist[i]);
  uint32_t* gbh = pool ? blk.hist1 + row * 4096 : nullptr;
  if (pool)
    for (int i = threadIdx.x; i < 4096; i += 256)
      if (bhist[i]) atomic_add_agent(gbh + i, bhist[i]);
}

template <int DI, int HB>
static hipError_t launch_scan_t(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                                const SelectWs* blk, hipStream_t s) {
  int64_t rows = (int64_t)a.B * a.Tq;
  // Largest tile (fewest histogram flushes) that still gives >= 4 workgroups
  // per compute unit; at least 1024 tokens.
  int tile = kScanTile;
  const int64_t want = 4LL * device_cu_count();
  while (tile > 1024 && rows * ((a.n_max + tile - 1) / tile) < want) tile >>= 1;
  int64_t tiles = (a.n_max + tile - 1) / tile;
  if (tiles < 1) tiles = 1;
  SelectWs bw = blk ? *blk : tok;
  dim3 grid((unsigned)tiles, (unsigned)rows);
  if (a.pool_block > 0) {
    CSA2_LAUNCH("index_score", (index_score_kernel<DI, HB, false, true>), grid, dim3(256), 0, s, a.q_idx, a.w,
                a.k_idx, a.k_bstride, a.k_rstride, a.ctx_len, a.q_pos, (const int32_t*)nullptr,
                (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys, key_stride, n_valid, tok,
                a.pool_block, a.pool_nblocks, bkeys, bkey_stride, nb_valid, bw);
  } else {
    CSA2_LAUNCH("index_score", (index_score_kernel<DI, HB, false, false>), grid, dim3(256), 0, s, a.q_idx, a.w,
                a.k_idx, a.k_bstride, a.k_rstride, a.ctx_len, a.q_pos, (const int32_t*)nullptr,
                (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys, key_stride, n_valid, tok, 0,
                0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, bw);
  }
  return hipGetLastError();
}

template <int DI, int HB>
static hipError_t launch_pool_t(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                                int64_t k_rstride, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                                int B, int Tq, int H_I, int k_top, uint32_t* keys, int64_t key_stride,
                                int32_t* n_valid, const SelectWs& ws, hipStream_t s) {
  int64_t rows = (int64_t)B * Tq;
  int64_t tiles = (pool_cap + kPoolTile - 1) / kPoolTile;
  if (tiles < 1) tiles = 1;
  CSA2_LAUNCH("pool_score", (index_score_kernel<DI, HB, true, false>), dim3((unsigned)tiles, (unsigned)rows), dim3(256),
              0, s, q_idx, w, k_idx, k_bstride, k_rstride, (const int32_t*)nullptr, (const int32_t*)nullptr,
              pool_idx, pool_len, pool_cap, Tq, H_I, (int64_t)pool_cap, k_top, kPoolTile, keys, key_stride, n_valid, ws,
              0, 0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, ws);
  return hipGetLastError();
}

#define CSA2_DISPATCH_DI_HB(DI_, HB_, CALL)                                       \
  do {                                                                           \
    int hb__ = (HB_) <= 16 ? 1 : 2;                                              \
    switch (DI_) {                                                               \
      case 32: return hb__ == 1 ? CALL(32, 1) : CALL(32, 2);                      \
      case 64: return hb__ == 1 ? CALL(64, 1) : CALL(64, 2);                      \
      case 128: return hb__ == 1 ? CALL(128, 1) : CALL(128, 2);                   \
      case 256: return hb__ == 1 ? CALL(256, 1) : CALL(256, 2);                   \
      default: return hipErrorInvalidValue;                                       \
    }                                                                            \
  } while (0)

hipError_t launch_index_score(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                              const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                              const SelectWs* blk, hipStream_t s) {
#define CALL_SCAN(D, H) launch_scan_t<D, H>(a, keys, key_stride, n_valid, tok, bkeys, bkey_stride, nb_valid, blk, s)
  CSA2_DISPATCH_DI_HB(a.D_I, a.H_I, CALL_SCAN);
#undef CALL_SCAN
}

hipError_t launch_pool_score(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                             int64_t k_rstride, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                             int B, int Tq, int H_I, int D_I, int k_top, uint32_t* keys, int64_t key_stride,
                             int32_t* n_valid, const SelectWs& ws, hipStream_t s) {
#define CALL_POOL(D, H) \
  launch_pool_t<D, H>(q_idx, w, k_idx, k_bstride, k_rstride, pool_idx, pool_len, pool_cap, B, Tq, H_I, k_top, keys, \
                      key_stride, n_valid, ws, s)
  CSA2_DISPATCH_DI_HB(D_I, H_I, CALL_POOL);
#undef CALL_POOL
}

}  // namespace csa2
