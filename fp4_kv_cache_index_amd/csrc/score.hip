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

// Waves per workgroup: 16 for the flat scan with one head block (one large
// tile per compute unit, so that each workgroup's prologue, histogram flush
// and key burst are paid once per 16K tokens), 4 for the pool gather and the
// wide-head variants (their LDS tiles are larger).
template <bool GATHER, int HB>
constexpr int kScanWavesT = (!GATHER && HB == 1) ? 16 : 4;
constexpr int kScanTileMax = 16384;   // flat-scan tokens per 16-wave workgroup (largest)
constexpr int kScanTileSmall = 1024;  // flat-scan tokens per 4-wave workgroup
constexpr int kPoolTile = 512;        // pool positions per workgroup (later layers)
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
template <int DI, int HB, bool GATHER, bool POOL, bool H8>
__global__ void __launch_bounds__((64 * kScanWavesT<GATHER, HB>))
index_score_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                   const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                   const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                   const int32_t* __restrict__ pool_idx, const int32_t* __restrict__ pool_len, int pool_cap,
                   int Tq, int H_I, int64_t n_max, int k_top, int tile,
                   uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                   SelectWs tok,
                   int pool_block, int nblocks, uint32_t* __restrict__ bkeys, int64_t bkey_stride,
                   int32_t* __restrict__ nb_valid_out, SelectWs blk) {
  constexpr int NW = kScanWavesT<GATHER, HB>;
  constexpr int NT = 64 * NW;
  constexpr int CH = DI / 4;           // bytes of a key row per lane
  constexpr int KS = DI / 32;          // MFMA k-steps
  constexpr int HMAX = 16 * HB;
  // Heads kept per token: 8 when the indexer has at most 8 heads, else all
  // 16*HB MFMA rows (padding heads have zero queries and weight 0).
  constexpr int HP = H8 ? 8 : HMAX;
  // Top-12-bit histogram, two 16-bit bins per word (a tile holds at most
  // 16384 positions); the last word takes positions past the visible count.
  __shared__ __attribute__((aligned(16))) uint32_t hist[2052];
  // Flat scan: the tile's keys are staged here and leave in one coalesced
  // burst at the end (interleaving small key stores with the key-row stream
  // costs more than the LDS round trip).
  constexpr bool kStage = !GATHER && !POOL;
  __shared__ __attribute__((aligned(16))) uint32_t kst[kStage ? (NW == 16 ? kScanTileMax : kScanTileSmall) : 1];
  __shared__ int32_t ptok[GATHER ? kPoolTile : 1];   // pool token ids of this tile
  __shared__ uint32_t bhist[POOL ? 4096 : 1];
  // per wave: the batch's dots, then one 4-float trash slot per lane (whole-line path)
  __shared__ __attribute__((aligned(16))) float dots[NW][16 * kScanGroups<HB> * HP + 256];
  __shared__ float wsh[HMAX];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t row = blockIdx.y;
  const int64_t b = row / Tq;
  constexpr bool pool = POOL;
  if (n_max <= 0) {   // nothing addressable: no position is visible
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      n_valid_out[row] = 0;
      if (pool) nb_valid_out[row] = 0;
    }
    return;
  }
  const int c16 = lane & 15, g = lane >> 4;
  constexpr bool FULL = (DI == 128 && HB == 1 && kScanGroups<HB> == 4);
  const int64_t tile0 = (int64_t)blockIdx.x * tile;
  constexpr int pitch = HP;
  float* my = dots[wave];
  const uint8_t* kb = k_idx + b * k_bstride;
  // Each wave owns tile/4 consecutive positions, SG*16 per iteration; the
  // next iteration's key rows are in flight while this one is scored.  Loads
  // are issued unconditionally (positions past the wave's range read the
  // last row of the range again, or 0 through the buffer range check, and
  // are never scored) so that waiting for one batch never waits for the
  // batch behind it.
  constexpr int SG = kScanGroups<HB>;
  constexpr int IT = 16 * SG;
  const int64_t wbase = tile0 + (int64_t)wave * (tile / NW);
  // Until the visible count is known, loads are clamped to the addressable
  // rows only (n_max > 0 here); rows past the visible count are never scored.
  int64_t wend = wbase + tile / NW;
  if (wend > n_max) wend = n_max;
  int64_t wlast = wend - 1;

  auto frag_ptr = [&](int64_t pos) -> const uint8_t* {
    const int64_t p = pos < wend ? pos : wlast;
    const int64_t tokid = GATHER ? (int64_t)ptok[p - tile0] : p;
    return frag_base<DI>(kb + tokid * k_rstride, g);
  };
  auto full_ptr = [&](int64_t pos) -> const uint8_t* {
    const int64_t p = pos < wend ? pos : wlast;
    const int64_t tokid = GATHER ? (int64_t)ptok[p - tile0] : p;
    return kb + tokid * k_rstride + 16 * (2 * g + (c16 & 1));
  };

  // Flat whole-line scan: buffer loads over exactly the wave's rows (the
  // hardware returns 0 for offsets past the end, without a memory access),
  // so no row clamps; offsets are 32-bit (row strides below 4 MiB).
  constexpr bool BUF = FULL && !GATHER;
  const uint32_t rs32 = (uint32_t)k_rstride;
  const uint32_t lane_off = (uint32_t)(c16 >> 1) * rs32 + 16u * (uint32_t)(2 * g + (c16 & 1));
  auto wave_rsrc = [&](int64_t lim) {
    const int64_t n = lim > wbase ? (lim - wbase) * k_rstride : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kb + wbase * k_rstride), (short)0,
                                             (int)(n < 0xFFFFFFFFLL ? n : 0xFFFFFFFFLL), 0x00020000);
  };
  __amdgpu_buffer_rsrc_t krs = wave_rsrc(wend);
  // Two fragment buffers used in ping-pong: while one batch of IT tokens is
  // scored, the other batch's loads are in flight.
  Frag<CH> fa[SG], fb[SG];
  auto load_batch = [&](Frag<CH>(&f)[SG], int64_t base) {
    if constexpr (BUF) {
      const uint32_t boff = (uint32_t)(base - wbase) * rs32;
#pragma unroll
      for (int u = 0; u < 2 * SG; ++u) {
        // (the uniform part stays in a scalar register: offsets recomputed per
        // batch instead of eight loop-invariant vector registers)
        const uint32_t uoff = __builtin_amdgcn_readfirstlane(boff + (uint32_t)(8 * u) * rs32);
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(krs, lane_off + uoff, 0, 2 /* non-temporal */);
        f[u >> 1].w[4 * (u & 1) + 0] = v[0]; f[u >> 1].w[4 * (u & 1) + 1] = v[1];
        f[u >> 1].w[4 * (u & 1) + 2] = v[2]; f[u >> 1].w[4 * (u & 1) + 3] = v[3];
      }
    } else if constexpr (FULL) {
      // 8 groups of 8 tokens; group u = 2s + half lands in f[s].w[4*half ..]
#pragma unroll
      for (int u = 0; u < 2 * SG; ++u) {
        const v4u v = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(full_ptr(base + 8 * u + (c16 >> 1))));
        f[u >> 1].w[4 * (u & 1) + 0] = v[0]; f[u >> 1].w[4 * (u & 1) + 1] = v[1];
        f[u >> 1].w[4 * (u & 1) + 2] = v[2]; f[u >> 1].w[4 * (u & 1) + 3] = v[3];
      }
    } else {
#pragma unroll
      for (int s = 0; s < SG; ++s) load_frag<CH, DI>(f[s], frag_ptr(base + 16 * s + c16), true);
    }
  };

  // Prologue loads first (visible count, weights, query fragments); the
  // flat scan then issues its first two key batches at once, so that the
  // stream starts while these are in flight (the vector-memory counter
  // retires in order: waiting for them below does not wait for the keys).
  int64_t craw;
  if (GATHER) craw = pool_len[row];
  else {
    craw = ctx_len[b];
    if (q_pos) {
      const int64_t qp = (int64_t)q_pos[row] + 1;
      if (qp < craw) craw = qp;
    }
  }
  // Unconditional loads from in-range addresses; the zeroing of heads past
  // H_I happens after the key loads are issued (a select on a loaded value
  // waits for it, and the counter retires in order).
  const float wraw = w[row * H_I + (threadIdx.x < H_I ? threadIdx.x : H_I - 1)];
  // Whole-line loads (D_I = 128, one head block): every token of a group of
  // 8 takes two B columns -- 2m holds bytes 32g..32g+15 of its row, 2m+1
  // bytes 32g+16..32g+31 (lane group g) -- so the 8 lanes of a token read its
  // whole 128-byte row in one instruction.  Two MFMA pairs with the matching
  // halves of the query rows give the two partial dots, which one adjacent-
  // lane exchange joins (exact: integers below 2^24).
  // A operand: query head (lane & 15) + 16*hb, slice (lane >> 4) of the row.
  long qh[2][2];   // FULL: [parity e][step s] = bytes 32g + 16e + 8s .. +8
  long qa[HB][KS];
  const bool hv = c16 < H_I;
  if constexpr (FULL) {
    const uint8_t* qp = q_idx + (row * H_I + (hv ? c16 : 0)) * DI + 32 * g;
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const v2u v = *reinterpret_cast<const v2u*>(qp + 16 * e + 8 * st);
        qh[e][st] = as_long(v[0], v[1]);
      }
  } else {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      int h = c16 + 16 * hb;
      Frag<CH> f;
      load_frag<CH, DI>(f, frag_base<DI>(q_idx + (row * H_I + h) * DI, g), h < H_I);
#pragma unroll
      for (int i = 0; i < KS; ++i) qa[hb][i] = as_long(f.w[2 * i], f.w[2 * i + 1]);
    }
  }
  if constexpr (!GATHER) {
    load_batch(fa, wbase);
    load_batch(fb, wbase + IT);
    __builtin_amdgcn_sched_barrier(0);   // keep them ahead of the prologue's waits
  }
  if constexpr (FULL) {
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int st = 0; st < 2; ++st) qh[e][st] = hv ? qh[e][st] : 0L;
    // The query fragments must have arrived before the stream loop (so that
    // the loop's waits cover only its own batches).
    asm volatile("" ::"v"(qh[0][0]), "v"(qh[0][1]), "v"(qh[1][0]), "v"(qh[1][1]));
  }
  const float wload = threadIdx.x < HMAX && threadIdx.x < H_I ? wraw : 0.0f;

  int64_t nv;
  if (GATHER) nv = craw < 0 ? 0 : (craw > pool_cap ? pool_cap : craw);
  else nv = craw < 0 ? 0 : (craw > n_max ? n_max : craw);
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    n_valid_out[row] = (int32_t)nv;
    if (pool) nb_valid_out[row] = (int32_t)((nv + pool_block - 1) / pool_block);
  }

  for (int i = threadIdx.x; i < 4096; i += NT) {
    if (i <= 2048) hist[i] = 0u;
    if (pool) bhist[i] = 0u;
  }
  if (threadIdx.x < HMAX) wsh[threadIdx.x] = wload;
  __syncthreads();
  float wv[HP];   // head weights (0 past H_I), wave-uniform: scalar registers
#pragma unroll
  for (int h = 0; h < HP; ++h)
    wv[h] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, wsh[h])));
  if (GATHER) {   // pool token ids of the tile, read from LDS by the loads below
    const int32_t* prow = pool_idx + row * (int64_t)pool_cap;
    for (int i = threadIdx.x; i < tile; i += NT) {
      const int64_t p = tile0 + i;
      ptok[i] = p < nv ? prow[p] : 0;
    }
    __syncthreads();
  }

  // From here on the wave's range ends at the visible count.
  wend = wbase + tile / NW;
  if (wend > nv) wend = nv;
  wlast = wend - 1;
  if constexpr (BUF) krs = wave_rsrc(wend);

  auto score_batch = [&](const Frag<CH>(&f)[SG], int64_t it) {
    if constexpr (FULL) {
#pragma unroll
      for (int u = 0; u < 2 * SG; ++u) {
        const uint32_t* w4 = &f[u >> 1].w[4 * (u & 1)];
        const long lo = as_long(w4[0], w4[1]), hi = as_long(w4[2], w4[3]);
        v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[0][0], lo, a0, 0, 0, 0);
        a0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[0][1], hi, a0, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[1][0], lo, a1, 0, 0, 0);
        a1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[1][1], hi, a1, 0, 0, 0);
        // even column 2m: a0 here plus a1 of the odd column 2m+1 (lane + 1).
        // (__shfl_xor: the DPP builtins applied to elements of an MFMA result
        // were folded into a single element by this compiler.)
        v4f d;
#pragma unroll
        for (int r = 0; r < 4; ++r) d[r] = a0[r] + __shfl_xor(a1[r], 1, 64);
        // d[r] = dot(head 4g + r, token 8u + m) on the even lanes; the other
        // lanes write their own trash slot (no branch around the loads' waits)
        const bool keep = (c16 & 1) == 0 && 4 * g < HP;
        const int at = keep ? (8 * u + (c16 >> 1)) * pitch + 4 * g : 16 * SG * HP + 4 * lane;
        *reinterpret_cast<v4f*>(my + at) = d;
      }
    } else {
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
        const int h0 = 16 * hb + 4 * g;
        if (h0 < HP) *reinterpret_cast<v4f*>(my + (16 * s + c16) * pitch + h0) = acc;
      }
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
      for (int h4 = 0; h4 < HP; h4 += 4) {
        const v4f d4 = *reinterpret_cast<const v4f*>(src + h4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // heads past H_I have weight 0: adding +0 leaves the sum unchanged
          float r = d4[e] > 0.0f ? d4[e] : 0.0f;
          sc = __fadd_rn(sc, __fmul_rn(wv[h4 + e], r));
        }
      }
      // Positions up to the next multiple of 64 lie inside the row's key
      // stride and belong to no other wave; past the visible count they are
      // never read.
      uint32_t key = vis ? score_key(sc) : 0u;
      if (kStage) kst[j - tile0] = key;
      else keys[row * key_stride + j] = key;
      atomicAdd(&hist[vis ? key >> 21 : 2048u], 1u << (16 * ((key >> 20) & 1u)));
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

  const int nb = wend > wbase ? (int)((wend - wbase + IT - 1) / IT) : 0;
  if constexpr (GATHER) {
    if (nb > 0) {
      load_batch(fa, wbase);
      load_batch(fb, wbase + IT);
    }
  }
  for (int ib = 0; ib < nb; ib += 2) {
    score_batch(fa, wbase + (int64_t)ib * IT);
    load_batch(fa, wbase + (int64_t)(ib + 2) * IT);
    if (ib + 1 < nb) score_batch(fb, wbase + (int64_t)(ib + 1) * IT);
    load_batch(fb, wbase + (int64_t)(ib + 3) * IT);
  }
  __syncthreads();
  if (kStage) {
    int64_t tend = tile0 + tile;
    if (tend > nv) tend = nv;
    // Whole 64-position groups: they stay inside the row's key stride.
    const int64_t tn = tend > tile0 ? ((tend - tile0 + 63) & ~63LL) : 0;
    for (int64_t i = 4 * threadIdx.x; i < tn; i += 4 * NT)
      *reinterpret_cast<v4u*>(keys + row * key_stride + tile0 + i) = *reinterpret_cast<const v4u*>(&kst[i]);
  }
  // Two adjacent bins per 64-bit atomic: the row histogram's 32-bit counters
  // 2i and 2i+1 are the low and high halves of one little-endian 64-bit word.
  if (tok.hist1) {
    uint64_t* gh = reinterpret_cast<uint64_t*>(tok.hist1 + row * 4096);
    for (int i = threadIdx.x; i < 2048; i += NT) {
      const uint32_t v = hist[i];
      if (v) atomic_add_agent64(gh + i, (uint64_t)(v & 0xFFFFu) | ((uint64_t)(v >> 16) << 32));
    }
  } else if (tok.tile_hist) {
    // The tile's histogram as it stands (two 16-bit bins per word), one slot
    // per tile: plain stores, nothing to clear beforehand.
    v4u* th = reinterpret_cast<v4u*>(tok.tile_hist + (row * tok.th_stride + blockIdx.x) * 2048);
    for (int i = threadIdx.x; i < 512; i += NT) th[i] = reinterpret_cast<const v4u*>(hist)[i];
  }
  if (pool) {
    uint64_t* gbh = reinterpret_cast<uint64_t*>(blk.hist1 + row * 4096);
    for (int i = threadIdx.x; i < 2048; i += NT) {
      const uint32_t lo = bhist[2 * i], hi = bhist[2 * i + 1];
      if (lo | hi) atomic_add_agent64(gbh + i, (uint64_t)lo | ((uint64_t)hi << 32));
    }
  }
}

// Flat-scan tile: the largest that still gives every compute unit a
// workgroup (16-wave workgroups), else kScanTileSmall.
static int scan_tile(int64_t rows, int64_t n_max, int nw) {
  int tile = nw == 16 ? kScanTileMax : kScanTileSmall;
  while (tile > kScanTileSmall && rows * ((n_max + tile - 1) / tile) < device_cu_count()) tile >>= 1;
  return tile;
}

template <int DI, int HB, bool H8>
static hipError_t launch_scan_t(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                                const SelectWs* blk, hipStream_t s) {
  int64_t rows = (int64_t)a.B * a.Tq;
  constexpr int NW = kScanWavesT<false, HB>;
  const int tile = scan_tile(rows, a.n_max, NW);
  int64_t tiles = (a.n_max + tile - 1) / tile;
  if (tiles < 1) tiles = 1;
  SelectWs bw = blk ? *blk : tok;
  dim3 grid((unsigned)tiles, (unsigned)rows);
  if (a.pool_block > 0) {
    CSA2_LAUNCH("index_score", (index_score_kernel<DI, HB, false, true, H8>), grid, dim3(64 * NW), 0, s, a.q_idx, a.w,
                a.k_idx, a.k_bstride, a.k_rstride, a.ctx_len, a.q_pos, (const int32_t*)nullptr,
                (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys, key_stride, n_valid, tok,
                a.pool_block, a.pool_nblocks, bkeys, bkey_stride, nb_valid, bw);
  } else {
    CSA2_LAUNCH("index_score", (index_score_kernel<DI, HB, false, false, H8>), grid, dim3(64 * NW), 0, s, a.q_idx, a.w,
                a.k_idx, a.k_bstride, a.k_rstride, a.ctx_len, a.q_pos, (const int32_t*)nullptr,
                (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys, key_stride, n_valid, tok, 0,
                0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, bw);
  }
  return hipGetLastError();
}

template <int DI, int HB, bool H8>
static hipError_t launch_pool_t(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                                int64_t k_rstride, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                                int B, int Tq, int H_I, int k_top, uint32_t* keys, int64_t key_stride,
                                int32_t* n_valid, const SelectWs& ws, hipStream_t s) {
  int64_t rows = (int64_t)B * Tq;
  int64_t tiles = (pool_cap + kPoolTile - 1) / kPoolTile;
  if (tiles < 1) tiles = 1;
  CSA2_LAUNCH("pool_score", (index_score_kernel<DI, HB, true, false, H8>), dim3((unsigned)tiles, (unsigned)rows),
              dim3(64 * kScanWavesT<true, HB>),
              0, s, q_idx, w, k_idx, k_bstride, k_rstride, (const int32_t*)nullptr, (const int32_t*)nullptr,
              pool_idx, pool_len, pool_cap, Tq, H_I, (int64_t)pool_cap, k_top, kPoolTile, keys, key_stride, n_valid, ws,
              0, 0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, ws);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Prefill chunk: many queries of one sequence against the same keys, so the
// scores form a dense product [queries x heads] x [D_I] . [D_I] x [keys] and
// run on the gfx950 FP8 matrix cores at full rate
// (v_mfma_scale_f32_16x16x128_f8f6f4, unit E8M0 scales).  A workgroup holds
// QW = 4*QG queries of one sequence and a tile of keys; its 8 waves split the
// tile into 16-key chunks.  For 4 queries, MFMA number hg takes A rows
// (query 4qg + r/4, head 4hg + r%4), so in the result lane l holds
// query 4qg + l/16, heads 4hg..4hg+3 of key l%16: all heads of one
// (query, key) pair end up in one lane, which adds them in ascending order
// with float32 roundings and no FMA (padding heads carry weight 0).  Each
// lane loads bytes [16g, 16g+16) and [64+16g, 64+16g+16) of each 128-byte
// k-step for both operands, so the k-permutation matches on both sides.
// The epilogue writes the score keys and builds per-query 12-bit histograms
// in LDS, two queries per 32-bit word (counts stay below 2^16 per tile).
constexpr int kPrefillWaves = 8;

template <int DI>
__device__ __forceinline__ void load_k128(uint32_t (&f)[DI / 16], const uint8_t* row, int g, bool ok) {
  if (!ok) {
#pragma unroll
    for (int i = 0; i < DI / 16; ++i) f[i] = 0u;
    return;
  }
#pragma unroll
  for (int ks = 0; ks < DI / 128; ++ks) {
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      v4u v = *reinterpret_cast<const v4u*>(row + 128 * ks + 64 * hf + 16 * g);
      f[8 * ks + 4 * hf + 0] = v[0]; f[8 * ks + 4 * hf + 1] = v[1];
      f[8 * ks + 4 * hf + 2] = v[2]; f[8 * ks + 4 * hf + 3] = v[3];
    }
  }
}

template <int DI, int HG, int QG>
__global__ void __launch_bounds__(64 * kPrefillWaves)
index_prefill_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                     const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                     const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                     int Tq, int H_I, int64_t n_max, int key_tile, int qtiles,
                     uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                     SelectWs tok) {
  constexpr int KS = DI / 128;          // MFMA k-steps
  constexpr int FW = DI / 16;           // fragment words per lane
  constexpr int QW = 4 * QG;            // queries per workgroup
  constexpr int HP = 4 * HG;            // heads incl. padding
  constexpr int NT = 64 * kPrefillWaves;
  typedef int v8i __attribute__((ext_vector_type(8)));
  __shared__ uint32_t hist[(QW / 2) * 4096];
  __shared__ int32_t nvs[QW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.y / qtiles;
  const int t0 = (int)(blockIdx.y % qtiles) * QW;
  const int64_t row0 = b * Tq + t0;

  if (threadIdx.x < QW) {
    const int t = t0 + threadIdx.x;
    int64_t nv = 0;
    if (t < Tq) {
      nv = ctx_len[b];
      if (q_pos) {
        int64_t qp = (int64_t)q_pos[row0 + threadIdx.x] + 1;
        if (qp < nv) nv = qp;
      }
      nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
      if (blockIdx.x == 0) n_valid_out[row0 + threadIdx.x] = (int32_t)nv;
    }
    nvs[threadIdx.x] = (int32_t)nv;
  }
  for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) hist[i] = 0u;
  __syncthreads();
  int max_nv = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) max_nv = nvs[i] > max_nv ? nvs[i] : max_nv;
  const int64_t k0 = (int64_t)blockIdx.x * key_tile;
  int64_t k1 = k0 + key_tile;
  if (k1 > max_nv) k1 = max_nv;
  if (k0 >= k1) return;   // uniform: nothing visible in this tile

  // A fragments: row c16 = (query 4qg + c16/4, head 4hg + c16%4).
  v8i qa[QG][HG][KS];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
#pragma unroll
    for (int hg = 0; hg < HG; ++hg) {
      const int t = t0 + 4 * qg + (c16 >> 2), h = 4 * hg + (c16 & 3);
      uint32_t f[FW];
      load_k128<DI>(f, q_idx + ((b * Tq + t) * H_I + h) * (int64_t)DI, g, t < Tq && h < H_I);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qa[qg][hg][ks] = v8i{(int)f[8 * ks], (int)f[8 * ks + 1], (int)f[8 * ks + 2], (int)f[8 * ks + 3],
                             (int)f[8 * ks + 4], (int)f[8 * ks + 5], (int)f[8 * ks + 6], (int)f[8 * ks + 7]};
    }
  }
  // Epilogue state of this lane: query 4qg + g of each group.
  float wv[QG][HP];
  int32_t nvq[QG];
  uint32_t* krow[QG];
#pragma unroll
  for (int qg = 0; qg < QG; ++qg) {
    const int ql = 4 * qg + g, t = t0 + ql;
#pragma unroll
    for (int h = 0; h < HP; ++h) wv[qg][h] = (t < Tq && h < H_I) ? w[(b * Tq + t) * H_I + h] : 0.0f;
    nvq[qg] = nvs[ql];
    krow[qg] = keys + (row0 + ql) * key_stride;
  }

  const uint8_t* kb = k_idx + b * k_bstride;
  const int nchunks = (int)((k1 - k0 + 15) >> 4);
  uint32_t fa[FW], fb[FW];
  auto load_chunk = [&](uint32_t (&f)[FW], int c) {
    const int64_t j = k0 + 16 * (int64_t)c + c16;
    load_k128<DI>(f, kb + (j < k1 ? j : k0) * k_rstride, g, j < k1);
  };
  auto score_chunk = [&](const uint32_t (&f)[FW], int c) {
    const int64_t j = k0 + 16 * (int64_t)c + c16;
    v8i kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = v8i{(int)f[8 * ks], (int)f[8 * ks + 1], (int)f[8 * ks + 2], (int)f[8 * ks + 3],
                   (int)f[8 * ks + 4], (int)f[8 * ks + 5], (int)f[8 * ks + 6], (int)f[8 * ks + 7]};
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      v4f acc[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        acc[hg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc[hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[qg][hg][ks], kf[ks], acc[hg], 0, 0, 0, 127,
                                                                     0, 127);
      }
      // acc[hg][i] = dot(query 4qg + g, head 4hg + i; key j)
      float sc = 0.0f;
#pragma unroll
      for (int hg = 0; hg < HG; ++hg)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r = acc[hg][i] > 0.0f ? acc[hg][i] : 0.0f;
          sc = __fadd_rn(sc, __fmul_rn(wv[qg][4 * hg + i], r));
        }
      if (j < nvq[qg]) {
        const uint32_t key = score_key(sc);
        __builtin_nontemporal_store(key, krow[qg] + j);
        const int ql = 4 * qg + g;
        atomicAdd(&hist[(ql >> 1) * 4096 + (key >> 20)], 1u << (16 * (ql & 1)));
      }
    }
  };
  int c = wave;
  if (c < nchunks) load_chunk(fa, c);
  for (; c < nchunks; c += 2 * kPrefillWaves) {
    const int cb = c + kPrefillWaves;
    if (cb < nchunks) load_chunk(fb, cb);
    score_chunk(fa, c);
    if (cb + kPrefillWaves < nchunks) load_chunk(fa, cb + kPrefillWaves);
    if (cb < nchunks) score_chunk(fb, cb);
  }
  __syncthreads();
  if (!tok.hist1) return;
  for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) {
    const uint32_t v = hist[i];
    if (!v) continue;
    const int p = i >> 12, bin = i & 4095;
    if (v & 0xFFFFu) atomic_add_agent(tok.hist1 + (row0 + 2 * p) * 4096 + bin, v & 0xFFFFu);
    if (v >> 16) atomic_add_agent(tok.hist1 + (row0 + 2 * p + 1) * 4096 + bin, v >> 16);
  }
}

// Variant for D_I = 128 and at most 8 indexer heads: the product is taken
// transposed, A = 16 keys of a chunk, B = one head of the workgroup's 16
// queries, one MFMA per head.  Lane l then holds, for query l%16, the dots of
// keys 4g..4g+3 (g = l/16) with every head in its own accumulator, so the
// head sum stays inside the lane and the four consecutive keys of one query
// leave in a single 16-byte store.
template <int PD>
__global__ void __launch_bounds__(64 * kPrefillWaves)
index_prefill_kt_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                        const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                        const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                        int Tq, int H_I, int64_t n_max, int key_tile, int qtiles,
                        uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                        SelectWs tok) {
  constexpr int DI = 128, FW = 8, QW = 16, HP = 8;
  constexpr int NT = 64 * kPrefillWaves;
  typedef int v8i __attribute__((ext_vector_type(8)));
  __shared__ uint32_t hist[(QW / 2) * 4096 + 1];   // last word: bin of invisible keys
  __shared__ int32_t nvs[QW];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t b = blockIdx.y / qtiles;
  const int t0 = (int)(blockIdx.y % qtiles) * QW;
  const int64_t row0 = b * Tq + t0;

  if (threadIdx.x < QW) {
    const int t = t0 + threadIdx.x;
    int64_t nv = 0;
    if (t < Tq) {
      nv = ctx_len[b];
      if (q_pos) {
        int64_t qp = (int64_t)q_pos[row0 + threadIdx.x] + 1;
        if (qp < nv) nv = qp;
      }
      nv = nv < 0 ? 0 : (nv > n_max ? n_max : nv);
      if (blockIdx.x == 0) n_valid_out[row0 + threadIdx.x] = (int32_t)nv;
    }
    nvs[threadIdx.x] = (int32_t)nv;
  }
  for (int i = threadIdx.x; i <= (QW / 2) * 4096; i += NT) hist[i] = 0u;
  __syncthreads();
  int max_nv = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) max_nv = nvs[i] > max_nv ? nvs[i] : max_nv;
  const int64_t k0 = (int64_t)blockIdx.x * key_tile;
  int64_t k1 = k0 + key_tile;
  if (k1 > max_nv) k1 = max_nv;
  if (k0 >= k1) return;   // uniform: nothing visible in this tile

  // B fragments: column c16 = query t0 + c16, one per head.
  const int t = t0 + c16;
  const bool tok_q = t < Tq;
  v8i qb[HP];
  float wv[HP];
#pragma unroll
  for (int h = 0; h < HP; ++h) {
    uint32_t f[FW];
    load_k128<DI>(f, q_idx + ((b * Tq + t) * H_I + h) * (int64_t)DI, g, tok_q && h < H_I);
    qb[h] = v8i{(int)f[0], (int)f[1], (int)f[2], (int)f[3], (int)f[4], (int)f[5], (int)f[6], (int)f[7]};
    wv[h] = (tok_q && h < H_I) ? w[(b * Tq + t) * H_I + h] : 0.0f;
  }
  const int32_t nvq = nvs[c16];
  uint32_t* krow = keys + (row0 + c16) * key_stride;
  const uint32_t hbase = (uint32_t)(c16 >> 1) * 4096u, add = 1u << (16 * (c16 & 1));
  constexpr uint32_t kTrash = (QW / 2) * 4096;

  // Positions fit in 32 bits (n_max <= 2^22).  Every load is issued
  // unconditionally from a clamped in-range row so that the compiler can
  // count the loads in flight instead of draining them all at each chunk.
  const int ik0 = (int)k0, ik1 = (int)k1;
  const uint8_t* kb = k_idx + b * k_bstride;
  const int nchunks = (ik1 - ik0 + 15) >> 4;
  uint32_t fk[PD][FW];
  auto load_chunk = [&](uint32_t (&f)[FW], int c) {
    int j = ik0 + 16 * c + c16;
    j = j < ik1 ? j : ik1 - 1;
    const uint8_t* p = kb + (int64_t)j * k_rstride + 16 * g;
    const v4u lo = *reinterpret_cast<const v4u*>(p);
    const v4u hi = *reinterpret_cast<const v4u*>(p + 64);
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
  };
  auto score_chunk = [&](const uint32_t (&f)[FW], int c) {
    const v8i ka = v8i{(int)f[0], (int)f[1], (int)f[2], (int)f[3], (int)f[4], (int)f[5], (int)f[6], (int)f[7]};
    v4f acc[HP];
#pragma unroll
    for (int h = 0; h < HP; ++h)
      acc[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb[h], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127,
                                                                0, 127);
    // acc[h][r] = dot(key j0 + r, query c16, head h)
    const int j0 = ik0 + 16 * c + 4 * g;
    uint32_t kk[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float sc = 0.0f;
#pragma unroll
      for (int h = 0; h < HP; ++h) {
        // ReLU on the bit pattern: negative floats (and -0) are negative integers.
        const int xi = __float_as_int(acc[h][r]);
        const float x = __int_as_float(xi > 0 ? xi : 0);
        sc = __fadd_rn(sc, __fmul_rn(wv[h], x));
      }
      // The sum starts at +0 and rounds to nearest, so it is never -0: the
      // order-preserving key needs no zero canonicalisation here.
      const uint32_t u = __float_as_uint(sc);
      const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
      const bool vis = j0 + r < nvq;
      kk[r] = vis ? key : 0u;
      atomicAdd(&hist[vis ? hbase + (key >> 20) : kTrash], add);
    }
    // Positions up to the next multiple of 16 lie inside the row's key
    // stride; entries past the visible count are never read.
    if (tok_q) *reinterpret_cast<v4u*>(krow + j0) = v4u{kk[0], kk[1], kk[2], kk[3]};
  };
  // Chunks c = wave, wave + 8, ...; PD chunks in flight per wave.
  int c = wave;
#pragma unroll
  for (int d = 0; d < PD; ++d) load_chunk(fk[d], c + d * kPrefillWaves);
  for (; c < nchunks; c += PD * kPrefillWaves) {
#pragma unroll
    for (int d = 0; d < PD; ++d) {
      const int cd = c + d * kPrefillWaves;
      if (cd < nchunks) score_chunk(fk[d], cd);
      load_chunk(fk[d], cd + PD * kPrefillWaves);
    }
  }
  __syncthreads();
  if (!tok.hist1) return;
  for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) {
    const uint32_t v = hist[i];
    if (!v) continue;
    const int p = i >> 12, bin = i & 4095;
    if (v & 0xFFFFu) atomic_add_agent(tok.hist1 + (row0 + 2 * p) * 4096 + bin, v & 0xFFFFu);
    if (v >> 16) atomic_add_agent(tok.hist1 + (row0 + 2 * p + 1) * 4096 + bin, v >> 16);
  }
}

template <int DI, int HG>
static hipError_t launch_prefill_t(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                   const SelectWs& tok, hipStream_t s) {
  constexpr int QG = (HG * (DI / 128) <= 2) ? 4 : (HG * (DI / 128) <= 4 ? 2 : 1);
  constexpr int QW = 4 * QG;
  const int qtiles = (a.Tq + QW - 1) / QW;
  const int64_t qrows = (int64_t)a.B * qtiles;
  // Key tiles: at most 8192 keys (per-tile counts stay below 2^16), smaller
  // while the grid would not cover the compute units twice.
  int key_tile = 8192;
  const int64_t want = 2LL * device_cu_count();
  while (key_tile > 512 && qrows * ((a.n_max + key_tile - 1) / key_tile) < want) key_tile >>= 1;
  int64_t tiles = (a.n_max + key_tile - 1) / key_tile;
  if (tiles < 1) tiles = 1;
  if (qrows > 65535) return hipErrorInvalidValue;
  if (DI == 128 && HG <= 2) {
    CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3>), dim3((unsigned)tiles, (unsigned)qrows),
                dim3(64 * kPrefillWaves), 0, s, a.q_idx, a.w, a.k_idx, a.k_bstride, a.k_rstride, a.ctx_len, a.q_pos,
                a.Tq, a.H_I, a.n_max, key_tile, qtiles, keys, key_stride, n_valid, tok);
  } else {
    CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG>), dim3((unsigned)tiles, (unsigned)qrows),
                dim3(64 * kPrefillWaves), 0, s, a.q_idx, a.w, a.k_idx, a.k_bstride, a.k_rstride, a.ctx_len,
                a.q_pos, a.Tq, a.H_I, a.n_max, key_tile, qtiles, keys, key_stride, n_valid, tok);
  }
  return hipGetLastError();
}

static bool prefill_gemm_applies(const ScoreArgs& a) {
  return a.Tq >= 16 && a.pool_block == 0 && (a.D_I == 128 || a.D_I == 256) && a.H_I <= 32;
}

static hipError_t launch_prefill(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                 const SelectWs& tok, hipStream_t s) {
  const int hg = (a.H_I + 3) / 4;
  const int HGp = hg <= 1 ? 1 : (hg <= 2 ? 2 : (hg <= 4 ? 4 : 8));
#define CALL_PF(D, H) launch_prefill_t<D, H>(a, keys, key_stride, n_valid, tok, s)
  if (a.D_I == 128) {
    switch (HGp) {
      case 1: return CALL_PF(128, 1);
      case 2: return CALL_PF(128, 2);
      case 4: return CALL_PF(128, 4);
      default: return CALL_PF(128, 8);
    }
  }
  switch (HGp) {
    case 1: return CALL_PF(256, 1);
    case 2: return CALL_PF(256, 2);
    case 4: return CALL_PF(256, 4);
    default: return CALL_PF(256, 8);
  }
#undef CALL_PF
}

#define CSA2_DISPATCH_DI_HB(DI_, HB_, CALL)                                       \
  do {                                                                           \
    int hb__ = (HB_) <= 8 ? 0 : ((HB_) <= 16 ? 1 : 2);                           \
    switch (DI_) {                                                               \
      case 32: return hb__ == 0 ? CALL(32, 1, true) : hb__ == 1 ? CALL(32, 1, false) : CALL(32, 2, false);      \
      case 64: return hb__ == 0 ? CALL(64, 1, true) : hb__ == 1 ? CALL(64, 1, false) : CALL(64, 2, false);      \
      case 128: return hb__ == 0 ? CALL(128, 1, true) : hb__ == 1 ? CALL(128, 1, false) : CALL(128, 2, false);  \
      case 256: return hb__ == 0 ? CALL(256, 1, true) : hb__ == 1 ? CALL(256, 1, false) : CALL(256, 2, false);  \
      default: return hipErrorInvalidValue;                                       \
    }                                                                            \
  } while (0)

hipError_t launch_index_score(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                              const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                              const SelectWs* blk, hipStream_t s) {
  if (prefill_gemm_applies(a)) return launch_prefill(a, keys, key_stride, n_valid, tok, s);
#define CALL_SCAN(D, H, E) launch_scan_t<D, H, E>(a, keys, key_stride, n_valid, tok, bkeys, bkey_stride, nb_valid, blk, s)
  CSA2_DISPATCH_DI_HB(a.D_I, a.H_I, CALL_SCAN);
#undef CALL_SCAN
}

int64_t index_score_tiles(const ScoreArgs& a) {
  if (prefill_gemm_applies(a)) return 0;
  const int64_t rows = (int64_t)a.B * a.Tq;
  const int tile = scan_tile(rows, a.n_max, a.H_I <= 16 ? kScanWavesT<false, 1> : kScanWavesT<false, 2>);
  const int64_t tiles = (a.n_max + tile - 1) / tile;
  return tiles < 1 ? 1 : tiles;
}

int64_t index_score_tiles_bound(int64_t n_max) {
  const int64_t tiles = (n_max + kScanTileSmall - 1) / kScanTileSmall;
  return tiles < 1 ? 1 : tiles;
}

hipError_t launch_pool_score(const uint8_t* q_idx, const float* w, const uint8_t* k_idx, int64_t k_bstride,
                             int64_t k_rstride, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                             int B, int Tq, int H_I, int D_I, int k_top, uint32_t* keys, int64_t key_stride,
                             int32_t* n_valid, const SelectWs& ws, hipStream_t s) {
#define CALL_POOL(D, H, E) \
  launch_pool_t<D, H, E>(q_idx, w, k_idx, k_bstride, k_rstride, pool_idx, pool_len, pool_cap, B, Tq, H_I, k_top, keys, \
                      key_stride, n_valid, ws, s)
  CSA2_DISPATCH_DI_HB(D_I, H_I, CALL_POOL);
#undef CALL_POOL
}

}  // namespace csa2
