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
#include <type_traits>

#include "common.h"
#include "internal.h"
#include "select_dev.h"

namespace csa2 {

// Waves per workgroup of the flat scan: 16 (one large tile per compute unit,
// so that each workgroup's prologue, histogram flush and key burst are paid
// once per 16K tokens), 8 for E4M3 keys with 17..32 heads (their key
// fragments and the two head blocks' results need twice the registers).  4
// for the pool gather (tiles of 512 pool positions).  With QT > 1 query rows
// of one sequence per workgroup (multi-query decode), 16 / QT waves: the
// per-wave dot buffers and the staged keys grow with QT.
template <bool GATHER, int HB, int QT = 1, bool F4 = false>
constexpr int kScanWavesT = QT > 1 ? 16 / QT : (GATHER ? 4 : ((HB == 1 || F4) ? 16 : 8));
constexpr int kScanTileMax = 16384;   // flat-scan tokens per 16-wave workgroup (largest)
constexpr int kScanTileSmall = 1024;  // smallest flat-scan tile
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

// 4 x 4 transpose across the lane groups g = lane >> 4 (rows of 16 lanes):
// on entry x[u] of lane (g, c) holds lane group g's value for index u; on
// exit x[s] holds the value that lane group s had for index g.  Two swap
// stages: the wave's halves (permlane32 swap: lanes 32..63 of the first
// operand trade places with lanes 0..31 of the second), then neighbouring
// rows (permlane16 swap: odd rows of the first with even rows of the
// second); the lane mapping of both was checked on the device.
__device__ __forceinline__ void transpose_lane_groups(float (&x)[4]) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, x[u]),
                                                    __builtin_bit_cast(unsigned, x[u + 2]), false, false);
    x[u] = __builtin_bit_cast(float, (unsigned)r[0]);
    x[u + 2] = __builtin_bit_cast(float, (unsigned)r[1]);
  }
#pragma unroll
  for (int s = 0; s < 4; s += 2) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, x[s]),
                                                    __builtin_bit_cast(unsigned, x[s + 1]), false, false);
    x[s] = __builtin_bit_cast(float, (unsigned)r[0]);
    x[s + 1] = __builtin_bit_cast(float, (unsigned)r[1]);
  }
}

// GATHER = false: tokens j = tile positions of the row (flat scan).
// GATHER = true : position p maps to token pool_idx[row][p] (pool layers);
//                 a pool id outside [0, ctx_len[b]) names no token: the
//                 position is not visible (key 0) and its loads read row 0.
// QT > 1 (D_I = 128, at most 8 indexer heads, flat scan only): the
// workgroup scores QT query rows of one sequence against the same key rows;
// query t takes MFMA rows 8t .. 8t+7 (its heads, zero-padded), so two
// queries fill one 16-row block and four take two, and the key stream is
// read once for all of them.
// F4: MXFP4 keys (the pages' indexer K: E2M1 codes, one E8M0 scale per 32
// channels, D_I = 128).  The products run on the scaled matrix instruction
// v_mfma_scale_f32_16x16x128_f8f6f4 with A = the E4M3 query rows and B = 16
// keys' codes, the E8M0 scale of each B lane's 32 channels passed per lane.
// Measured lane layout of that instruction (128 K values): an FP4 lane of
// group g holds K 32g .. 32g+31 in 16 bytes, low nibble first, so a lane
// takes bytes 16g .. 16g+15 of its key's code row and the byte g of its scale
// row; an FP8 lane of group g holds K 16g .. 16g+15 then 64+16g .. 64+16g+15,
// so the query fragments take those bytes.  With integer-valued queries the
// products and partial sums stay exact in fp32 while a key's four exponents
// span at most 11 binades.
template <int DI, int HB, bool GATHER, bool POOL, bool H8, int QT, bool F4>
__global__ void __launch_bounds__((64 * kScanWavesT<GATHER, HB, QT, F4>))
index_score_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                   const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                   const uint8_t* __restrict__ k_scales, int64_t ks_bstride, int64_t ks_rstride,
                   const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                   const int32_t* __restrict__ pool_idx, const int32_t* __restrict__ pool_len, int pool_cap,
                   int Tq, int H_I, int64_t n_max, int k_top, int tile,
                   uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                   SelectWs tok,
                   int pool_block, int nblocks, uint32_t* __restrict__ bkeys, int64_t bkey_stride,
                   int32_t* __restrict__ nb_valid_out, SelectWs blk) {
  static_assert(QT == 1 || (DI == 128 && HB == 1 && H8 && !GATHER && !POOL), "multi-query scan: flat, 8 heads");
  static_assert(!F4 || DI == 128, "MXFP4 keys: 128 channels");
  constexpr int NW = kScanWavesT<GATHER, HB, QT, F4>;
  constexpr int NT = 64 * NW;
  constexpr int CH = DI / 4;           // bytes of a key row per lane
  constexpr int KS = DI / 32;          // MFMA k-steps
  constexpr int HMAX = QT > 1 ? 8 * QT : 16 * HB;   // MFMA rows (query heads, padded)
  constexpr int RB = QT > 1 ? QT / 2 : (F4 ? HB : 1);   // 16-row blocks of the whole-line / MXFP4 paths
  // Heads kept per token: 8 per query when the indexer has at most 8 heads,
  // else all 16*HB MFMA rows (padding heads have zero queries and weight 0).
  constexpr int HP = H8 ? 8 * QT : HMAX;
  // Top-12-bit histogram of each query row, two 16-bit bins per word (a tile
  // holds at most 16384 positions); the last word takes positions past the
  // visible count.
  __shared__ __attribute__((aligned(16))) uint32_t hist[QT][2052];
  // Whole-line path: per wave the batch's dots, then one 4-float trash slot
  // per lane (the other paths move the dots to their token's lane in
  // registers: RT).
  constexpr bool FULL = !F4 && (DI == 128 && HB == 1 && kScanGroups<HB> == 4);
  constexpr bool RT = !FULL;
  constexpr int kDots = RT ? 1 : 16 * kScanGroups<HB> * HP + 256;
  __shared__ __attribute__((aligned(16))) float dots[NW][kDots];
  // Flat and pool scans: the tile's keys are staged here and leave in one
  // coalesced burst at the end (interleaving small key stores with the
  // key-row stream costs more than the LDS round trip); a pool scan whose
  // staged keys would not fit beside its block histogram stores them
  // directly.
  constexpr int kTileCap = 1024 * NW;
  constexpr bool kStage =
      !GATHER && (!POOL || 4 * (QT * 2052 + QT * kTileCap + 4096 + NW * kDots + HMAX) <= 150 * 1024);
  __shared__ __attribute__((aligned(16))) uint32_t kst[kStage ? QT * kTileCap : 1];
  __shared__ int32_t ptok[GATHER ? kPoolTile : 1];   // pool token ids of this tile
  __shared__ uint32_t bhist[POOL ? 4096 : 1];
  __shared__ float wsh[HMAX];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Query rows row .. row + nq - 1 of sequence b (QT == 1: row = blockIdx.y).
  const int ngrp = (Tq + QT - 1) / QT;
  const int64_t b = (int64_t)blockIdx.y / ngrp;
  const int t0 = (int)((int64_t)blockIdx.y - b * ngrp) * QT;
  const int64_t row = b * Tq + t0;
  const int nq = Tq - t0 < QT ? Tq - t0 : QT;
  constexpr bool pool = POOL;
  if (n_max <= 0) {   // nothing addressable: no position is visible
    if (blockIdx.x == 0 && threadIdx.x < nq) {
      n_valid_out[row + threadIdx.x] = 0;
      if (pool) nb_valid_out[row] = 0;
    }
    return;
  }
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t tile0 = (int64_t)blockIdx.x * tile;
  constexpr int pitch = HP;
  float* my = dots[wave];
  const uint8_t* kb = k_idx + b * k_bstride;
  const uint8_t* ksb = F4 ? k_scales + b * ks_bstride : nullptr;
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

  // (pool ids are staged as -1 when invalid: their loads read row 0)
  auto frag_ptr = [&](int64_t pos) -> const uint8_t* {
    const int64_t p = pos < wend ? pos : wlast;
    const int64_t tokid = GATHER ? (int64_t)max(ptok[p - tile0], 0) : p;
    return frag_base<DI>(kb + tokid * k_rstride, g);
  };
  auto full_ptr = [&](int64_t pos) -> const uint8_t* {
    const int64_t p = pos < wend ? pos : wlast;
    const int64_t tokid = GATHER ? (int64_t)max(ptok[p - tile0], 0) : p;
    return kb + tokid * k_rstride + 16 * (2 * g + (c16 & 1));
  };

  // Flat whole-line scan: buffer loads over exactly the wave's rows (the
  // hardware returns 0 for offsets past the end, without a memory access),
  // so no row clamps; offsets are 32-bit (row strides below 4 MiB).
  constexpr bool BUF = (FULL || F4) && !GATHER;
  static_assert(!F4 || kScanGroups<HB> == 4, "MXFP4 batches: four groups of 16 keys");
  const uint32_t rs32 = (uint32_t)k_rstride;
  const uint32_t ss32 = (uint32_t)ks_rstride;
  // FP8 whole lines: 8 lanes per key row; MXFP4: lane (c16, g) reads bytes
  // 16g .. 16g+15 of key c16's code row.
  const uint32_t lane_off = F4 ? (uint32_t)c16 * rs32 + 16u * (uint32_t)g
                               : (uint32_t)(c16 >> 1) * rs32 + 16u * (uint32_t)(2 * g + (c16 & 1));
  auto wave_rsrc = [&](int64_t lim) {
    const int64_t n = lim > wbase ? (lim - wbase) * k_rstride : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(kb + wbase * k_rstride), (short)0,
                                             (int)(n < 0xFFFFFFFFLL ? n : 0xFFFFFFFFLL), 0x00020000);
  };
  auto wave_srsrc = [&](int64_t lim) {   // MXFP4 scale rows of the wave
    const int64_t n = lim > wbase ? (lim - wbase) * ks_rstride : 0;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(ksb + wbase * ks_rstride), (short)0,
                                             (int)(n < 0xFFFFFFFFLL ? n : 0xFFFFFFFFLL), 0x00020000);
  };
  __amdgpu_buffer_rsrc_t krs = wave_rsrc(wend);
  __amdgpu_buffer_rsrc_t srs = F4 && BUF ? wave_srsrc(wend) : krs;
  // Two fragment buffers used in ping-pong: while one batch of IT tokens is
  // scored, the other batch's loads are in flight.
  Frag<CH> fa[SG], fb[SG];
  // MXFP4: f[u].w[0..3] = the codes of keys base + 16u + c16 (bytes 16g..),
  // f[0].w[4] = the 4-byte scale row of key base + lane.
  auto load_batch = [&](Frag<CH>(&f)[SG], int64_t base) {
    if constexpr (F4 && BUF) {
      const uint32_t boff = (uint32_t)(base - wbase) * rs32;
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        const uint32_t uoff = __builtin_amdgcn_readfirstlane(boff + (uint32_t)(16 * u) * rs32);
        const v4u v = __builtin_amdgcn_raw_buffer_load_b128(krs, lane_off + uoff, 0, 2 /* non-temporal */);
        f[u].w[0] = v[0]; f[u].w[1] = v[1]; f[u].w[2] = v[2]; f[u].w[3] = v[3];
      }
      const uint32_t soff = (uint32_t)(base - wbase + lane) * ss32;
      f[0].w[4] = __builtin_amdgcn_raw_buffer_load_b32(srs, soff, 0, 2);
    } else if constexpr (F4) {
      auto tok = [&](int64_t pos) -> int64_t {
        const int64_t p = pos < wend ? pos : wlast;
        return GATHER ? (int64_t)max(ptok[p - tile0], 0) : p;
      };
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        const v4u v = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(kb + tok(base + 16 * u + c16) * k_rstride + 16 * g));
        f[u].w[0] = v[0]; f[u].w[1] = v[1]; f[u].w[2] = v[2]; f[u].w[3] = v[3];
      }
      f[0].w[4] = *reinterpret_cast<const uint32_t*>(ksb + tok(base + lane) * ks_rstride);
    } else if constexpr (BUF) {
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
  int64_t craw;              // visible positions (the largest of the group's queries)
  int64_t cq[QT];            // QT > 1: per query
  int64_t ctx_b = 0;   // pool layers: ids at or past it name no token
  if (GATHER) {
    craw = pool_len[row];
    ctx_b = ctx_len[b];
  } else if constexpr (QT > 1) {
    const int64_t c = ctx_len[b];
    craw = 0;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      int64_t v = c;
      if (q_pos) {
        const int64_t qp = (int64_t)q_pos[row + (t < nq ? t : nq - 1)] + 1;
        if (qp < v) v = qp;
      }
      cq[t] = t < nq ? v : 0;
      craw = cq[t] > craw ? cq[t] : craw;
    }
  } else {
    craw = ctx_len[b];
    if (q_pos) {
      const int64_t qp = (int64_t)q_pos[row] + 1;
      if (qp < craw) craw = qp;
    }
  }
  // Unconditional loads from in-range addresses; the zeroing of heads past
  // H_I happens after the key loads are issued (a select on a loaded value
  // waits for it, and the counter retires in order).  QT > 1: thread i
  // holds head i % 8 of query i / 8.
  const int wq = QT > 1 ? (int)threadIdx.x >> 3 : 0, wh = QT > 1 ? (int)threadIdx.x & 7 : (int)threadIdx.x;
  const float wraw = w[(row + (wq < nq ? wq : nq - 1)) * H_I + (wh < H_I ? wh : H_I - 1)];
  // Whole-line loads (D_I = 128, one head block): every token of a group of
  // 8 takes two B columns -- 2m holds bytes 32g..32g+15 of its row, 2m+1
  // bytes 32g+16..32g+31 (lane group g) -- so the 8 lanes of a token read its
  // whole 128-byte row in one instruction.  Two MFMA pairs with the matching
  // halves of the query rows give the two partial dots, which one adjacent-
  // lane exchange joins (exact: integers below 2^24).
  // A operand: query head (lane & 15) + 16*hb, slice (lane >> 4) of the row.
  // QT > 1: A row 16*rb + (lane & 15) is head (row & 7) of query (row >> 3).
  long qh[RB][2][2];   // FULL: [row block][parity e][step s] = bytes 32g + 16e + 8s .. +8
  long qa[HB][KS];
  bool hv[RB];
  v8i qa4[F4 ? RB : 1];   // MXFP4: A = E4M3 query rows, bytes 16g.. and 64+16g.. (see the kernel's note)
  if constexpr (F4) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int R = 16 * rb + c16;
      const int qt = QT > 1 ? R >> 3 : 0, qhd = QT > 1 ? R & 7 : R;
      hv[rb] = qt < nq && qhd < H_I;
      const uint8_t* qp = q_idx + ((row + (hv[rb] ? qt : 0)) * H_I + (hv[rb] ? qhd : 0)) * DI;
      const v4u lo = *reinterpret_cast<const v4u*>(qp + 16 * g);
      const v4u hi = *reinterpret_cast<const v4u*>(qp + 64 + 16 * g);
      qa4[rb] = v8i{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
  } else if constexpr (FULL) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int R = 16 * rb + c16;
      const int qt = QT > 1 ? R >> 3 : 0, qhd = QT > 1 ? R & 7 : R;
      hv[rb] = qt < nq && qhd < H_I;
      const uint8_t* qp = q_idx + ((row + (hv[rb] ? qt : 0)) * H_I + (hv[rb] ? qhd : 0)) * DI + 32 * g;
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int st = 0; st < 2; ++st) {
          const v2u v = *reinterpret_cast<const v2u*>(qp + 16 * e + 8 * st);
          qh[rb][e][st] = as_long(v[0], v[1]);
        }
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
  if constexpr (F4) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      if (!hv[rb]) qa4[rb] = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      // (per element: the host pass rejects a 256-bit vector operand here and
      // would silently drop the kernel's host stub)
      asm volatile("" ::"v"(qa4[rb][0]), "v"(qa4[rb][1]), "v"(qa4[rb][2]), "v"(qa4[rb][3]), "v"(qa4[rb][4]),
                   "v"(qa4[rb][5]), "v"(qa4[rb][6]), "v"(qa4[rb][7]));
    }
  }
  if constexpr (FULL) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
      for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int st = 0; st < 2; ++st) qh[rb][e][st] = hv[rb] ? qh[rb][e][st] : 0L;
      // The query fragments must have arrived before the stream loop (so
      // that the loop's waits cover only its own batches).
      asm volatile("" ::"v"(qh[rb][0][0]), "v"(qh[rb][0][1]), "v"(qh[rb][1][0]), "v"(qh[rb][1][1]));
    }
  }
  const float wload = threadIdx.x < HMAX && wq < nq && wh < H_I ? wraw : 0.0f;

  int64_t nv;
  if (GATHER) nv = (craw < 0 || ctx_b <= 0) ? 0 : (craw > pool_cap ? pool_cap : craw);
  else nv = craw < 0 ? 0 : (craw > n_max ? n_max : craw);
  int64_t nvq[QT];   // visible positions of each query of the group
  if constexpr (QT > 1) {
#pragma unroll
    for (int t = 0; t < QT; ++t) nvq[t] = cq[t] < 0 ? 0 : (cq[t] > n_max ? n_max : cq[t]);
  } else {
    nvq[0] = nv;
  }
  if (blockIdx.x == 0 && threadIdx.x < nq) {
    int64_t v = nvq[0];
#pragma unroll
    for (int t = 1; t < QT; ++t) v = (int)threadIdx.x == t ? nvq[t] : v;
    n_valid_out[row + threadIdx.x] = (int32_t)v;
    if (pool) nb_valid_out[row] = (int32_t)((nv + pool_block - 1) / pool_block);
  }

  for (int i = threadIdx.x; i < 4096; i += NT) {
    if (i <= 2048) {
#pragma unroll
      for (int t = 0; t < QT; ++t) hist[t][i] = 0u;
    }
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
      const int32_t id = p < nv ? prow[p] : -1;
      ptok[i] = (id >= 0 && id < ctx_b) ? id : -1;
    }
    __syncthreads();
  }

  // From here on the wave's range ends at the visible count.
  wend = wbase + tile / NW;
  if (wend > nv) wend = nv;
  wlast = wend - 1;
  if constexpr (BUF) krs = wave_rsrc(wend);
  if constexpr (F4 && BUF) srs = wave_srsrc(wend);

  // RT: the 16x16 results of a batch stay in registers, x[b][r][u] =
  // dot(MFMA row 16b + 4g + r, token 16u + c16); one 4x4 transpose across
  // the lane groups per (b, r) then leaves lane (g, c16) with every row of
  // token 16g + c16 = lane: x[b][r][s] = dot(row 16b + 4s + r, token lane).
  constexpr int NRB = F4 ? RB : HB;
  static_assert(!RT || SG == 4, "register transpose: four groups of 16 tokens per batch");
  auto score_batch = [&](const Frag<CH>(&f)[SG], int64_t it) {
    float x[RT ? NRB : 1][4][4];
    if constexpr (F4) {
#pragma unroll
      for (int u = 0; u < SG; ++u) {
        // E8M0 scale of this lane's 32 channels: byte g of key 16u + c16's row
        const uint32_t sw = (uint32_t)__shfl((int)f[0].w[4], 16 * u + c16, 64);
        const int sb = (int)((sw >> (8 * g)) & 0xFFu);
        const v8i bk = v8i{(int)f[u].w[0], (int)f[u].w[1], (int)f[u].w[2], (int)f[u].w[3], 0, 0, 0, 0};
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          v4f acc = {0.f, 0.f, 0.f, 0.f};
          acc = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa4[rb], bk, acc, 0 /* A E4M3 */, 4 /* B E2M1 */,
                                                                 0, 127, 0, sb);
#pragma unroll
          for (int r = 0; r < 4; ++r) x[rb][r][u] = acc[r];
        }
      }
    } else if constexpr (FULL) {
#pragma unroll
      for (int u = 0; u < 2 * SG; ++u) {
        const uint32_t* w4 = &f[u >> 1].w[4 * (u & 1)];
        const long lo = as_long(w4[0], w4[1]), hi = as_long(w4[2], w4[3]);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          v4f a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[rb][0][0], lo, a0, 0, 0, 0);
          a0 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[rb][0][1], hi, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[rb][1][0], lo, a1, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qh[rb][1][1], hi, a1, 0, 0, 0);
          // even column 2m: a0 here plus a1 of the odd column 2m+1 (lane + 1).
          // (__shfl_xor: the DPP builtins applied to elements of an MFMA
          // result were folded into a single element by this compiler.)
          v4f d;
#pragma unroll
          for (int r = 0; r < 4; ++r) d[r] = a0[r] + __shfl_xor(a1[r], 1, 64);
          // d[r] = dot(A row 16 rb + 4g + r, token 8u + m) on the even lanes;
          // the other lanes write their own trash slot (no branch around the
          // loads' waits)
          const bool keep = (c16 & 1) == 0 && 16 * rb + 4 * g < HP;
          const int at = keep ? (8 * u + (c16 >> 1)) * pitch + 16 * rb + 4 * g : 16 * SG * HP + 4 * lane;
          *reinterpret_cast<v4f*>(my + at) = d;
        }
      }
    } else {
#pragma unroll
      for (int su = 0; su < SG; ++su) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          v4f acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int i = 0; i < KS; ++i)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_fp8_fp8(qa[hb][i], as_long(f[su].w[2 * i], f[su].w[2 * i + 1]),
                                                             acc, 0, 0, 0);
          // acc[r] = dot(head 16*hb + 4*g + r, token 16*su + c16)
#pragma unroll
          for (int r = 0; r < 4; ++r) x[hb][r][su] = acc[r];
        }
      }
    }
    if constexpr (RT) {
#pragma unroll
      for (int rb = 0; rb < NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 4; ++r) transpose_lane_groups(x[rb][r]);
    } else {
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    }
#pragma unroll
    for (int u = 0; u < SG / 4; ++u) {
      // Lane owns token it + 64u + lane.
      const int64_t j = it + 64 * u + lane;
      bool vis_w = j < wend;
      if constexpr (GATHER) vis_w = vis_w && ptok[j < wend ? j - tile0 : 0] >= 0;
      const float* src = my + (64 * u + lane) * pitch;
      uint32_t key = 0u;
      bool vis = vis_w;
      constexpr int HPQ = QT > 1 ? 8 : HP;   // dots per query in a token's row
#pragma unroll
      for (int t = 0; t < QT; ++t) {
        if (t >= nq) break;   // (uniform)
        float sc = 0.0f;
        if constexpr (RT) {
#pragma unroll
          for (int hq = 0; hq < HPQ; ++hq) {
            // MFMA row of head hq of query t
            const int R = (QT > 1 ? 8 * t : 0) + hq;
            const float d = x[R >> 4][R & 3][(R >> 2) & 3];
            // heads past H_I have weight 0: adding +0 leaves the sum unchanged
            const float r = d > 0.0f ? d : 0.0f;
            sc = __fadd_rn(sc, __fmul_rn(wv[HPQ * t + hq], r));
          }
        } else {
#pragma unroll
          for (int h4 = 0; h4 < HPQ; h4 += 4) {
            const v4f d4 = *reinterpret_cast<const v4f*>(src + HPQ * t + h4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              float r = d4[e] > 0.0f ? d4[e] : 0.0f;
              sc = __fadd_rn(sc, __fmul_rn(wv[HPQ * t + h4 + e], r));
            }
          }
        }
        vis = vis_w && (QT == 1 || j < nvq[t]);
        // Positions up to the next multiple of 64 lie inside the row's key
        // stride and belong to no other wave; past the visible count they
        // are never read.
        key = vis ? score_key(sc) : 0u;
        if (kStage) kst[t * kTileCap + (j - tile0)] = key;
        else keys[row * key_stride + j] = key;
        atomicAdd(&hist[t][vis ? key >> 21 : 2048u], 1u << (16 * ((key >> 20) & 1u)));
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
    if constexpr (!RT) {
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
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
    // Whole 64-position groups: they stay inside the row's key stride (every
    // one of them was written by a wave; past a query's visible count they
    // hold key 0).
    const int64_t tn = tend > tile0 ? ((tend - tile0 + 63) & ~63LL) : 0;
#pragma unroll
    for (int t = 0; t < QT; ++t) {
      if (t >= nq) break;
      for (int64_t i = 4 * threadIdx.x; i < tn; i += 4 * NT)
        *reinterpret_cast<v4u*>(keys + (row + t) * key_stride + tile0 + i) =
            *reinterpret_cast<const v4u*>(&kst[t * kTileCap + i]);
    }
  }
  // Two adjacent bins per 64-bit atomic: the row histogram's 32-bit counters
  // 2i and 2i+1 are the low and high halves of one little-endian 64-bit word.
#pragma unroll
  for (int t = 0; t < QT; ++t) {
    if (t >= nq) break;
    if (tok.hist1) {
      uint64_t* gh = reinterpret_cast<uint64_t*>(tok.hist1 + (row + t) * 4096);
      for (int i = threadIdx.x; i < 2048; i += NT) {
        const uint32_t v = hist[t][i];
        if (v) atomic_add_agent64(gh + i, (uint64_t)(v & 0xFFFFu) | ((uint64_t)(v >> 16) << 32));
      }
    } else if (tok.tile_hist) {
      // The tile's histogram as it stands (two 16-bit bins per word), one
      // slot per tile: plain stores, nothing to clear beforehand.
      v4u* th = reinterpret_cast<v4u*>(tok.tile_hist + ((row + t) * tok.th_stride + blockIdx.x) * 2048);
      for (int i = threadIdx.x; i < 512; i += NT) th[i] = reinterpret_cast<const v4u*>(hist[t])[i];
    }
  }
  if (pool) {
    uint64_t* gbh = reinterpret_cast<uint64_t*>(blk.hist1 + row * 4096);
    for (int i = threadIdx.x; i < 2048; i += NT) {
      const uint32_t lo = bhist[2 * i], hi = bhist[2 * i + 1];
      if (lo | hi) atomic_add_agent64(gbh + i, (uint64_t)lo | ((uint64_t)hi << 32));
    }
  }
}

// Flat-scan tile: 1024 tokens per wave, halved while the grid would leave
// compute units without a workgroup (down to kScanTileSmall).
// (`rows` counts workgroup rows: query rows, or groups of them)
static int scan_tile(int64_t rows, int64_t n_max, int nw, int qt = 1) {
  (void)qt;
  int tile = 1024 * nw;
  while (tile > kScanTileSmall && rows * ((n_max + tile - 1) / tile) < device_cu_count()) tile >>= 1;
  return tile;
}

// Query rows per scan workgroup: 2..15 query rows of one sequence (multi-
// query decode; 16 or more take the dense prefill product) share one pass
// over the key rows when D_I = 128 and there are at most 8 indexer heads
// (two queries fill one 16-row MFMA block).
static int scan_qt(const ScoreArgs& a) {
  if (a.pool_block > 0 || a.D_I != 128 || a.H_I > 8 || a.Tq < 2) return 1;
  return a.Tq == 2 ? 2 : 4;
}

template <int QT, bool F4>
static hipError_t launch_scan_mq(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                 const SelectWs& tok, hipStream_t s) {
  constexpr int NW = kScanWavesT<false, 1, QT, F4>;
  const int64_t groups = (int64_t)a.B * ((a.Tq + QT - 1) / QT);
  const int tile = scan_tile(groups, a.n_max, NW, QT);
  int64_t tiles = (a.n_max + tile - 1) / tile;
  if (tiles < 1) tiles = 1;
  CSA2_LAUNCH("index_score", (index_score_kernel<128, 1, false, false, true, QT, F4>),
              dim3((unsigned)tiles, (unsigned)groups), dim3(64 * NW), 0, s, a.q_idx, a.w, a.k_idx, a.k_bstride,
              a.k_rstride, a.k_scales, a.ks_bstride, a.ks_rstride, a.ctx_len, a.q_pos,
              (const int32_t*)nullptr, (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys,
              key_stride, n_valid, tok, 0, 0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, tok);
  return hipGetLastError();
}

template <int DI, int HB, bool H8, bool F4 = false>
static hipError_t launch_scan_t(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                const SelectWs& tok, uint32_t* bkeys, int64_t bkey_stride, int32_t* nb_valid,
                                const SelectWs* blk, hipStream_t s) {
  int64_t rows = (int64_t)a.B * a.Tq;
  constexpr int NW = kScanWavesT<false, HB, 1, F4>;
  const int tile = scan_tile(rows, a.n_max, NW);
  int64_t tiles = (a.n_max + tile - 1) / tile;
  if (tiles < 1) tiles = 1;
  SelectWs bw = blk ? *blk : tok;
  dim3 grid((unsigned)tiles, (unsigned)rows);
  if (a.pool_block > 0) {
    CSA2_LAUNCH("index_score", (index_score_kernel<DI, HB, false, true, H8, 1, F4>), grid, dim3(64 * NW), 0, s,
                a.q_idx, a.w, a.k_idx, a.k_bstride, a.k_rstride, a.k_scales, a.ks_bstride, a.ks_rstride, a.ctx_len,
                a.q_pos, (const int32_t*)nullptr,
                (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys, key_stride, n_valid, tok,
                a.pool_block, a.pool_nblocks, bkeys, bkey_stride, nb_valid, bw);
  } else {
    CSA2_LAUNCH("index_score", (index_score_kernel<DI, HB, false, false, H8, 1, F4>), grid, dim3(64 * NW), 0, s,
                a.q_idx, a.w, a.k_idx, a.k_bstride, a.k_rstride, a.k_scales, a.ks_bstride, a.ks_rstride, a.ctx_len,
                a.q_pos, (const int32_t*)nullptr,
                (const int32_t*)nullptr, 0, a.Tq, a.H_I, a.n_max, a.k_top, tile, keys, key_stride, n_valid, tok, 0,
                0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, bw);
  }
  return hipGetLastError();
}

template <int DI, int HB, bool H8, bool F4 = false>
static hipError_t launch_pool_t(const ScoreArgs& a, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                                uint32_t* keys, int64_t key_stride, int32_t* n_valid, const SelectWs& ws,
                                hipStream_t s) {
  int64_t rows = (int64_t)a.B * a.Tq;
  int64_t tiles = (pool_cap + kPoolTile - 1) / kPoolTile;
  if (tiles < 1) tiles = 1;
  CSA2_LAUNCH("pool_score", (index_score_kernel<DI, HB, true, false, H8, 1, F4>),
              dim3((unsigned)tiles, (unsigned)rows), dim3(64 * kScanWavesT<true, HB, 1, F4>), 0, s, a.q_idx, a.w, a.k_idx,
              a.k_bstride, a.k_rstride, a.k_scales, a.ks_bstride, a.ks_rstride, a.ctx_len, (const int32_t*)nullptr,
              pool_idx, pool_len, pool_cap, a.Tq, a.H_I, (int64_t)pool_cap, a.k_top, kPoolTile, keys, key_stride,
              n_valid, ws, 0, 0, (uint32_t*)nullptr, (int64_t)0, (int32_t*)nullptr, ws);
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

// Per-row state of a prefill selection pass (see PfRow), in registers: the
// keys emitted now form the range [e_lo, e_hi] (empty: e_lo > e_hi), the
// undecided bucket [b_lo, b_hi] (empty when the pass takes it whole).
struct PfLane {
  uint32_t mode, n_ps, n_pfx, e_lo, e_hi, b_lo, b_hi;
};
__device__ __forceinline__ PfLane pf_load(const PfArgs& pf, int64_t grow, bool ok) {
  PfLane L{PF_DONE, 32u, 0u, 1u, 0u, 1u, 0u};   // (empty ranges)
  if (ok && pf.rows[grow - pf.row_base].mode == PF_GUESS) {
    // the guessed window: candidates in [g_cand, g_emit), emitted above
    const PfRow& r = pf.rows[grow - pf.row_base];
    L.mode = PF_CAND;
    if (!r.g_emit_none) {
      L.e_lo = r.g_emit;
      L.e_hi = 0xFFFFFFFFu;
    }
    const uint32_t chi = r.g_emit_none ? 0xFFFFFFFFu : r.g_emit - 1u;
    if (r.g_emit_none || r.g_emit > r.g_cand) {
      L.b_lo = r.g_cand;
      L.b_hi = chi;
    }
  } else if (ok && pf.rows[grow - pf.row_base].mode != PF_DONE) {
    const PfRow& r = pf.rows[grow - pf.row_base];
    L.mode = r.mode;
    L.n_ps = r.n_ps;
    L.n_pfx = r.n_pfx;
    // bucket: keys with key >> n_ps == n_pfx
    const uint64_t blo = r.n_ps >= 32u ? 0ull : (uint64_t)r.n_pfx << r.n_ps;
    const uint64_t bhi = r.n_ps >= 32u ? 0xFFFFFFFFull : blo + (1ull << r.n_ps) - 1ull;
    if (!r.e_incl) {
      L.b_lo = (uint32_t)blo;
      L.b_hi = (uint32_t)bhi;
    }
    if (r.e_on && r.n_ps < 32u) {
      // above the bucket (or from its start when it is taken whole), inside
      // the previous bucket
      const uint64_t plo = r.e_incl ? blo : bhi + 1ull;
      const uint64_t phi = r.e_ps >= 32u ? 0xFFFFFFFFull : ((uint64_t)r.e_pfx << r.e_ps) + (1ull << r.e_ps) - 1ull;
      if (plo <= phi) {
        L.e_lo = (uint32_t)plo;
        L.e_hi = (uint32_t)phi;
      }
    }
  }
  return L;
}
// 1: selected for certain (emit now); 2: in the undecided bucket; 0: neither.
__device__ __forceinline__ int pf_class(const PfLane& L, uint32_t k) {
  return (k >= L.e_lo && k <= L.e_hi) ? 1 : ((k >= L.b_lo && k <= L.b_hi) ? 2 : 0);
}
// The next radix digit of a key inside the bucket of n_ps: bits 31..20,
// 19..8, then 7..0.
__device__ __forceinline__ uint32_t pf_digit(uint32_t k, uint32_t n_ps) {
  return n_ps >= 32u ? k >> 20 : (n_ps == 20u ? (k >> 8) & 0xFFFu : k & 0xFFu);
}
__device__ __forceinline__ void pf_emit(const PfArgs& pf, int64_t grow, int64_t j, uint32_t k) {
  const uint32_t slot = atomicAdd(&pf.rows[grow - pf.row_base].out_cnt, 1u);
  if (slot < (uint32_t)pf.k_top) {   // (never false: the counts are exact)
    pf.out_idx[grow * pf.k_top + slot] = (int32_t)j;
    if (pf.out_key) pf.out_key[grow * pf.k_top + slot] = k;
  }
}
__device__ __forceinline__ void pf_cand(const PfArgs& pf, int64_t grow, int64_t j, uint32_t k) {
  const int64_t lrow = grow - pf.row_base;
  const uint32_t slot = atomicAdd(&pf.rows[lrow].cand_cnt, 1u);
  if (slot < (uint32_t)kPfCap) pf.cand[lrow * kPfCap + slot] = ((uint64_t)k << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)j);
}
// Selection passes (PFM 2) stage emitted positions and candidates of a
// workgroup in LDS (in the histogram's space, when no row of the tile
// histograms) and reserve their slots with one global atomic per row and
// kind at the end: a global atomic per key kept its wave waiting for the
// returned slot.  kPfStage entries of (position, key) per row and kind;
// beyond them a key takes its slot directly.
constexpr int kPfStage = 512;
template <int QW>
__device__ __forceinline__ void pf_stage(const PfArgs& pf, uint32_t* stg, uint32_t* scnt, int kind, int ql,
                                         int64_t grow, int64_t j, uint32_t k) {
  const uint32_t sl = atomicAdd(&scnt[kind * QW + ql], 1u);
  if (sl < (uint32_t)kPfStage) {
    uint32_t* e = stg + ((ql * 2 + kind) * kPfStage + sl) * 2;
    e[0] = (uint32_t)j;
    e[1] = k;
  } else if (kind == 0) {
    pf_emit(pf, grow, j, k);
  } else {
    pf_cand(pf, grow, j, k);
  }
}
// The transposed product's passes stage per lane instead (no atomics on the
// key loop): entry i of kind `kind` of workgroup thread tl sits at word
// ((kind * kPfLane + i) * threads + tl) * 2, its counts stay in registers,
// and the end of the workgroup reserves one global range per row and kind.
constexpr int kPfLane = 8;
// Beyond a lane's kPfLane entries: a shared pool of kPfPool entries
// (position, key, kind << 4 | row) in LDS; beyond the pool the workgroup
// sets `spill` and scores its tile again with direct global slots.  Nothing
// in the key loop then touches global memory (a global atomic there made
// the compiler drain the key loads in flight).
constexpr int kPfPool = 4096;
__device__ __forceinline__ void pf_lane_put2(uint32_t* stg, uint32_t* pool, uint32_t* pool_cnt, uint32_t* spill,
                                             int kind, int ql, uint32_t& cnt, int64_t j, uint32_t k) {
  if (cnt < (uint32_t)kPfLane) {
    // consecutive lanes at consecutive entries (no bank conflicts)
    uint32_t* e = stg + ((kind * kPfLane + cnt) * (64 * kPrefillWaves) + threadIdx.x) * 2;
    e[0] = (uint32_t)j;
    e[1] = k;
  } else {
    const uint32_t ps = atomicAdd(pool_cnt, 1u);
    if (ps < (uint32_t)kPfPool) {
      pool[3 * ps] = (uint32_t)j;
      pool[3 * ps + 1] = k;
      pool[3 * ps + 2] = ((uint32_t)kind << 4) | (uint32_t)ql;
    } else {
      *spill = 1u;
    }
  }
  ++cnt;
}
// stg: 2*kPfLane*NWV*64*2 words, then 2*NWV*64 count words and 2*NWV*64
// offset words.  Lane (c16, g) of every wave holds row ql = c16.
template <int QW, int NWV>
__device__ void pf_lane_flush(const PfArgs& pf, uint32_t* stg, uint32_t ne, uint32_t nc, uint32_t* sbase,
                              int64_t row0, int Tq, int t0) {
  constexpr int NL = NWV * 64;
  uint32_t* cnts = stg + NL * 2 * kPfLane * 2;   // [kind][lane of the workgroup]
  uint32_t* offs = cnts + 2 * NL;
  const int tl = threadIdx.x;
  cnts[tl] = ne < (uint32_t)kPfLane ? ne : (uint32_t)kPfLane;
  cnts[NL + tl] = nc < (uint32_t)kPfLane ? nc : (uint32_t)kPfLane;
  __syncthreads();
  if (tl < 2 * QW) {
    const int kind = tl / QW, ql = tl % QW;
    uint32_t run = 0;
    for (int wv = 0; wv < NWV; ++wv)
      for (int gg = 0; gg < 4; ++gg) {
        const int l = wv * 64 + gg * 16 + ql;
        offs[kind * NL + l] = run;
        run += cnts[kind * NL + l];
      }
    uint32_t base = 0;
    if (run && t0 + ql < Tq) {
      PfRow& r = pf.rows[row0 + ql - pf.row_base];
      base = atomicAdd(kind ? &r.cand_cnt : &r.out_cnt, run);
    }
    sbase[kind * QW + ql] = base;
  }
  __syncthreads();
  const int ql = tl & 15;
  if (t0 + ql >= Tq) return;
  const int64_t grow = row0 + ql;
#pragma unroll
  for (int kind = 0; kind < 2; ++kind) {
    const uint32_t n = cnts[kind * NL + tl];
    const uint32_t b0 = sbase[kind * QW + ql] + offs[kind * NL + tl];
    for (uint32_t i = 0; i < n; ++i) {
      const uint32_t* v = stg + ((kind * kPfLane + i) * NL + tl) * 2;
      const uint32_t slot = b0 + i;
      if (kind == 0) {
        if (slot < (uint32_t)pf.k_top) {
          pf.out_idx[grow * pf.k_top + slot] = (int32_t)v[0];
          if (pf.out_key) pf.out_key[grow * pf.k_top + slot] = v[1];
        }
      } else if (slot < (uint32_t)kPfCap) {
        pf.cand[(grow - pf.row_base) * kPfCap + slot] = ((uint64_t)v[1] << 32) | (uint64_t)(0xFFFFFFFFu - v[0]);
      }
    }
  }
}

template <int QW, int NT>
__device__ void pf_unstage(const PfArgs& pf, const uint32_t* stg, const uint32_t* scnt, uint32_t* sbase, int64_t row0,
                           int Tq, int t0) {
  if (threadIdx.x < 2 * QW) {
    const int kind = threadIdx.x / QW, ql = threadIdx.x % QW;
    uint32_t n = scnt[kind * QW + ql];
    n = n < (uint32_t)kPfStage ? n : (uint32_t)kPfStage;
    uint32_t base = 0;
    if (n && t0 + ql < Tq) {
      PfRow& r = pf.rows[row0 + ql - pf.row_base];
      base = atomicAdd(kind ? &r.cand_cnt : &r.out_cnt, n);
    }
    sbase[kind * QW + ql] = base;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < 2 * QW * kPfStage; i += NT) {
    const int kind = i / (QW * kPfStage), rem = i % (QW * kPfStage), ql = rem / kPfStage, e = rem % kPfStage;
    uint32_t n = scnt[kind * QW + ql];
    n = n < (uint32_t)kPfStage ? n : (uint32_t)kPfStage;
    if ((uint32_t)e >= n || t0 + ql >= Tq) continue;
    const uint32_t* v = stg + ((ql * 2 + kind) * kPfStage + e) * 2;
    const uint32_t slot = sbase[kind * QW + ql] + e;
    const int64_t grow = row0 + ql;
    if (kind == 0) {
      if (slot < (uint32_t)pf.k_top) {
        pf.out_idx[grow * pf.k_top + slot] = (int32_t)v[0];
        if (pf.out_key) pf.out_key[grow * pf.k_top + slot] = v[1];
      }
    } else if (slot < (uint32_t)kPfCap) {
      pf.cand[(grow - pf.row_base) * kPfCap + slot] = ((uint64_t)v[1] << 32) | (uint64_t)(0xFFFFFFFFu - v[0]);
    }
  }
}
// Pass 0 of the selection (PFM 1) scores a sample of a tile's 16-key chunks:
// chunk kPfSample*m + m % kPfSample for m = 0, 1, ... (every part of the
// tile, and every offset within kPfSample chunks, represented).
static_assert((kPfSample & (kPfSample - 1)) == 0, "power of two");
template <int PFM>
__device__ __forceinline__ int pf_chunk(int m) {
  return PFM == 1 ? kPfSample * m + (m & (kPfSample - 1)) : m;
}
template <int PFM>
__device__ __forceinline__ int pf_nloop(int nchunks) {
  return PFM == 1 ? (nchunks + kPfSample - 1) / kPfSample : nchunks;
}
// The row's histogram range in a sample pass: (h_base, h_shift), see PfRow.
__device__ __forceinline__ void pf_sample_range(const PfArgs& pf, int64_t grow, bool ok, uint32_t& base,
                                                uint32_t& shift) {
  base = 0xFFFFFFFFu;   // (rows outside the sample: nothing counted)
  shift = 31u;
  if (ok) {
    const PfRow& r = pf.rows[grow - pf.row_base];
    if (r.sampled != 0u) {
      base = r.h_base;
      shift = r.h_shift;
    }
  }
}
// Sample-pass bin of a key (-1: below the range; the last bin takes every
// key above it).
__device__ __forceinline__ int pf_sbin(uint32_t key, uint32_t base, uint32_t shift) {
  if (key < base) return -1;
  const uint32_t d = (key - base) >> shift;
  return d > 4095u ? 4095 : (int)d;
}
// Histogram pass (PFM 1: every row of the block histograms the top 12 bits
// of its sampled visible keys): the tile's LDS histogram into the rows'.
template <int QW, int NT>
__device__ void pf_flush_hist(const PfArgs& pf, const uint32_t* hist, int64_t row0, int Tq, int t0) {
  for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) {
    const uint32_t v = hist[i];
    if (!v) continue;
    const int p = i >> 12, bin = i & 4095;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const int ql = 2 * p + hf;
      const uint32_t c = hf ? v >> 16 : v & 0xFFFFu;
      if (c && t0 + ql < Tq) atomic_add_agent(pf.hist + (row0 + ql - pf.row_base) * 4096 + bin, c);
    }
  }
}

// End of a pass workgroup: histogram counts and tie counts to global memory,
// tie emission in position order.  hist holds (QW/2) x 4096 words (two
// queries per word) or, for tie emission, nchunks x QW masks of 16 bits.
template <int QW, int NT>
__device__ void pf_finish(const PfArgs& pf, const PfLane* pfl, uint32_t flags, const uint32_t* hist,
                          const uint32_t* tcnt, int64_t row0, int Tq, int t0, int kx, int64_t k0, int nchunks) {
  if (flags & (1u << PF_HIST)) {
    for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) {
      const uint32_t v = hist[i];
      if (!v) continue;
      const int p = i >> 12, bin = i & 4095;
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int ql = 2 * p + hf;
        const uint32_t c = hf ? v >> 16 : v & 0xFFFFu;
        if (c && pfl[ql].mode == PF_HIST) atomic_add_agent(pf.hist + (row0 + ql - pf.row_base) * 4096 + bin, c);
      }
    }
  }
  if (threadIdx.x < QW && t0 + (int)threadIdx.x < Tq) {
    const int ql = threadIdx.x;
    const int64_t lrow = row0 + ql - pf.row_base;
    if (pfl[ql].mode == PF_TIECOUNT && tcnt[ql]) atomic_add_agent(pf.hist + lrow * 4096 + kx, tcnt[ql]);
    if (pfl[ql].mode == PF_TIEEMIT) {
      // ties of earlier key tiles (exclusive prefix by the step kernel)
      const uint32_t base = pf.hist[lrow * 4096 + kx];
      const uint32_t need = pf.rows[lrow].need;
      uint32_t cnt = 0;
      for (int c = 0; c < nchunks && base + cnt < need; ++c) {
        uint32_t m = hist[c * QW + ql];
        while (m && base + cnt < need) {
          const int bit = __builtin_ctz(m);
          m &= m - 1u;
          pf_emit(pf, row0 + ql, k0 + 16 * (int64_t)c + bit, pfl[ql].n_pfx);   // (the tie key T)
          ++cnt;
        }
      }
    }
  }
}

// (key tile, query tile) of a prefill workgroup.  XO: workgroups are dealt
// round-robin over the 8 XCDs in launch order (workgroup i on XCD i mod 8),
// and each XCD is given a contiguous run of the pairs, query tile fastest, so
// that the workgroups resident on one XCD at a time score the same key tile
// for different queries and find it in that XCD's L2.  Measured: the
// four-query tiles of wide indexers (which read every key again for each
// four queries) gain from it on their full passes; the sixteen-query tiles
// of the transposed product and the sample passes (few, long key tiles,
// whose short last tile then falls to one XCD) ran slower, and keep the
// launch order (key tile fastest).
template <bool XO>
__device__ __forceinline__ void prefill_tile(int& kx, int64_t& qy) {
  if constexpr (!XO) {
    kx = blockIdx.x;
    qy = blockIdx.y;
  } else {
    const uint32_t ny = gridDim.y, nwg = gridDim.x * ny;   // (< 2^28: at most 4096 x 65535)
    const uint32_t lin = blockIdx.x + gridDim.x * blockIdx.y;
    const uint32_t x = lin & 7u, per = nwg >> 3, rem = nwg & 7u;
    const uint32_t pr = x * per + (x < rem ? x : rem) + (lin >> 3);
    kx = (int)(pr / ny);
    qy = pr - (uint32_t)kx * ny;
  }
}

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

// F4: MXFP4 keys as the B operand, as in the decode scan: lane (key c16,
// group g) takes bytes 16g .. 16g+15 of the key's code row (channels 32g ..
// 32g+31) and scale byte g; the E4M3 query fragments keep their pairing.
template <int DI, int HG, int QG, int PFM, bool F4>
__global__ void __launch_bounds__(64 * kPrefillWaves)
index_prefill_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                     const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                     const uint8_t* __restrict__ k_scales, int64_t ks_bstride, int64_t ks_rstride,
                     const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                     int Tq, int H_I, int64_t n_max, int key_tile, int qtiles,
                     uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                     SelectWs tok, PfArgs pf, int64_t y0) {
  static_assert(!F4 || DI == 128, "MXFP4 keys: 128 channels");
  constexpr int KS = DI / 128;          // MFMA k-steps
  constexpr int FW = DI / 16;           // fragment words per lane
  constexpr int QW = 4 * QG;            // queries per workgroup
  constexpr int HP = 4 * HG;            // heads incl. padding
  constexpr int NT = 64 * kPrefillWaves;
  typedef int v8i __attribute__((ext_vector_type(8)));
  constexpr bool PF = PFM == 2;
  __shared__ uint32_t hist[(QW / 2) * 4096];
  __shared__ int32_t nvs[QW];
  __shared__ uint32_t shb[PFM == 1 ? QW : 1], shs[PFM == 1 ? QW : 1];   // sample passes: bin ranges
  __shared__ PfLane pfl[PF ? QW : 1];
  __shared__ uint32_t tcnt[PF ? QW : 1];
  __shared__ uint32_t scnt[PF ? 2 * QW : 1], sbase[PF ? 2 * QW : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  if constexpr (PF) {
    if (pf.active[pf.pass - 1] == 0u) return;   // (uniform: every row of the block done)
  }
  int kx;
  int64_t qy;
  prefill_tile<PFM != 1 && QG == 1>(kx, qy);
  const int64_t yy = qy + y0;
  const int64_t b = yy / qtiles;
  const int t0 = (int)(yy % qtiles) * QW;
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
      if (kx == 0) n_valid_out[row0 + threadIdx.x] = (int32_t)nv;
    }
    nvs[threadIdx.x] = (int32_t)nv;
    if constexpr (PFM == 1) pf_sample_range(pf, row0 + threadIdx.x, t < Tq, shb[threadIdx.x], shs[threadIdx.x]);
    if constexpr (PF) {
      pfl[threadIdx.x] = pf_load(pf, row0 + threadIdx.x, t < Tq);
      tcnt[threadIdx.x] = 0u;
      scnt[threadIdx.x] = 0u;
      scnt[QW + threadIdx.x] = 0u;
    }
  }
  uint32_t flags = 0;   // PF: bit m set when some row of the tile is in mode m
  bool stage = false;   // PF: emitted keys and candidates staged in LDS
  if constexpr (PF) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < QW; ++i) flags |= 1u << pfl[i].mode;
    if (!(flags & ~1u)) return;   // uniform: every row done
    stage = !(flags & ((1u << PF_HIST) | (1u << PF_TIEEMIT)));
    if (!stage)
      for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) hist[i] = 0u;
  } else {
    for (int i = threadIdx.x; i < (QW / 2) * 4096; i += NT) hist[i] = 0u;
  }
  __syncthreads();
  int max_nv = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) max_nv = nvs[i] > max_nv ? nvs[i] : max_nv;
  const int64_t k0 = (int64_t)kx * key_tile;
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
    krow[qg] = PFM ? nullptr : keys + (row0 + ql) * key_stride;
  }

  const uint8_t* kb = k_idx + b * k_bstride;
  const uint8_t* ksb = F4 ? k_scales + b * ks_bstride : nullptr;
  const int nchunks = (int)((k1 - k0 + 15) >> 4);
  uint32_t fa[FW], fb[FW];
  auto load_chunk = [&](uint32_t (&f)[FW], int c) {
    const int64_t j = k0 + 16 * (int64_t)c + c16;
    if constexpr (F4) {
      // (keys past the tile read its first row: their scores are masked)
      const int64_t jj = j < k1 ? j : k0;
      const v4u v = *reinterpret_cast<const v4u*>(kb + jj * k_rstride + 16 * g);
      f[0] = v[0]; f[1] = v[1]; f[2] = v[2]; f[3] = v[3];
      f[4] = ksb[jj * ks_rstride + g];   // the E8M0 scale of this lane's 32 channels
    } else {
      load_k128<DI>(f, kb + (j < k1 ? j : k0) * k_rstride, g, j < k1);
    }
  };
  auto score_chunk = [&](const uint32_t (&f)[FW], int c) {
    const int64_t j = k0 + 16 * (int64_t)c + c16;
    v8i kf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = F4 ? v8i{(int)f[0], (int)f[1], (int)f[2], (int)f[3], 0, 0, 0, 0}
                  : v8i{(int)f[8 * ks], (int)f[8 * ks + 1], (int)f[8 * ks + 2], (int)f[8 * ks + 3],
                        (int)f[8 * ks + 4], (int)f[8 * ks + 5], (int)f[8 * ks + 6], (int)f[8 * ks + 7]};
#pragma unroll
    for (int qg = 0; qg < QG; ++qg) {
      v4f acc[HG];
#pragma unroll
      for (int hg = 0; hg < HG; ++hg) {
        acc[hg] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if constexpr (F4)
            acc[hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[qg][hg][ks], kf[ks], acc[hg], 0 /* A E4M3 */,
                                                                       4 /* B E2M1 */, 0, 127, 0, (int)f[4]);
          else
            acc[hg] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(qa[qg][hg][ks], kf[ks], acc[hg], 0, 0, 0, 127,
                                                                       0, 127);
        }
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
        const int ql = 4 * qg + g;
        if constexpr (PF) {
          const PfLane pl = pfl[ql];
          {
            const int cls = pf_class(pl, key);
            if (cls == 1) {
              if (stage) pf_stage<QW>(pf, hist, scnt, 0, ql, row0 + ql, j, key);
              else pf_emit(pf, row0 + ql, j, key);
            } else if (cls == 2) {
              if (pl.mode == PF_HIST) atomicAdd(&hist[(ql >> 1) * 4096 + pf_digit(key, pl.n_ps)], 1u << (16 * (ql & 1)));
              else if (pl.mode == PF_CAND) {
                if (stage) pf_stage<QW>(pf, hist, scnt, 1, ql, row0 + ql, j, key);
                else pf_cand(pf, row0 + ql, j, key);
              } else if (pl.mode == PF_TIECOUNT) atomicAdd(&tcnt[ql], 1u);
              else if (pl.mode == PF_TIEEMIT) atomicOr(&hist[c * QW + ql], 1u << c16);
            }
          }
        } else if constexpr (PFM == 1) {
          const int bin = pf_sbin(key, shb[ql], shs[ql]);
          if (bin >= 0) atomicAdd(&hist[(ql >> 1) * 4096 + bin], 1u << (16 * (ql & 1)));
        } else {
          __builtin_nontemporal_store(key, krow[qg] + j);
          atomicAdd(&hist[(ql >> 1) * 4096 + (key >> 20)], 1u << (16 * (ql & 1)));
        }
      }
    }
  };
  const int nloop = pf_nloop<PFM>(nchunks);
  auto live = [&](int m) { return m < nloop && pf_chunk<PFM>(m) < nchunks; };
  int c = wave;
  if (live(c)) load_chunk(fa, pf_chunk<PFM>(c));
  for (; c < nloop; c += 2 * kPrefillWaves) {
    const int cb = c + kPrefillWaves;
    if (live(cb)) load_chunk(fb, pf_chunk<PFM>(cb));
    if (live(c)) score_chunk(fa, pf_chunk<PFM>(c));
    if (live(cb + kPrefillWaves)) load_chunk(fa, pf_chunk<PFM>(cb + kPrefillWaves));
    if (live(cb)) score_chunk(fb, pf_chunk<PFM>(cb));
  }
  __syncthreads();
  if constexpr (PF) {
    // (staging excludes histogram and tie-emission rows; tie counts are
    // flushed either way)
    if (stage) pf_unstage<QW, NT>(pf, hist, scnt, sbase, row0, Tq, t0);
    pf_finish<QW, NT>(pf, pfl, flags, hist, tcnt, row0, Tq, t0, kx, k0, nchunks);
    return;
  }
  if constexpr (PFM == 1) {
    pf_flush_hist<QW, NT>(pf, hist, row0, Tq, t0);
    return;
  }
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
// leave in a single 16-byte store.  F4: MXFP4 keys (E2M1 codes + E8M0 per 32
// channels) as the A operand: lane (c16, g) holds bytes 16g .. 16g+15 of key
// c16's code row (channels 32g .. 32g+31) and passes that block's scale byte.
// PFM: 0 = score keys stored for the radix select; 1 = the level-1
// histogram pass of the prefill selection (no keys stored); 2 = a later
// selection pass steered by each row's PfRow; query tiles from y0 on.
template <int PD, bool F4, int PFM>
__global__ void __launch_bounds__(64 * kPrefillWaves)
index_prefill_kt_kernel(const uint8_t* __restrict__ q_idx, const float* __restrict__ w,
                        const uint8_t* __restrict__ k_idx, int64_t k_bstride, int64_t k_rstride,
                        const uint8_t* __restrict__ k_scales, int64_t ks_bstride, int64_t ks_rstride,
                        const int32_t* __restrict__ ctx_len, const int32_t* __restrict__ q_pos,
                        int Tq, int H_I, int64_t n_max, int key_tile, int qtiles,
                        uint32_t* __restrict__ keys, int64_t key_stride, int32_t* __restrict__ n_valid_out,
                        SelectWs tok, PfArgs pf, int64_t y0) {
  constexpr int DI = 128, FW = 8, QW = 16, HP = 8;
  constexpr int NT = 64 * kPrefillWaves;
  constexpr bool PF = PFM == 2;
  __shared__ uint32_t hist[(QW / 2) * 4096 + 1];   // last word: bin of invisible keys
  __shared__ int32_t nvs[QW];
  __shared__ uint32_t shb[PFM == 1 ? QW : 1], shs[PFM == 1 ? QW : 1];   // sample passes: bin ranges
  __shared__ PfLane pfl[PF ? QW : 1];
  __shared__ uint32_t tcnt[PF ? QW : 1];
  __shared__ uint32_t scnt[PF ? 2 * QW : 1], sbase[PF ? 2 * QW : 1];
  __shared__ uint32_t pool_cnt, spill;
  // staged entries of the selection passes: per lane, then the pool
  constexpr int kPoolOff = kPrefillWaves * 64 * 2 * kPfLane * 2 + 4 * kPrefillWaves * 64;
  static_assert(kPoolOff + 3 * kPfPool <= (QW / 2) * 4096, "staging fits the histogram space");

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  if constexpr (PF) {
    if (pf.active[pf.pass - 1] == 0u) return;   // (uniform: every row of the block done)
  }
  int kx;
  int64_t qy;
  prefill_tile<false>(kx, qy);
  const int64_t yy = qy + y0;
  const int64_t b = yy / qtiles;
  const int t0 = (int)(yy % qtiles) * QW;
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
      if (kx == 0) n_valid_out[row0 + threadIdx.x] = (int32_t)nv;
    }
    nvs[threadIdx.x] = (int32_t)nv;
    if constexpr (PFM == 1) pf_sample_range(pf, row0 + threadIdx.x, t < Tq, shb[threadIdx.x], shs[threadIdx.x]);
    if constexpr (PF) {
      pfl[threadIdx.x] = pf_load(pf, row0 + threadIdx.x, t < Tq);
      tcnt[threadIdx.x] = 0u;
      scnt[threadIdx.x] = 0u;
      scnt[QW + threadIdx.x] = 0u;
      if (threadIdx.x == 0) {
        pool_cnt = 0u;
        spill = 0u;
      }
    }
  }
  uint32_t flags = 0;   // PF: bit m set when some row of the tile is in mode m
  bool stage = false;   // PF: emitted keys and candidates staged in LDS
  if constexpr (PF) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < QW; ++i) flags |= 1u << pfl[i].mode;
    if (!(flags & ~1u)) return;   // uniform: every row done
    stage = !(flags & ((1u << PF_HIST) | (1u << PF_TIEEMIT)));
    if (!stage)
      for (int i = threadIdx.x; i <= (QW / 2) * 4096; i += NT) hist[i] = 0u;
  } else {
    for (int i = threadIdx.x; i <= (QW / 2) * 4096; i += NT) hist[i] = 0u;
  }
  __syncthreads();
  int max_nv = 0;
#pragma unroll
  for (int i = 0; i < QW; ++i) max_nv = nvs[i] > max_nv ? nvs[i] : max_nv;
  const int64_t k0 = (int64_t)kx * key_tile;
  int64_t k1 = k0 + key_tile;
  if (k1 > max_nv) k1 = max_nv;
  if (k0 >= k1) return;   // uniform: nothing visible in this tile
  PfLane pl{};
  if constexpr (PF) pl = pfl[c16];
  uint32_t s_lo = 0u, s_sh = 20u;   // sample passes: this lane's bin range
  if constexpr (PFM == 1) {
    s_lo = shb[c16];
    s_sh = shs[c16];
  }
  uint32_t lane_ne = 0u, lane_nc = 0u;   // PF: entries this lane staged (emits, candidates)

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
  uint32_t* krow = PFM ? nullptr : keys + (row0 + c16) * key_stride;
  const uint32_t hbase = (uint32_t)(c16 >> 1) * 4096u, add = 1u << (16 * (c16 & 1));
  constexpr uint32_t kTrash = (QW / 2) * 4096;

  // Positions fit in 32 bits (n_max <= 2^22).  Every load is issued
  // unconditionally from a clamped in-range row so that the compiler can
  // count the loads in flight instead of draining them all at each chunk.
  const int ik0 = (int)k0, ik1 = (int)k1;
  const uint8_t* kb = k_idx + b * k_bstride;
  const uint8_t* ksb = F4 ? k_scales + b * ks_bstride : nullptr;
  const int nchunks = (ik1 - ik0 + 15) >> 4;
  uint32_t fk[PD][FW];
  auto load_at = [&](uint32_t (&f)[FW], const uint8_t* p, const uint8_t* ps) {
    const v4u lo = *reinterpret_cast<const v4u*>(p);
    f[0] = lo[0]; f[1] = lo[1]; f[2] = lo[2]; f[3] = lo[3];
    if constexpr (F4) {
      f[4] = *ps;   // the E8M0 scale of this lane's 32 channels
    } else {
      const v4u hi = *reinterpret_cast<const v4u*>(p + 64);
      f[4] = hi[0]; f[5] = hi[1]; f[6] = hi[2]; f[7] = hi[3];
    }
  };
  // A chunk wholly inside the tile: this lane's row address plus the chunk's
  // offset, computed once per wave in scalar registers (the 64-bit vector
  // multiply per chunk cost about 6% of the pass); the tile's last chunk and
  // those past it read clamped rows.
  const uint8_t* lane_k = kb + (int64_t)(ik0 + c16) * k_rstride + 16 * g;
  const uint8_t* lane_s = F4 ? ksb + (int64_t)(ik0 + c16) * ks_rstride + g : nullptr;
  auto load_chunk = [&](uint32_t (&f)[FW], int c) {
    const int cu = __builtin_amdgcn_readfirstlane(c);
    if (16 * cu + 16 <= ik1 - ik0) {
      const int64_t r = 16 * (int64_t)cu;
      load_at(f, lane_k + r * k_rstride, F4 ? lane_s + r * ks_rstride : nullptr);
    } else {
      int j = ik0 + 16 * cu + c16;
      j = j < ik1 ? j : ik1 - 1;
      load_at(f, kb + (int64_t)j * k_rstride + 16 * g, F4 ? ksb + (int64_t)j * ks_rstride + g : nullptr);
    }
  };
  // ST (PF): selected keys and candidates staged in LDS, as a compile-time
  // choice, so that the staged loop holds no global memory operation.
  auto score_chunk = [&](auto st_tag, const uint32_t (&f)[FW], int c) {
    constexpr bool ST = decltype(st_tag)::value;
    v4f acc[HP];
    if constexpr (F4) {
      const v8i ka = v8i{(int)f[0], (int)f[1], (int)f[2], (int)f[3], 0, 0, 0, 0};
      const int sa = (int)f[4];
#pragma unroll
      for (int h = 0; h < HP; ++h)
        acc[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb[h], v4f{0.f, 0.f, 0.f, 0.f}, 4 /* A E2M1 */,
                                                                  0 /* B E4M3 */, 0, sa, 0, 127);
    } else {
      const v8i ka = v8i{(int)f[0], (int)f[1], (int)f[2], (int)f[3], (int)f[4], (int)f[5], (int)f[6], (int)f[7]};
#pragma unroll
      for (int h = 0; h < HP; ++h)
        acc[h] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ka, qb[h], v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 127,
                                                                  0, 127);
    }
    // acc[h][r] = dot(key j0 + r, query c16, head h)
    const int j0 = ik0 + 16 * c + 4 * g;
    uint32_t kk[4];
    uint32_t em = 0u, bm = 0u;   // PF: keys to emit / in the undecided bucket
    uint32_t pm = 0u;            // PF: visible keys
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
      if constexpr (PF) {
        kk[r] = key;
        pm |= (vis ? 1u : 0u) << r;
      } else if constexpr (PFM == 1) {
        // (most keys of the fine sample pass lie below the range: skipped,
        // not sent to one shared word)
        const uint32_t d = (key - s_lo) >> s_sh;
        if (vis && key >= s_lo) atomicAdd(&hist[hbase + (d > 4095u ? 4095u : d)], add);
      } else {
        kk[r] = vis ? key : 0u;
        atomicAdd(&hist[vis ? hbase + (key >> 20) : kTrash], add);
      }
    }
    // Positions up to the next multiple of 16 lie inside the row's key
    // stride; entries past the visible count are never read.
    if constexpr (PFM == 0) {
      if (tok_q) *reinterpret_cast<v4u*>(krow + j0) = v4u{kk[0], kk[1], kk[2], kk[3]};
    }
    if constexpr (PF) {
      // (branch-free: the exact key ranges on every visible key; a score
      // prefilter that skipped the ranges paid more in branches than it saved)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool in = (pm >> r) & 1u;
        em |= (in && kk[r] >= pl.e_lo && kk[r] <= pl.e_hi ? 1u : 0u) << r;
        bm |= (in && kk[r] >= pl.b_lo && kk[r] <= pl.b_hi ? 1u : 0u) << r;
      }
      if constexpr (ST) {
        // (a staged tile holds no histogram or tie-emission row) One put
        // per selected key, in a loop over the lane's set bits: the wave
        // runs it as often as its busiest lane needs (mostly once), not once
        // per key slot and kind.
        if (bm && pl.mode == PF_TIECOUNT) atomicAdd(&tcnt[c16], (uint32_t)__builtin_popcount(bm));
        uint32_t sel = em | (pl.mode == PF_CAND ? bm : 0u);
        while (sel) {
          const int r = __builtin_ctz(sel);
          sel &= sel - 1u;
          const uint32_t k = r == 0 ? kk[0] : (r == 1 ? kk[1] : (r == 2 ? kk[2] : kk[3]));
          const uint32_t kind = (em >> r) & 1u ? 0u : 1u;
          uint32_t n = kind ? lane_nc : lane_ne;
          pf_lane_put2(hist, hist + kPoolOff, &pool_cnt, &spill, (int)kind, c16, n, j0 + r, k);
          if (kind) lane_nc = n;
          else lane_ne = n;
        }
      } else {
        if (em) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (em & (1u << r)) pf_emit(pf, row0 + c16, j0 + r, kk[r]);
        }
        if (bm) {
          if (pl.mode == PF_HIST) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (bm & (1u << r)) atomicAdd(&hist[hbase + pf_digit(kk[r], pl.n_ps)], add);
          } else if (pl.mode == PF_CAND) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
              if (bm & (1u << r)) pf_cand(pf, row0 + c16, j0 + r, kk[r]);
          } else if (pl.mode == PF_TIECOUNT) {
            atomicAdd(&tcnt[c16], (uint32_t)__builtin_popcount(bm));
          } else if (pl.mode == PF_TIEEMIT) {
            atomicOr(&hist[c * QW + c16], bm << (4 * g));
          }
        }
      }
    }
  };
  // Chunks c = wave, wave + 8, ... (pass 0: of the sampled chunks); PD
  // chunks in flight per wave (loads past the tile read clamped rows).
  auto key_loop = [&](auto st_tag) {
    const int nloop = pf_nloop<PFM>(nchunks);
    int c = wave;
#pragma unroll
    for (int d = 0; d < PD; ++d) load_chunk(fk[d], pf_chunk<PFM>(c + d * kPrefillWaves));
    for (; c < nloop; c += PD * kPrefillWaves) {
#pragma unroll
      for (int d = 0; d < PD; ++d) {
        const int cd = c + d * kPrefillWaves;
        if (cd < nloop && pf_chunk<PFM>(cd) < nchunks) score_chunk(st_tag, fk[d], pf_chunk<PFM>(cd));
        load_chunk(fk[d], pf_chunk<PFM>(cd + PD * kPrefillWaves));
      }
    }
  };
  if (PF && stage) key_loop(std::true_type{});
  else key_loop(std::false_type{});
  __syncthreads();
  if constexpr (PF) {
    if (stage && spill) {
      // The staging space overflowed: score the tile again, every selected
      // key and candidate taking its global slot directly (tie counts start
      // over; staging excludes histogram and tie-emission rows).
      stage = false;
      if (threadIdx.x < QW) tcnt[threadIdx.x] = 0u;
      __syncthreads();
      key_loop(std::false_type{});
      __syncthreads();
    }
    if (stage) {
      pf_lane_flush<QW, kPrefillWaves>(pf, hist, lane_ne, lane_nc, sbase, row0, Tq, t0);
      const uint32_t np = pool_cnt < (uint32_t)kPfPool ? pool_cnt : (uint32_t)kPfPool;
      const uint32_t* pool = hist + kPoolOff;
      for (uint32_t i = threadIdx.x; i < np; i += NT) {
        const uint32_t tag = pool[3 * i + 2];
        const int ql = tag & 15;
        if (tag >> 4) pf_cand(pf, row0 + ql, pool[3 * i], pool[3 * i + 1]);
        else pf_emit(pf, row0 + ql, pool[3 * i], pool[3 * i + 1]);
      }
    }
    pf_finish<QW, NT>(pf, pfl, flags, hist, tcnt, row0, Tq, t0, kx, k0, nchunks);
    return;
  }
  if constexpr (PFM == 1) {
    pf_flush_hist<QW, NT>(pf, hist, row0, Tq, t0);
    return;
  }
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
constexpr int kPrefillQW = 4 * ((HG * (DI / 128) <= 2) ? 4 : (HG * (DI / 128) <= 4 ? 2 : 1));

// pf == nullptr: the whole chunk, score keys stored for the radix select;
// else selection pass `pass` over the query tiles [y0, y0 + ny) (pass 0:
// the level-1 histograms, later ones steered by the rows' states).
template <int DI, int HG>
static hipError_t launch_prefill_t(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                   const SelectWs& tok, const PfArgs* pf, int pass, int64_t y0, int64_t ny,
                                   hipStream_t s) {
  constexpr int QG = (HG * (DI / 128) <= 2) ? 4 : (HG * (DI / 128) <= 4 ? 2 : 1);
  constexpr int QW = 4 * QG;
  static_assert(QW == kPrefillQW<DI, HG>, "query tile");
  const bool kt = DI == 128 && HG <= 2;   // the transposed product (16 queries per workgroup)
  const int qtiles = (a.Tq + QW - 1) / QW;
  const int64_t qrows = pf ? ny : (int64_t)a.B * qtiles;
  // Key tiles: at most 8192 keys (per-tile counts stay below 2^16; sample
  // passes: kPfSample times as many keys, of which they score 8192), smaller
  // while the grid would not cover the compute units twice; for the
  // selection passes at most 4096 tiles per row (their tie counts).
  const int pfm = !pf ? 0 : (pass < 2 ? 1 : 2);
  int key_tile = pfm == 1 ? 8192 * kPfSample : 8192;
  const int64_t want = 2LL * device_cu_count();
  while (key_tile > 512 && qrows * ((a.n_max + key_tile - 1) / key_tile) < want) key_tile >>= 1;
  while (pf && key_tile < 8192 && (a.n_max + key_tile - 1) / key_tile > 4096) key_tile <<= 1;
  int64_t tiles = (a.n_max + key_tile - 1) / key_tile;
  if (tiles < 1) tiles = 1;
  if (qrows > 65535 || (pf && tiles > 4096)) return hipErrorInvalidValue;
  if (a.k_scales && DI != 128) return hipErrorInvalidValue;   // (MXFP4 keys: 128 channels)
  const dim3 grid((unsigned)tiles, (unsigned)qrows), block(64 * kPrefillWaves);
  PfArgs pfa = pf ? *pf : PfArgs{};
  pfa.pass = pass;
  const uint8_t* ks = a.k_scales;
#define KT_ARGS a.q_idx, a.w, a.k_idx, a.k_bstride, a.k_rstride, ks, a.ks_bstride, a.ks_rstride, a.ctx_len, a.q_pos, \
                a.Tq, a.H_I, a.n_max, key_tile, qtiles, keys, key_stride, n_valid, tok, pfa, y0
#define GEN_ARGS a.q_idx, a.w, a.k_idx, a.k_bstride, a.k_rstride, ks, a.ks_bstride, a.ks_rstride, a.ctx_len, a.q_pos, \
                 a.Tq, a.H_I, a.n_max, key_tile, qtiles, keys, key_stride, n_valid, tok, pfa, y0
  if (kt) {
    if (a.k_scales) {
      if (pfm == 0) CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3, true, 0>), grid, block, 0, s, KT_ARGS);
      else if (pfm == 1) CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3, true, 1>), grid, block, 0, s, KT_ARGS);
      else CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3, true, 2>), grid, block, 0, s, KT_ARGS);
    } else {
      if (pfm == 0) CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3, false, 0>), grid, block, 0, s, KT_ARGS);
      else if (pfm == 1) CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3, false, 1>), grid, block, 0, s, KT_ARGS);
      else CSA2_LAUNCH("index_prefill", (index_prefill_kt_kernel<3, false, 2>), grid, block, 0, s, KT_ARGS);
    }
  } else if (a.k_scales) {
    if constexpr (DI == 128) {
      if (pfm == 0) CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG, 0, true>), grid, block, 0, s, GEN_ARGS);
      else if (pfm == 1) CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG, 1, true>), grid, block, 0, s, GEN_ARGS);
      else CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG, 2, true>), grid, block, 0, s, GEN_ARGS);
    }
  } else {
    if (pfm == 0) CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG, 0, false>), grid, block, 0, s, GEN_ARGS);
    else if (pfm == 1) CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG, 1, false>), grid, block, 0, s, GEN_ARGS);
    else CSA2_LAUNCH("index_prefill", (index_prefill_kernel<DI, HG, QG, 2, false>), grid, block, 0, s, GEN_ARGS);
  }
#undef KT_ARGS
#undef GEN_ARGS
  return hipGetLastError();
}

bool prefill_gemm_applies(const ScoreArgs& a) {
  if (a.k_scales) return a.Tq >= 16 && a.pool_block == 0 && a.D_I == 128 && a.H_I <= 32;
  return a.Tq >= 16 && a.pool_block == 0 && (a.D_I == 128 || a.D_I == 256) && a.H_I <= 32;
}

static int prefill_hg(const ScoreArgs& a) {
  const int hg = (a.H_I + 3) / 4;
  return hg <= 1 ? 1 : (hg <= 2 ? 2 : (hg <= 4 ? 4 : 8));
}

int prefill_rows_per_tile(const ScoreArgs& a) {
  const int H = prefill_hg(a);
  if (a.D_I == 128) return H == 1 ? kPrefillQW<128, 1> : H == 2 ? kPrefillQW<128, 2> : H == 4 ? kPrefillQW<128, 4>
                                                                                       : kPrefillQW<128, 8>;
  return H == 1 ? kPrefillQW<256, 1> : H == 2 ? kPrefillQW<256, 2> : H == 4 ? kPrefillQW<256, 4> : kPrefillQW<256, 8>;
}

static hipError_t launch_prefill_any(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                     const SelectWs& tok, const PfArgs* pf, int pass, int64_t y0, int64_t ny,
                                     hipStream_t s) {
  const int HGp = prefill_hg(a);
#define CALL_PF(D, H) launch_prefill_t<D, H>(a, keys, key_stride, n_valid, tok, pf, pass, y0, ny, s)
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

static hipError_t launch_prefill(const ScoreArgs& a, uint32_t* keys, int64_t key_stride, int32_t* n_valid,
                                 const SelectWs& tok, hipStream_t s) {
  return launch_prefill_any(a, keys, key_stride, n_valid, tok, nullptr, 0, 0, 0, s);
}

hipError_t launch_prefill_pass(const ScoreArgs& a, const PfArgs& pf, int pass, int64_t y0, int64_t ny,
                               int32_t* n_valid, hipStream_t s) {
  return launch_prefill_any(a, nullptr, 0, n_valid, SelectWs{}, &pf, pass, y0, ny, s);
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
  const bool f4 = a.k_scales != nullptr;
  switch (scan_qt(a)) {
    case 2: return f4 ? launch_scan_mq<2, true>(a, keys, key_stride, n_valid, tok, s)
                      : launch_scan_mq<2, false>(a, keys, key_stride, n_valid, tok, s);
    case 4: return f4 ? launch_scan_mq<4, true>(a, keys, key_stride, n_valid, tok, s)
                      : launch_scan_mq<4, false>(a, keys, key_stride, n_valid, tok, s);
    default: break;
  }
  if (f4) {   // MXFP4 keys: D_I = 128, up to 32 indexer heads
    if (a.D_I != 128 || a.H_I > 32) return hipErrorInvalidValue;
    if (a.H_I <= 8) return launch_scan_t<128, 1, true, true>(a, keys, key_stride, n_valid, tok, bkeys, bkey_stride,
                                                             nb_valid, blk, s);
    if (a.H_I <= 16) return launch_scan_t<128, 1, false, true>(a, keys, key_stride, n_valid, tok, bkeys, bkey_stride,
                                                               nb_valid, blk, s);
    return launch_scan_t<128, 2, false, true>(a, keys, key_stride, n_valid, tok, bkeys, bkey_stride, nb_valid, blk, s);
  }
#define CALL_SCAN(D, H, E) launch_scan_t<D, H, E>(a, keys, key_stride, n_valid, tok, bkeys, bkey_stride, nb_valid, blk, s)
  CSA2_DISPATCH_DI_HB(a.D_I, a.H_I, CALL_SCAN);
#undef CALL_SCAN
}

int64_t index_score_tiles(const ScoreArgs& a) {
  if (prefill_gemm_applies(a)) return 0;
  const int qt = scan_qt(a);
  int tile;
  if (qt == 2) {
    tile = scan_tile((int64_t)a.B * ((a.Tq + 1) / 2), a.n_max, kScanWavesT<false, 1, 2>, 2);
  } else if (qt == 4) {
    tile = scan_tile((int64_t)a.B * ((a.Tq + 3) / 4), a.n_max, kScanWavesT<false, 1, 4>, 4);
  } else {
    const bool f4 = a.k_scales != nullptr;
    tile = scan_tile((int64_t)a.B * a.Tq, a.n_max,
                     a.H_I <= 16 ? kScanWavesT<false, 1> : (f4 ? kScanWavesT<false, 2, 1, true> : kScanWavesT<false, 2>));
  }
  const int64_t tiles = (a.n_max + tile - 1) / tile;
  return tiles < 1 ? 1 : tiles;
}

int64_t index_score_tiles_bound(int64_t n_max) {
  const int64_t tiles = (n_max + kScanTileSmall - 1) / kScanTileSmall;
  return tiles < 1 ? 1 : tiles;
}

hipError_t launch_pool_score(const ScoreArgs& a, const int32_t* pool_idx, const int32_t* pool_len, int pool_cap,
                             uint32_t* keys, int64_t key_stride, int32_t* n_valid, const SelectWs& ws, hipStream_t s) {
  if (a.k_scales) {   // MXFP4 keys
    if (a.D_I != 128 || a.H_I > 32) return hipErrorInvalidValue;
    if (a.H_I <= 8) return launch_pool_t<128, 1, true, true>(a, pool_idx, pool_len, pool_cap, keys, key_stride, n_valid,
                                                             ws, s);
    if (a.H_I <= 16) return launch_pool_t<128, 1, false, true>(a, pool_idx, pool_len, pool_cap, keys, key_stride,
                                                               n_valid, ws, s);
    return launch_pool_t<128, 2, false, true>(a, pool_idx, pool_len, pool_cap, keys, key_stride, n_valid, ws, s);
  }
#define CALL_POOL(D, H, E) launch_pool_t<D, H, E>(a, pool_idx, pool_len, pool_cap, keys, key_stride, n_valid, ws, s)
  CSA2_DISPATCH_DI_HB(a.D_I, a.H_I, CALL_POOL);
#undef CALL_POOL
}

}  // namespace csa2
