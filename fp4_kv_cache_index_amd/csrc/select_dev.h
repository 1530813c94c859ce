// Device-side helpers of the radix select: workgroup scans and the
// resolution of a radix digit from a histogram.
#pragma once

#include "common.h"
#include "internal.h"

namespace csa2 {

// Inclusive suffix sum over the 256 threads of a workgroup (thread t gets
// the sum of v over threads t..255).  `red` is LDS scratch of 4 words.
__device__ __forceinline__ uint32_t block_suffix_sum_256(uint32_t v, uint32_t* red) {
  int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_down(v, off, 64);
    if (lane + off < 64) v += y;
  }
  if (lane == 0) red[wv] = v;  // wave total
  __syncthreads();
  uint32_t add = 0;
  for (int w2 = wv + 1; w2 < 4; ++w2) add += red[w2];
  __syncthreads();
  return v + add;
}

// Inclusive prefix sum over 256 threads (thread t gets v_0 + ... + v_t).
__device__ __forceinline__ uint32_t block_prefix_sum_256(uint32_t v, uint32_t* red) {
  int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    uint32_t y = __shfl_up(v, off, 64);
    if (lane >= off) v += y;
  }
  if (lane == 63) red[wv] = v;
  __syncthreads();
  uint32_t add = 0;
  for (int w2 = 0; w2 < wv; ++w2) add += red[w2];
  __syncthreads();
  return v + add;
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP lane moves:
// shifts by 1, 2, 4 and 8 inside each 16-lane row, then lane 15 of a row
// into the next row and lane 31 into the upper half.  Lanes whose source is
// outside the row receive 0.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  int x = (int)v;
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);   // row_bcast:15 into rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);   // row_bcast:31 into rows 2, 3
  return (uint32_t)x;
}

// Digit of a BINS-bin histogram (global or shared memory) at which the
// running count from the top reaches `need` (1 <= need <= total):
//   sum_{e>d} h[e] < need <= sum_{e>=d} h[e].
// Every thread returns the same (d, above = sum_{e>d} h[e], h[d]).
struct Digit {
  uint32_t d, above, cnt;
};

// Resolution from per-thread bin counts h[0..BPT) of bins tid*BPT + i.
template <int BPT>
__device__ Digit resolve_digit_regs(const uint32_t (&h)[BPT], uint32_t need, uint32_t* red, uint32_t* res) {
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) sum += h[i];
  uint32_t incl = block_suffix_sum_256(sum, red);
  uint32_t excl = incl - sum;
  if (excl < need && need <= incl) {
    uint32_t run = excl;
#pragma unroll
    for (int i = BPT - 1; i >= 0; --i) {
      if (run + h[i] >= need && run < need) {
        res[0] = threadIdx.x * BPT + i;
        res[1] = run;
        res[2] = h[i];
      }
      run += h[i];
    }
  }
  __syncthreads();
  Digit r{res[0], res[1], res[2]};
  __syncthreads();
  return r;
}

template <int BINS>
__device__ Digit resolve_digit(const uint32_t* hist, uint32_t need, uint32_t* red, uint32_t* res) {
  constexpr int BPT = BINS / 256;
  uint32_t h[BPT];
#pragma unroll
  for (int i = 0; i < BPT; ++i) h[i] = hist[threadIdx.x * BPT + i];
  return resolve_digit_regs<BPT>(h, need, red, res);
}

// First-digit state of a row, derived from its complete 12-bit histogram.
struct Level1 {
  uint32_t total;   // valid positions of the row
  uint32_t mode;    // 0: refine inside bucket d; 1: take every valid position;
                    // 2: take buckets >= d whole (threshold thr1 = (d << 20) - 1)
  uint32_t d, above, cnt;
};

__device__ __forceinline__ Level1 resolve_level1(const uint32_t* hist1, uint32_t k, uint32_t* red, uint32_t* res) {
  uint32_t h[16];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    h[i] = hist1[threadIdx.x * 16 + i];
    sum += h[i];
  }
  // Total: thread 0's inclusive suffix sum.
  uint32_t incl = block_suffix_sum_256(sum, red);
  if (threadIdx.x == 0) res[3] = incl;
  __syncthreads();
  Level1 L{res[3], 1u, 0u, 0u, 0u};
  __syncthreads();
  if (L.total <= k) return L;
  const uint32_t excl = incl - sum;
  if (excl < k && k <= incl) {
    uint32_t run = excl;
#pragma unroll
    for (int i = 15; i >= 0; --i) {
      if (run + h[i] >= k && run < k) {
        res[0] = threadIdx.x * 16 + i;
        res[1] = run;
        res[2] = h[i];
      }
      run += h[i];
    }
  }
  __syncthreads();
  L.d = res[0];
  L.above = res[1];
  L.cnt = res[2];
  __syncthreads();
  L.mode = (k - L.above == L.cnt) ? 2u : 0u;
  return L;
}

}  // namespace csa2
