// Device-side pieces of the radix select shared by the select passes and by
// the producers (scoring kernels) that build the first histogram themselves.
#pragma once

#include "common.h"
#include "internal.h"

namespace csa2 {

// ------------------------------------------------------------ helpers ---

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

// Given a global histogram of BINS bins and need >= 1 (<= total), find the
// digit d with  sum_{e>d} h[e] < need <= sum_{e>=d} h[e].  Returns (d, above,
// count of d) in res[0..2].  Run by all 256 threads of the workgroup.
template <int BINS>
__device__ void resolve_digit(const uint32_t* hist, uint32_t need, uint32_t* red, uint32_t* res) {
  constexpr int BPT = BINS / 256;
  uint32_t h[BPT];
  uint32_t sum = 0;
#pragma unroll
  for (int i = 0; i < BPT; ++i) {
    h[i] = load_agent(hist + threadIdx.x * BPT + i);
    sum += h[i];
  }
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
}

__device__ __forceinline__ uint32_t row_total_from_hist(const uint32_t* hist, uint32_t* red) {
  uint32_t sum = 0;
  for (int i = 0; i < 16; ++i) sum += load_agent(hist + threadIdx.x * 16 + i);
  uint32_t incl = block_suffix_sum_256(sum, red);
  __shared__ uint32_t tot;
  if (threadIdx.x == 0) tot = incl;
  __syncthreads();
  return tot;
}

// Digit-1 resolution, run by the last workgroup of a row's first pass
// (producers that build histogram 1 call this too).
__device__ __forceinline__ void select_resolve1(SelectRowCtl* ctl, const uint32_t* hist1, uint32_t k) {
  __shared__ uint32_t red[4];
  __shared__ uint32_t res[3];
  uint32_t total = row_total_from_hist(hist1, red);
  if (total <= k) {
    if (threadIdx.x == 0) {
      ctl->mode = 1u; ctl->thr = 0u; ctl->need_eq = 0u; ctl->total = total;
    }
    return;
  }
  resolve_digit<4096>(hist1, k, red, res);
  if (threadIdx.x == 0) {
    uint32_t d = res[0], above = res[1], cnt = res[2];
    uint32_t need = k - above;
    ctl->mode = 0u;
    ctl->prefix = d;
    ctl->need = need;
    ctl->total = k;
    if (need == cnt) {              // the whole bucket is taken
      ctl->mode = 2u;
      ctl->thr = (d << 20) - 1u;
      ctl->need_eq = 0u;
    }
  }
}


}  // namespace csa2
