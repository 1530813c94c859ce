// Cache writers: FP4 main KV (E2M1 + E4M3 per 16 channels), the FP8
// sliding window (E4M3 + E8M0 per 32 channels) and the MXFP4 indexer keys
// (E2M1 + E8M0 per 32 channels).
//
// The main-KV format is the one the DeepSeek-V4.1 blog gives for CSA2 (FP4
// E2M1 values, one E4M3 scale per 16 channels) with the fact sheet's entry
// layout (256 data bytes then 32 scale bytes for 512 elements); the cache is
// written after RoPE (techniques map, post-RoPE KV-cache quantization), so
// every channel goes through the same quantiser.  The window format is the
// fact sheet's SWA group (E4M3 values, one E8M0 scale per 32 channels).
// Rounding rules (not given on the pages): the FP4 scale is E4M3(amax / 6)
// and each element takes the E2M1 value nearest its exact quotient by the
// scale, ties to the even code; the window uses the OCP MX shared exponent
// floor(log2 amax) - 8.  Both are HBM-streaming kernels: one thread per
// channel group, consecutive threads on consecutive groups of a row.
#include "common.h"
#include "internal.h"

namespace csa2 {

// One thread per 16-channel group: 64 B in, 8 code bytes + 1 scale byte out.
__global__ void __launch_bounds__(256)
kv_fp4_quantize_kernel(const float* __restrict__ x, int64_t n_groups, int gpr, int64_t x_stride,
                       uint8_t* __restrict__ codes, int64_t c_stride, uint8_t* __restrict__ scales,
                       int64_t s_stride) {
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < n_groups;
       gid += (int64_t)gridDim.x * blockDim.x) {
    int64_t row = gid / gpr;
    int g = (int)(gid - row * gpr);
    const float* src = x + row * x_stride + (int64_t)g * 16;
    float v[16];
    if ((((uintptr_t)src) & 15u) == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4 f = reinterpret_cast<const float4*>(src)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = src[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t sc = f32_to_e4m3(amax / 6.0f);   // IEEE float32 division
    float s = e4m3_to_f32(sc);
    // E2M1 code = number of thresholds t*s that |x| passes; the ties
    // 0.25, 1.25, 2.5, 5 go down (strict) and 0.75, 1.75, 3.5 go up, which is
    // round-to-nearest-even on the code.  Every t*s is exact in float32.
    float t025 = 0.25f * s, t075 = 0.75f * s, t125 = 1.25f * s, t175 = 1.75f * s;
    float t250 = 2.5f * s, t350 = 3.5f * s, t500 = 5.0f * s;
    uint32_t lo = 0, hi = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a = fabsf(v[i]);
      uint32_t c = (uint32_t)(a > t025) + (uint32_t)(a >= t075) + (uint32_t)(a > t125) +
                   (uint32_t)(a >= t175) + (uint32_t)(a > t250) + (uint32_t)(a >= t350) +
                   (uint32_t)(a > t500);
      if (sc == 0u) c = 0u;
      c |= (c != 0u && v[i] < 0.0f) ? 8u : 0u;
      if (i < 8) lo |= c << (4 * i); else hi |= c << (4 * (i - 8));
    }
    uint8_t* cdst = codes + row * c_stride + (int64_t)g * 8;
    uint32_t* c32 = reinterpret_cast<uint32_t*>(cdst);
    c32[0] = lo;
    c32[1] = hi;
    scales[row * s_stride + g] = (uint8_t)sc;
  }
}

// One thread per 32-channel group: 128 B in, 32 value bytes + 1 scale byte out.
__global__ void __launch_bounds__(256)
swa_fp8_quantize_kernel(const float* __restrict__ x, int64_t n_groups, int gpr, int64_t x_stride,
                        uint8_t* __restrict__ vals, int64_t v_stride, uint8_t* __restrict__ scales,
                        int64_t s_stride) {
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < n_groups;
       gid += (int64_t)gridDim.x * blockDim.x) {
    int64_t row = gid / gpr;
    int g = (int)(gid - row * gpr);
    const float* src = x + row * x_stride + (int64_t)g * 32;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = src[i];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t code = 127u;
    if (amax > 0.0f) {
      uint32_t u = __float_as_uint(amax);
      int e = (u >= 0x00800000u) ? (int)(u >> 23) - 127 : (31 - __clz((int)u)) - 149;  // floor(log2 amax)
      int c = e - 8 + 127;
      code = (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
    }
    // x / 2^(code-127) as a multiply by the exact power of two 2^(127-code);
    // 127 - code lies in [-119, 127], so the factor is a normal float.
    float inv = __uint_as_float((uint32_t)(254 - (int)code) << 23);
    uint32_t packed[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t p = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) p |= f32_to_e4m3(v[4 * i + j] * inv) << (8 * j);
      packed[i] = p;
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(vals + row * v_stride + (int64_t)g * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[i] = packed[i];
    scales[row * s_stride + g] = (uint8_t)code;
  }
}

// Indexer K write (fact sheet, indexer K groups: MXFP4, E2M1 values with one
// E8M0 scale per 32 channels).  One thread per 32-channel group: 128 B in,
// 16 code bytes + 1 scale byte out.  Shared exponent floor(log2 amax) - 2
// (the OCP MX rule; 2 is E2M1's largest exponent), code 127 for an all-zero
// group; each element takes the E2M1 value nearest x / 2^shared, ties to the
// even code, saturating at 6 -- the same threshold comparisons as the main
// KV write with a power-of-two scale (every t * 2^e is exact in float32).
__global__ void __launch_bounds__(256)
idx_mxfp4_quantize_kernel(const float* __restrict__ x, int64_t n_groups, int gpr, int64_t x_stride,
                          uint8_t* __restrict__ codes, int64_t c_stride, uint8_t* __restrict__ scales,
                          int64_t s_stride) {
  for (int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; gid < n_groups;
       gid += (int64_t)gridDim.x * blockDim.x) {
    int64_t row = gid / gpr;
    int g = (int)(gid - row * gpr);
    const float* src = x + row * x_stride + (int64_t)g * 32;
    float v[32];
    if ((((uintptr_t)src) & 15u) == 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float4 f = reinterpret_cast<const float4*>(src)[i];
        v[4 * i] = f.x; v[4 * i + 1] = f.y; v[4 * i + 2] = f.z; v[4 * i + 3] = f.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = src[i];
    }
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    uint32_t code = 127u;
    if (amax > 0.0f) {
      uint32_t u = __float_as_uint(amax);
      int e = (u >= 0x00800000u) ? (int)(u >> 23) - 127 : (31 - __clz((int)u)) - 149;  // floor(log2 amax)
      int c = e - 2 + 127;
      code = (uint32_t)(c < 0 ? 0 : (c > 254 ? 254 : c));
    }
    const float sc = e8m0_to_f32(code);   // 2^(code - 127), exact (subnormal for code 0)
    const float t025 = 0.25f * sc, t075 = 0.75f * sc, t125 = 1.25f * sc, t175 = 1.75f * sc;
    const float t250 = 2.5f * sc, t350 = 3.5f * sc, t500 = 5.0f * sc;
    uint32_t words[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const float a = fabsf(v[i]);
      uint32_t c = (uint32_t)(a > t025) + (uint32_t)(a >= t075) + (uint32_t)(a > t125) + (uint32_t)(a >= t175) +
                   (uint32_t)(a > t250) + (uint32_t)(a >= t350) + (uint32_t)(a > t500);
      c |= (c != 0u && v[i] < 0.0f) ? 8u : 0u;
      words[i >> 3] |= c << (4 * (i & 7));
    }
    uint32_t* c32 = reinterpret_cast<uint32_t*>(codes + row * c_stride + (int64_t)g * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) c32[i] = words[i];
    scales[row * s_stride + g] = (uint8_t)code;
  }
}

static int grid_for(int64_t work, int block) {
  int64_t g = (work + block - 1) / block;
  int64_t cap = (int64_t)device_cu_count() * 32;
  if (g > cap) g = cap;
  return (int)(g < 1 ? 1 : g);
}

hipError_t launch_kv_fp4_quantize(const float* x, int64_t n_rows, int d, int64_t x_stride,
                                  uint8_t* codes, int64_t c_stride, uint8_t* scales, int64_t s_stride,
                                  hipStream_t s) {
  int gpr = d / 16;
  int64_t n_groups = n_rows * gpr;
  if (n_groups == 0) return hipSuccess;
  CSA2_LAUNCH("kv_fp4_quantize", kv_fp4_quantize_kernel, dim3(grid_for(n_groups, 256)), dim3(256), 0, s,
              x, n_groups, gpr, x_stride, codes, c_stride, scales, s_stride);
  return hipGetLastError();
}

hipError_t launch_idx_mxfp4_quantize(const float* x, int64_t n_rows, int d, int64_t x_stride,
                                     uint8_t* codes, int64_t c_stride, uint8_t* scales, int64_t s_stride,
                                     hipStream_t s) {
  int gpr = d / 32;
  int64_t n_groups = n_rows * gpr;
  if (n_groups == 0) return hipSuccess;
  CSA2_LAUNCH("idx_mxfp4_quantize", idx_mxfp4_quantize_kernel, dim3(grid_for(n_groups, 256)), dim3(256), 0, s,
              x, n_groups, gpr, x_stride, codes, c_stride, scales, s_stride);
  return hipGetLastError();
}

hipError_t launch_swa_fp8_quantize(const float* x, int64_t n_rows, int d, int64_t x_stride,
                                   uint8_t* vals, int64_t v_stride, uint8_t* scales, int64_t s_stride,
                                   hipStream_t s) {
  int gpr = d / 32;
  int64_t n_groups = n_rows * gpr;
  if (n_groups == 0) return hipSuccess;
  CSA2_LAUNCH("swa_fp8_quantize", swa_fp8_quantize_kernel, dim3(grid_for(n_groups, 256)), dim3(256), 0, s,
              x, n_groups, gpr, x_stride, vals, v_stride, scales, s_stride);
  return hipGetLastError();
}

}  // namespace csa2
