// Device helpers shared by the CSA2 kernels: number-format codecs written from
// the OCP MX v1.0 bit definitions, order-preserving score keys, agent-scope
// atomics and the launch/trace plumbing.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

typedef float v4f __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));
typedef int v8i __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- codecs ---

// E4M3FN byte -> float (exact).  Bias 7; exponent field 0 is subnormal
// (m * 2^-9).  0x7F / 0xFF (NaN) are outside the contract.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
  uint32_t e = (b >> 3) & 15u, m = b & 7u;
  float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * (1.0f / 512.0f);
  return (b & 0x80u) ? -v : v;
}

// float -> E4M3FN byte, round to nearest even, saturating at 448.  The sign
// bit of x is kept (a tiny negative value encodes as 0x80).
__device__ __forceinline__ uint32_t f32_to_e4m3(float x) {
  uint32_t u = __float_as_uint(x);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7FFFFFFFu;
  uint32_t code;
  if (a >= 0x43E80000u) {          // |x| >= 464: 464 ties to 448, above saturates
    code = 0x7Eu;
  } else if (a < 0x3C800000u) {    // |x| < 2^-6: subnormal grid m * 2^-9
    float t = __uint_as_float(a) * 512.0f;  // exact power-of-two scaling
    code = (uint32_t)__builtin_rintf(t);    // RNE; 8 becomes the first normal
  } else {
    uint32_t exp = (a >> 23) - 120u;        // E4M3 biased exponent, 1..15
    uint32_t mant = a & 0x7FFFFFu;
    uint32_t keep = mant >> 20, rest = mant & 0xFFFFFu;
    keep += (rest > 0x80000u) || (rest == 0x80000u && (keep & 1u));
    code = (exp << 3) + keep;               // a mantissa carry moves into the exponent
  }
  return code | sign;
}

// E8M0 byte -> float 2^(b-127) for b in [1, 254]; b = 0 gives 2^-127.
__device__ __forceinline__ float e8m0_to_f32(uint32_t b) {
  return b ? __uint_as_float(b << 23) : __uint_as_float(0x00400000u);
}

// Magnitude code of an E2M1 value (0..7) -> fp16 bit pattern.
// Codes 2..7 are normal: exponent (c >> 1) - 1, one mantissa bit; code 1 is 0.5.
__device__ __forceinline__ uint32_t e2m1_mag_to_f16_bits(uint32_t c) {
  return c >= 2u ? ((((c >> 1) + 14u) << 10) | ((c & 1u) << 9)) : (c ? 0x3800u : 0u);
}

// -------------------------------------------------------- ordered keys ---

// Order-preserving map float -> u32 (larger score -> larger key).  -0 is
// folded onto +0 first.  Finite scores map to keys >= 0x00800000, so key 0
// never belongs to a visible token.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if ((u << 1) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

// ------------------------------------------------------------- atomics ---

__device__ __forceinline__ uint32_t atomic_add_agent(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint64_t atomic_add_agent64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t atomic_add_agent_acq_rel(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_agent(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_agent(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// "Last workgroup" election: every workgroup of a group calls this once after
// publishing its contribution with agent-scope atomics (RMW or atomic
// stores); exactly one workgroup -- the last to arrive -- gets true, and its
// agent-scope loads then observe every other workgroup's contribution.  No
// workgroup waits for another.  Each thread first waits for its own memory
// operations to be acknowledged (they are performed at the agent coherence
// point by then), so the counter increment that follows the barrier is
// ordered after all of them without a release fence; a release fence here
// would write back the whole L2 of the XCD once per workgroup.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected, uint32_t* lds_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *lds_flag = (prev == expected - 1u) ? 1u : 0u;
  }
  __syncthreads();
  return *lds_flag != 0u;
}

}  // namespace csa2
