// Sparse MLA attention over the Top-K FP4 main-KV rows plus the FP8 window.
//
// What it computes (DeepSeek-V4.1-Flash techniques map, "Checked in its
// code": multi-head latent attention with a single latent KV head and a
// learnable per-head sink logit in the sparse-MLA softmax denominator; fact
// sheet: one shared K=V entry per token, a 128-token window per layer; blog,
// CSA2 paragraph: attention runs over the indexer's Top-K entries of the FP4
// main cache): for each query row and head h, softmax over the selected
// entries (and the sink) of scale * q_h . k_e, applied to v_e = the first
// d_v channels of the same row.
//
// gfx950 mapping.  A workgroup holds one query row and a contiguous split of
// its entry list (Top-K rows, then the window rows); workgroups are numbered
// so that the splits of one row land on the same XCD and share its q in L2.
// Chunks of 64 entries are double-buffered in LDS as fp16 rows: while a
// chunk is consumed, the next one is dequantised into the other buffer and
// the rows of the one after it are in flight.  A gather task is one entry's
// 32-channel block, consecutive lanes taking consecutive 16-byte pieces of a
// row; the rows are dequantised with the gfx950 scaled converts
// (v_cvt_scalef32_pk_f16_fp4 / _fp8, which apply the power-of-two part of
// their scale; the E4M3 scale of a main row is applied as an fp16 multiply)
// -- exact, since E2M1 x E4M3 has at most 6 significant bits within
// [2^-10, 2688].  q is read once per workgroup with coalesced loads, rounded
// to fp16 once and passed through LDS into registers.  Then, per chunk,
//   S^T = K Q^T   on v_mfma_f32_16x16x32_f16: the 8 waves (two per SIMD) are
//                 4 head groups of 16 heads x 2 halves of the chunk's entries,
//                 q held in registers;
//   online softmax in fp32 (exp2 domain); the two waves of a head group
//                 exchange row maxima; P fragments and per-head rescale
//                 factors go to LDS;
//   O  += P V     on the same instruction, the waves now 2 halves of the
//                 heads (32 each) x 4 quarters of the output dims, so every V
//                 fragment serves two head tiles (64 fp32 accumulator
//                 registers per lane).  P keeps the lane layout of the S^T
//                 accumulators (the A-operand layout once the k index is
//                 permuted identically for V), and V is read from the same
//                 fp16 rows with the LDS transpose read (ds_read_b64_tr_b16),
//                 so no transposed copy is stored.
// Splits write unnormalised partial (O, m, l); a combine kernel merges them
// with the log-sum-exp rule and adds the sink.  A row with a single split
// (4096-query prefill chunks) is normalised by the split kernel itself.
#include <type_traits>

#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kChunk = 64;           // entries per LDS chunk
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <int DQK>
struct AttnShape {
  static constexpr int G16 = DQK / 16;          // 16-channel groups per row
  static constexpr int KQ = DQK / 32;           // MFMA k-steps for S = K Q^T
  static constexpr int PITCH = DQK + 16;         // fp16 row pitch in LDS (bank spread)
};

__device__ __forceinline__ v8h load_f32x8_as_f16(const float* p) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v8h r;
  r[0] = (_Float16)a.x; r[1] = (_Float16)a.y; r[2] = (_Float16)a.z; r[3] = (_Float16)a.w;
  r[4] = (_Float16)b.x; r[5] = (_Float16)b.y; r[6] = (_Float16)b.z; r[7] = (_Float16)b.w;
  return r;
}

constexpr int kAttnThreads = 512;   // 8 waves (see the mapping above)

// Raw bytes of one gather task: one entry, one 32-channel block.
struct RawTask {
  uint32_t w[8];      // main: 16 code bytes in w[0..3]; window: 32 value bytes
  uint32_t sc;        // main: the block's two E4M3 scale bytes; window: its E8M0 byte
  uint32_t kind;      // 0 skip, 1 main, 2 window
};

template <int DQK, int DV>
__global__ void __launch_bounds__(kAttnThreads)
sparse_attn_split_kernel(AttnArgs a, int prefill, int splits, int span,
                         float* __restrict__ part_o, float* __restrict__ part_ml) {
  using S = AttnShape<DQK>;
  constexpr int NT = DV / 64;                         // output dim tiles per wave (a quarter of the dims)
  constexpr int NB = DQK / 32;                        // 32-channel blocks per row
  constexpr int NTASK = kChunk * NB;                  // (entry, block) tasks per chunk
  constexpr int QP = DQK + 8;                         // fp16 pitch of the staged q rows
  static_assert(64 * QP <= kChunk * S::PITCH, "q staging must fit one K buffer");
  constexpr int TPT = (NTASK + kAttnThreads - 1) / kAttnThreads;
  __shared__ __attribute__((aligned(16))) _Float16 kbuf[2][kChunk * S::PITCH];   // K rows, row-major, 2 chunks
  // Entry ids of three chunks (the one consumed, the one being dequantised,
  // the one being gathered): main: token id; window: window row; -1 = skip.
  __shared__ __attribute__((aligned(16))) int32_t eidc[3][kChunk];
  __shared__ float pmx[2][64];        // per-head partial maxima / sums of the two dim halves
  __shared__ __attribute__((aligned(16))) v8h pex[8][64];   // P fragments of every S wave
  __shared__ __attribute__((aligned(16))) float alf[64];     // per-head rescale factor of the chunk

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15, g = lane >> 4;
  // XCD-aware order: workgroups are dealt round-robin over the 8 XCDs in
  // launch order; renumber them so that the splits of one query row (which
  // all read its q) sit on the same XCD and share its L2.
  const int nwg = gridDim.x * gridDim.y;
  const int lin = blockIdx.x + gridDim.x * blockIdx.y;
  const int flat = (nwg & 7) == 0 ? (lin & 7) * (nwg >> 3) + (lin >> 3) : lin;
  const int64_t row = flat / gridDim.x;
  const int split = flat - (int)row * gridDim.x;
  const int64_t b = row / a.Tq;
  const int H = a.H;
  const int K = a.k_top;
  const int E = K + a.W;
  const int e_begin = split * span;
  int e_end = e_begin + span;
  if (e_end > E) e_end = E;

  const int64_t ctx = a.ctx_len[b];
  int64_t swa_r0 = 0, n_swa = 0;
  if (prefill) {
    int64_t p = a.q_pos[row];
    int64_t p0 = a.swa_pos0[b];
    int64_t lo = p - a.W + 1 > p0 ? p - a.W + 1 : p0;
    int64_t hi = p < p0 + a.swa_rows - 1 ? p : p0 + a.swa_rows - 1;
    swa_r0 = lo - p0;
    n_swa = hi >= lo ? hi - lo + 1 : 0;
  } else if (a.W > 0) {
    int64_t sl = a.swa_len[b];
    n_swa = sl < 0 ? 0 : (sl > a.W ? a.W : sl);
  }
  const int32_t* idx_row = a.topk_idx + row * (int64_t)K;
  // Validated id of entry ce (raw: its Top-K slot when ce < K).
  auto entry_id = [&](int ce, int32_t raw) -> int32_t {
    if (ce >= e_end) return -1;
    if (ce < K) return raw >= 0 && raw < ctx ? raw : -1;
    const int64_t wv = ce - K;
    return wv < n_swa ? (int32_t)(swa_r0 + wv) : -1;
  };
  // Ids of the first two chunks (threads 0..127, one entry each).
  static_assert(2 * kChunk <= kAttnThreads, "one entry per thread");
  const int ce0 = e_begin + (int)threadIdx.x;
  const int32_t ld0 = threadIdx.x < 2 * kChunk && ce0 < e_end && ce0 < K ? idx_row[ce0] : -1;
  // q of all heads (at most 64): its loads follow the ids' and are in flight
  // while the ids are staged; every thread issues the same number (clamped
  // addresses), so waiting for the ids does not wait for them.
  constexpr int QL = (64 * DQK / 4 + kAttnThreads - 1) / kAttnThreads;   // float4 loads per thread
  const float4* qrow = reinterpret_cast<const float4*>(a.q + row * H * (int64_t)DQK);
  const int n4 = H * DQK / 4;
  float4 qv[QL];
#pragma unroll
  for (int u = 0; u < QL; ++u) {
    const int i = (int)threadIdx.x + u * kAttnThreads;
    qv[u] = qrow[i < n4 ? i : n4 - 1];
  }
  if (threadIdx.x < 2 * kChunk) eidc[threadIdx.x / kChunk][threadIdx.x % kChunk] = entry_id(ce0, ld0);

  // q fragments of this wave's 16 heads: lane holds head 16*hg + c16,
  // dims 32*i + 8*g .. +8 of k-step i (the B operand of S^T = K Q^T).
  const int hg = wave & 3, dh = wave >> 2;
  const bool active = 16 * hg < H;
  const int head_b = 16 * hg + c16;
  v8h qf[S::KQ];
  const float sl2 = a.softmax_scale * kLog2e;
  const uint8_t* codes_b = a.kv_codes + b * a.c_bstride;
  const uint8_t* scales_b = a.kv_scales + b * a.s_bstride;
  const uint8_t* sv_b = a.swa_vals ? a.swa_vals + b * a.sv_bstride : nullptr;
  const uint8_t* ss_b = a.swa_scales ? a.swa_scales + b * a.ss_bstride : nullptr;
  __syncthreads();

  // ---- gather: task = (entry e, 32-channel block j), j fastest, so that
  // consecutive lanes read consecutive 16-byte pieces of one row.
  const bool sc_pair = ((reinterpret_cast<uintptr_t>(a.kv_scales) | (uint64_t)a.s_bstride | (uint64_t)a.s_rstride) &
                        1u) == 0;
  RawTask raw[TPT];
  auto gather = [&](int c0, int slot) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = threadIdx.x + u * kAttnThreads;
      raw[u].kind = 0;
      if (task < NTASK) {
        const int e = task / NB;
        // The block's byte offsets are recomputed every chunk (an opaque j):
        // hoisted out of the loop, their 64-bit addresses held registers
        // across it and forced spills.
        int j = task - (task / NB) * NB;
        asm volatile("" : "+v"(j));
        const int ce = c0 + e;
        const int32_t id = ce < e_end ? eidc[slot][e] : -1;
        if (id >= 0 && ce < K) {
          const uint32_t* cp = reinterpret_cast<const uint32_t*>(codes_b + (int64_t)id * a.c_rstride + 16 * j);
          raw[u].w[0] = cp[0]; raw[u].w[1] = cp[1]; raw[u].w[2] = cp[2]; raw[u].w[3] = cp[3];
          const uint8_t* sp = scales_b + (int64_t)id * a.s_rstride + 2 * j;
          raw[u].sc = sc_pair ? (uint32_t)*reinterpret_cast<const uint16_t*>(sp) : (uint32_t)sp[0] | ((uint32_t)sp[1] << 8);
          raw[u].kind = 1u;
        } else if (id >= 0) {
          const uint32_t* vp = reinterpret_cast<const uint32_t*>(sv_b + (int64_t)id * a.sv_rstride + 32 * j);
#pragma unroll
          for (int i = 0; i < 8; ++i) raw[u].w[i] = vp[i];
          raw[u].sc = ss_b[(int64_t)id * a.ss_rstride + j];
          raw[u].kind = 2u;
        }
      }
    }
  };
  // ---- dequantise the staged bytes into fp16 K rows.
  auto store = [&](_Float16* kt) {
    // Every staged word counts as read here, whatever the task's kind, so
    // that no load into these registers is still pending when the next
    // gather overwrites them (the compiler would otherwise wait there,
    // between the gather's own loads).
#pragma unroll
    for (int u = 0; u < TPT; ++u)
      asm volatile("" ::"v"(raw[u].w[0]), "v"(raw[u].w[1]), "v"(raw[u].w[2]), "v"(raw[u].w[3]), "v"(raw[u].w[4]),
                   "v"(raw[u].w[5]), "v"(raw[u].w[6]), "v"(raw[u].w[7]), "v"(raw[u].sc));
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = threadIdx.x + u * kAttnThreads;
      if (task >= NTASK) break;
      const int e = task / NB, j = task - (task / NB) * NB;
      uint32_t hv[16];
      if (raw[u].kind == 1u) {
        // E2M1 -> fp16 in hardware (scale 1), then the E4M3 scale of each
        // 16-channel group as an fp16 multiply; both steps are exact (at most
        // 6 significant bits).
#pragma unroll
        for (int hgp = 0; hgp < 2; ++hgp) {
          const _Float16 sh = (_Float16)e4m3_to_f32((raw[u].sc >> (8 * hgp)) & 0xFFu);
          const v2h s2 = {sh, sh};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t word = raw[u].w[2 * hgp + (i >> 2)];
            v2h v;
            switch (i & 3) {
              case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0); break;
              case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1); break;
              case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2); break;
              default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3); break;
            }
            v = v * s2;
            hv[8 * hgp + i] = __builtin_bit_cast(uint32_t, v);
          }
        }
      } else if (raw[u].kind == 2u) {
        // E4M3 -> fp16 scaled by the E8M0 power of two, in one instruction.
        const float sc = e8m0_to_f32(raw[u].sc);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const uint32_t word = raw[u].w[i >> 1];
          v2h v = (i & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, sc, true)
                          : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, sc, false);
          hv[i] = __builtin_bit_cast(uint32_t, v);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) hv[i] = 0u;
      }
      uint4* dst = reinterpret_cast<uint4*>(kt + e * S::PITCH + 32 * j);
#pragma unroll
      for (int p = 0; p < 4; ++p) dst[p] = uint4{hv[4 * p], hv[4 * p + 1], hv[4 * p + 2], hv[4 * p + 3]};
    }
  };

  // O tiles: wave (ph, dq) owns heads 32*ph .. +31 (two 16-head tiles) and
  // output dims 128*dq .. +127.
  const int ph = wave & 1, dq = wave >> 1;
  const bool pv_active = 32 * ph < H;
  v4f o[2][NT];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) o[t][n] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  // q of all heads through LDS (the second K buffer is free until the first
  // iteration refills it): one fp16 rounding, then each wave reads its B
  // fragments; the first chunk's loads are issued in between.
  {
    _Float16* qs = kbuf[1];
#pragma unroll
    for (int u = 0; u < QL; ++u) {
      const int i = (int)threadIdx.x + u * kAttnThreads;
      if (i < n4) {
        const int h = (4 * i) / DQK, d = 4 * i - h * DQK;
        v2h lo = {(_Float16)qv[u].x, (_Float16)qv[u].y}, hi = {(_Float16)qv[u].z, (_Float16)qv[u].w};
        *reinterpret_cast<uint2*>(qs + h * QP + d) =
            uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
      }
    }
    if (e_begin < e_end) gather(e_begin, 0);
    __syncthreads();
    if (active) {
#pragma unroll
      for (int i = 0; i < S::KQ; ++i) qf[i] = *reinterpret_cast<const v8h*>(qs + head_b * QP + 32 * i + 8 * g);
    }
  }
  if (e_begin < e_end) store(kbuf[0]);
  __syncthreads();
  if (e_begin + kChunk < e_end) gather(e_begin + kChunk, 1);
  int cur = 0, slot = 0;   // kbuf and id slot of the chunk being consumed
  for (int c0 = e_begin; c0 < e_end; c0 += kChunk, cur ^= 1, slot = slot == 2 ? 0 : slot + 1) {
    const bool has_next = c0 + kChunk < e_end;
    const _Float16* kt = kbuf[cur];
    const int slot2 = slot == 0 ? 2 : slot - 1;   // (slot + 2) % 3: the chunk after next
    // Ids of the chunk after next (wave 0), stored before the first barrier.
    const int ce2 = c0 + 2 * kChunk + lane;
    int32_t ld2 = -1;
    if (wave == 0 && ce2 < e_end && ce2 < K) ld2 = idx_row[ce2];
    // ---- S^T = K Q^T for this wave's 2 tiles of 16 entries: entries 32*dh ..
    float z[8];
    float cmax = -__builtin_inff();
    if (active) {
      v4f st[2] = {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}};
      const _Float16* krow0 = kt + (32 * dh + c16) * S::PITCH + 8 * g;
      const _Float16* krow1 = krow0 + 16 * S::PITCH;
      constexpr int BATCH = 6;
#pragma unroll
      for (int i0 = 0; i0 < S::KQ; i0 += BATCH) {
        v8h ka[BATCH], kb[BATCH];
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          if (i0 + j < S::KQ) {
            ka[j] = *reinterpret_cast<const v8h*>(krow0 + 32 * (i0 + j));
            kb[j] = *reinterpret_cast<const v8h*>(krow1 + 32 * (i0 + j));
          }
        }
#pragma unroll
        for (int j = 0; j < BATCH; ++j) {
          if (i0 + j < S::KQ) {
            st[0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[j], qf[i0 + j], st[0], 0, 0, 0);
            st[1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kb[j], qf[i0 + j], st[1], 0, 0, 0);
          }
        }
      }
      // st[t][r] = S^T[entry 32dh + 16t + 4g + r][head c16]
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int ce = c0 + 32 * dh + 16 * t + 4 * g + r;
          bool ok = ce < e_end && eidc[slot][ce - c0] >= 0;
          float v = ok ? st[t][r] * sl2 : -__builtin_inff();
          z[4 * t + r] = v;
          cmax = fmaxf(cmax, v);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      if (g == 0) pmx[dh][16 * hg + c16] = cmax;
    }
    if (wave == 0 && c0 + 2 * kChunk < e_end) eidc[slot2][lane] = entry_id(ce2, ld2);
    __syncthreads();
    float alpha = 1.0f;
    if (active) {
      cmax = fmaxf(cmax, pmx[dh ^ 1][16 * hg + c16]);   // max over the whole 64-entry chunk
      const float m_new = fmaxf(m_run, cmax);
      float psum = 0.0f;
      v8h pa;
      if (m_new == -__builtin_inff()) {
#pragma unroll
        for (int i = 0; i < 8; ++i) pa[i] = (_Float16)0.0f;
      } else {
        alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          float p = __builtin_amdgcn_exp2f(z[i] - m_new);
          psum += p;
          pa[i] = (_Float16)p;
        }
      }
      l_run = l_run * alpha + psum;
      m_run = m_new;
      pex[wave][lane] = pa;
    } else {
      v8h pz;
#pragma unroll
      for (int i = 0; i < 8; ++i) pz[i] = (_Float16)0.0f;
      pex[wave][lane] = pz;
    }
    if (dh == 0 && g == 0) alf[16 * hg + c16] = alpha;
    __syncthreads();
    if (pv_active) {
      // P of head tile t for entries 32j .. (k-step j) was written by the S
      // wave of head group 2*ph + t and entry half j.
      v8h pf[2][2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int j = 0; j < 2; ++j) pf[t][j] = pex[2 * ph + t + 4 * j][lane];
      float4 al[2];
      al[0] = *reinterpret_cast<const float4*>(&alf[32 * ph + 4 * g]);
      al[1] = *reinterpret_cast<const float4*>(&alf[32 * ph + 16 + 4 * g]);
      if (!__all(al[0].x == 1.0f && al[0].y == 1.0f && al[0].z == 1.0f && al[0].w == 1.0f && al[1].x == 1.0f &&
                 al[1].y == 1.0f && al[1].z == 1.0f && al[1].w == 1.0f)) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            o[t][n][0] *= al[t].x; o[t][n][1] *= al[t].y; o[t][n][2] *= al[t].z; o[t][n][3] *= al[t].w;
          }
      }
      // ---- O += P V over dims 128*dq ..; k-step j: entries 32j + {4g..4g+3, 16+4g..16+4g+3}.
      // V is read from the row-major K rows with the LDS transpose read: in each
      // 16-lane group, source lane s names entry (.. + s/4), dims 4(s%4)..+3, and
      // lane i receives dim i of those four entries.  Each V fragment serves both
      // head tiles.
      const int s16 = lane & 15;
      const _Float16* vbase = kt + (4 * g + (s16 >> 2)) * S::PITCH + 128 * dq + 4 * (s16 & 3);
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s* lds_v4s;
      constexpr int VB = 4;
#pragma unroll
      for (int n0 = 0; n0 < NT; n0 += VB) {
        v8h vf[VB][2];
#pragma unroll
        for (int jn = 0; jn < VB; ++jn) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const _Float16* vp = vbase + 32 * j * S::PITCH + 16 * (n0 + jn);
            v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vp));
            v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vp + 16 * S::PITCH));
            vf[jn][j] = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          }
        }
#pragma unroll
        for (int jn = 0; jn < VB; ++jn)
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            o[t][n0 + jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[t][0], vf[jn][0], o[t][n0 + jn], 0, 0, 0);
            o[t][n0 + jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[t][1], vf[jn][1], o[t][n0 + jn], 0, 0, 0);
          }
      }
    }
    // Next chunk into the other buffer (last read one iteration ago), then
    // the loads of the chunk after it.
    if (has_next) {
      store(kbuf[cur ^ 1]);
      if (c0 + 2 * kChunk < e_end) gather(c0 + 2 * kChunk, slot2);
    }
    __syncthreads();
  }

  // ---- partial results: l summed over the 4 lane groups and both dim halves
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (active && g == 0) pmx[dh][16 * hg + c16] = l_tot;
  __syncthreads();
  if (splits == 1) {
    // The row's only split: normalise here, with the combine's operations in
    // its order (O * 2^(m - M), then * 1/L; L = l * 2^(m - M) + 2^(sink - M)),
    // and write out and lse; no partials and no combine launch.
    if (active && g == 0 && dh == 0) {
      l_tot += pmx[1][head_b];
      const float sk = a.sink ? a.sink[head_b] * kLog2e : -__builtin_inff();
      const float M = fmaxf(m_run, sk);
      float w = 0.0f, L = 0.0f;
      if (M != -__builtin_inff()) {
        if (m_run != -__builtin_inff()) {
          w = __builtin_amdgcn_exp2f(m_run - M);
          L += l_tot * w;
        }
        if (sk != -__builtin_inff()) L += __builtin_amdgcn_exp2f(sk - M);
      }
      pmx[0][head_b] = w;
      pmx[1][head_b] = L > 0.0f ? 1.0f / L : 0.0f;
      if (a.lse) a.lse[row * H + head_b] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
    }
    __syncthreads();
    if (!pv_active) return;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      if (32 * ph + 16 * t >= H) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 32 * ph + 16 * t + 4 * g + r;
        const float w = pmx[0][h], inv = pmx[1][h];
#pragma unroll
        for (int n = 0; n < NT; ++n) a.out[(row * H + h) * DV + 128 * dq + 16 * n + c16] = (o[t][n][r] * w) * inv;
      }
    }
    return;
  }
  const int64_t pbase = (row * splits + split) * (int64_t)H;
  if (active && g == 0 && dh == 0) {
    l_tot += pmx[1][16 * hg + c16];
    part_ml[(pbase + head_b) * 2 + 0] = m_run;
    part_ml[(pbase + head_b) * 2 + 1] = l_tot;
  }
  if (!pv_active) return;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    if (32 * ph + 16 * t >= H) break;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 32 * ph + 16 * t + 4 * g + r;
        part_o[(pbase + h) * DV + 128 * dq + 16 * n + c16] = o[t][n][r];
      }
  }
}

// Merge split partials: out = sum_s O_s 2^(m_s - M) / L, L = sum_s l_s 2^(m_s - M)
// (+ 2^(sink*log2e - M)), lse = (M + log2 L) ln 2.  One workgroup per
// (row, head): the split maxima are reduced in parallel, then each thread
// accumulates its four output dims over the splits in ascending order with
// the loads of up to sixteen splits in flight.
template <int DV>
__global__ void __launch_bounds__(128)
sparse_attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits, int H,
                           const float* __restrict__ sink, float* __restrict__ out, float* __restrict__ lse) {
  static_assert(DV == 4 * 128, "one float4 of output dims per thread");
  __shared__ float red[2];
  const int64_t rh = blockIdx.x;            // row * H + h
  const int h = (int)(rh % H);
  const int64_t row = rh / H;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float sk = sink ? sink[h] * kLog2e : -__builtin_inff();
  const float* mlb = part_ml + (row * splits * (int64_t)H + h) * 2;   // split s at mlb[2 * s * H]
  float mx = -__builtin_inff();
  for (int sp = threadIdx.x; sp < splits; sp += 128) mx = fmaxf(mx, mlb[2 * (int64_t)sp * H]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  if (lane == 0) red[wave] = mx;
  __syncthreads();
  const float M = fmaxf(fmaxf(red[0], red[1]), sk);
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
  if (M != -__builtin_inff()) {
    const float4* ob = reinterpret_cast<const float4*>(part_o + (row * splits * (int64_t)H + h) * DV) + threadIdx.x;
    // Batches of U splits with all their loads in flight (U no larger than
    // needed: padding loads are issue slots too), in ascending split order.
    auto run = [&](auto u_tag) {
      constexpr int U = decltype(u_tag)::value;
      for (int s0 = 0; s0 < splits; s0 += U) {
        float2 ml[U];
        float4 ov[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const int sp = s0 + u < splits ? s0 + u : splits - 1;
          ml[u] = *reinterpret_cast<const float2*>(mlb + 2 * (int64_t)sp * H);
          ov[u] = ob[(int64_t)sp * H * (DV / 4)];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          if (s0 + u >= splits || ml[u].x == -__builtin_inff()) continue;
          const float wgt = __builtin_amdgcn_exp2f(ml[u].x - M);
          L += ml[u].y * wgt;
          acc.x += ov[u].x * wgt; acc.y += ov[u].y * wgt; acc.z += ov[u].z * wgt; acc.w += ov[u].w * wgt;
        }
      }
    };
    if (splits <= 2) run(std::integral_constant<int, 2>{});
    else if (splits <= 4) run(std::integral_constant<int, 4>{});
    else if (splits <= 8) run(std::integral_constant<int, 8>{});
    else run(std::integral_constant<int, 16>{});
    if (sk != -__builtin_inff()) L += __builtin_amdgcn_exp2f(sk - M);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  reinterpret_cast<float4*>(out + rh * DV)[threadIdx.x] = float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv};
  if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

int attn_num_splits(int64_t rows, int k_top, int W) {
  // One resident workgroup per compute unit (LDS and registers allow one).
  int E = k_top + W;
  int max_splits = (E + 63) / 64;
  int64_t want = ((int64_t)device_cu_count() + rows - 1) / rows;
  int s = (int)(want < 1 ? 1 : (want > max_splits ? max_splits : want));
  return s < 1 ? 1 : s;
}

size_t attn_ws_bytes(int64_t rows, int H, int d_v, int splits) {
  size_t po = sizeof(float) * (size_t)rows * splits * H * d_v;
  size_t pm = sizeof(float) * (size_t)rows * splits * H * 2;
  return ((po + 255) & ~(size_t)255) + ((pm + 255) & ~(size_t)255);
}

template <int DQK, int DV>
static hipError_t launch_attn_t(const AttnArgs& a, bool prefill, void* ws, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * a.Tq;
  const int splits = attn_num_splits(rows, a.k_top, a.W);
  const int E = a.k_top + a.W;
  int span = (E + splits - 1) / splits;
  span = (span + kChunk - 1) / kChunk * kChunk;
  const int real_splits = (E + span - 1) / span;
  size_t po = sizeof(float) * (size_t)rows * real_splits * a.H * DV;
  float* part_o = (float*)ws;
  float* part_ml = (float*)((char*)ws + ((po + 255) & ~(size_t)255));
  CSA2_LAUNCH("sparse_attn_split", (sparse_attn_split_kernel<DQK, DV>), dim3(real_splits, (unsigned)rows),
              dim3(kAttnThreads), 0, s, a, prefill ? 1 : 0, real_splits, span, part_o, part_ml);
  if (real_splits > 1)   // (a single split normalises and writes the output itself)
    CSA2_LAUNCH("sparse_attn_combine", (sparse_attn_combine_kernel<DV>), dim3((unsigned)(rows * a.H)), dim3(128), 0,
                s, part_o, part_ml, real_splits, a.H, a.sink, a.out, a.lse);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs& a, bool prefill, void* ws, hipStream_t s) {
  if (a.d_qk == 576 && a.d_v == 512) return launch_attn_t<576, 512>(a, prefill, ws, s);
  if (a.d_qk == 512 && a.d_v == 512) return launch_attn_t<512, 512>(a, prefill, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace csa2
