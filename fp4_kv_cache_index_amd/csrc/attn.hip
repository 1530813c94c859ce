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
// its entry list (Top-K rows, then the window rows).  Its 8 waves (two per
// SIMD) form 4 head groups of 16 heads; the two waves of a head group own
// one half each of the 64 entries of a chunk for S and one half each of the
// 512 output dims for O (64 fp32 accumulator registers per lane).  Chunks of
// 64 entries are double-buffered in LDS as fp16 rows: while a chunk is
// consumed, the next one is dequantised into the other buffer and the rows
// of the one after it are in flight.  The rows are gathered by index and
// dequantised with the gfx950 scaled converts (v_cvt_scalef32_pk_f16_fp4 /
// _fp8, which apply the power-of-two part of their scale; the E4M3 scale of
// a main row is applied as an fp16 multiply) -- exact, since E2M1 x E4M3 has
// at most 6 significant bits within [2^-10, 2688] -- and then
//   S^T = K Q^T   on v_mfma_f32_16x16x32_f16 (q rounded to fp16 once), each
//                 wave for its 32 entries,
//   online softmax in fp32 (exp2 domain); the wave pair exchanges row maxima
//                 and its P fragments through LDS,
//   O  += P V     on the same instruction, P taken straight from the S^T
//                 accumulators (their lane layout is the A-operand layout of
//                 P once the k index is permuted identically for V), and V
//                 read from the same fp16 rows with the LDS transpose read
//                 (ds_read_b64_tr_b16), so no transposed copy is stored.
// Splits write unnormalised partial (O, m, l); a combine kernel merges them
// with the log-sum-exp rule and adds the sink.
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

constexpr int kMaxSpan = 640;       // entries per split (ids staged in LDS)
constexpr int kAttnThreads = 512;   // 8 waves; wave w: heads 16*(w&3).., output dims 256*(w>>2)..

// Raw bytes of one gather task: two entries (2*ep, 2*ep+1) of one 16-channel group.
struct RawTask {
  uint32_t w[2][4];   // main: 8 code bytes in w[k][0..1]; window: 16 value bytes
  uint32_t sc[2];     // scale byte (E4M3 for main rows, E8M0 for window rows)
  uint32_t kind;      // 2 bits per entry: 0 skip, 1 main, 2 window
};

template <int DQK, int DV>
__global__ void __launch_bounds__(kAttnThreads)
sparse_attn_split_kernel(AttnArgs a, int prefill, int splits, int span,
                         float* __restrict__ part_o, float* __restrict__ part_ml) {
  using S = AttnShape<DQK>;
  constexpr int NT = DV / 32;                         // output tiles per wave (half the dims)
  constexpr int NTASK = (kChunk / 2) * S::G16;        // (entry pair, group) tasks per chunk
  constexpr int NEP = kChunk / 2;                     // entry pairs per chunk
  constexpr int TPT = (NTASK + kAttnThreads - 1) / kAttnThreads;
  __shared__ __attribute__((aligned(16))) _Float16 kbuf[2][kChunk * S::PITCH];   // K rows, row-major, 2 chunks
  __shared__ int32_t eid[kMaxSpan];   // main: token id; window: window row; -1 = skip
  __shared__ float pmx[2][64];        // per-head partial maxima / sums of the two dim halves
  __shared__ __attribute__((aligned(16))) v8h pex[8][64];   // P fragments exchanged between wave pairs

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c16 = lane & 15, g = lane >> 4;
  const int64_t row = blockIdx.y;
  const int split = blockIdx.x;
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
  for (int e = e_begin + threadIdx.x; e < e_end; e += kAttnThreads) {
    int32_t v = -1;
    if (e < K) {
      int64_t id = idx_row[e];
      if (id >= 0 && id < ctx) v = (int32_t)id;
    } else {
      int64_t wv = e - K;
      if (wv < n_swa) v = (int32_t)(swa_r0 + wv);
    }
    eid[e - e_begin] = v;
  }

  // q fragments of this wave's 16 heads: lane holds head 16*wave + c16,
  // dims 32*i + 8*g .. +8 of k-step i (the B operand of S^T = K Q^T).
  const int hg = wave & 3, dh = wave >> 2;
  const bool active = 16 * hg < H;
  const int head_b = 16 * hg + c16;
  v8h qf[S::KQ];
  if (active) {
    const float* qrow = a.q + (row * H + head_b) * (int64_t)DQK;
#pragma unroll
    for (int i = 0; i < S::KQ; ++i) qf[i] = load_f32x8_as_f16(qrow + 32 * i + 8 * g);
  }
  const float sl2 = a.softmax_scale * kLog2e;
  const uint8_t* codes_b = a.kv_codes + b * a.c_bstride;
  const uint8_t* scales_b = a.kv_scales + b * a.s_bstride;
  const uint8_t* sv_b = a.swa_vals ? a.swa_vals + b * a.sv_bstride : nullptr;
  const uint8_t* ss_b = a.swa_scales ? a.swa_scales + b * a.ss_bstride : nullptr;
  __syncthreads();

  // ---- gather: task = (entry pair ep, 16-channel group gq), ep fastest so
  // that a wave's V^T stores hit consecutive words.
  RawTask raw[TPT];
  auto gather = [&](int c0) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = threadIdx.x + u * kAttnThreads;
      raw[u].kind = 0;
      if (task < NTASK) {
        const int ep = task % NEP, gq = task / NEP;
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          const int ce = c0 + 2 * ep + k;
          const int32_t id = ce < e_end ? eid[ce - e_begin] : -1;
          if (id >= 0 && ce < K) {
            const uint32_t* cp = reinterpret_cast<const uint32_t*>(codes_b + (int64_t)id * a.c_rstride + 8 * gq);
            raw[u].w[k][0] = cp[0];
            raw[u].w[k][1] = cp[1];
            raw[u].sc[k] = scales_b[(int64_t)id * a.s_rstride + gq];
            raw[u].kind |= 1u << (2 * k);
          } else if (id >= 0) {
            const uint32_t* vp = reinterpret_cast<const uint32_t*>(sv_b + (int64_t)id * a.sv_rstride + 16 * gq);
            raw[u].w[k][0] = vp[0]; raw[u].w[k][1] = vp[1]; raw[u].w[k][2] = vp[2]; raw[u].w[k][3] = vp[3];
            raw[u].sc[k] = ss_b[(int64_t)id * a.ss_rstride + (gq >> 1)];
            raw[u].kind |= 2u << (2 * k);
          }
        }
      }
    }
  };
  // ---- dequantise the staged bytes into K rows and V^T columns.
  auto store = [&](_Float16* kt) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = threadIdx.x + u * kAttnThreads;
      if (task >= NTASK) break;
      const int ep = task % NEP, gq = task / NEP;
      uint32_t hv[2][8];
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint32_t kind = (raw[u].kind >> (2 * k)) & 3u;
        if (kind == 1u) {
          // E2M1 -> fp16 in hardware (scale 1), then the E4M3 scale as an fp16
          // multiply; both steps are exact (at most 6 significant bits).
          _Float16 sh = (_Float16)e4m3_to_f32(raw[u].sc[k]);
          v2h s2 = {sh, sh};
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t word = raw[u].w[k][i >> 2];
            v2h v;
            switch (i & 3) {
              case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 0); break;
              case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 1); break;
              case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 2); break;
              default: v = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(word, 1.0f, 3); break;
            }
            v = v * s2;
            hv[k][i] = __builtin_bit_cast(uint32_t, v);
          }
        } else if (kind == 2u) {
          // E4M3 -> fp16 scaled by the E8M0 power of two, in one instruction.
          const float sc = e8m0_to_f32(raw[u].sc[k]);
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const uint32_t word = raw[u].w[k][i >> 1];
            v2h v = (i & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, sc, true)
                            : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(word, sc, false);
            hv[k][i] = __builtin_bit_cast(uint32_t, v);
          }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) hv[k][i] = 0u;
        }
        uint4* dst = reinterpret_cast<uint4*>(kt + (2 * ep + k) * S::PITCH + 16 * gq);
        dst[0] = uint4{hv[k][0], hv[k][1], hv[k][2], hv[k][3]};
        dst[1] = uint4{hv[k][4], hv[k][5], hv[k][6], hv[k][7]};
      }
    }
  };

  v4f o[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) o[n] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -__builtin_inff();
  float l_run = 0.0f;

  if (e_begin < e_end) {
    gather(e_begin);
    store(kbuf[0]);
  }
  __syncthreads();
  if (e_begin + kChunk < e_end) gather(e_begin + kChunk);
  int cur = 0;
  for (int c0 = e_begin; c0 < e_end; c0 += kChunk, cur ^= 1) {
    const bool has_next = c0 + kChunk < e_end;
    const _Float16* kt = kbuf[cur];
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
          bool ok = ce < e_end && eid[ce - e_begin] >= 0;
          float v = ok ? st[t][r] * sl2 : -__builtin_inff();
          z[4 * t + r] = v;
          cmax = fmaxf(cmax, v);
        }
      cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
      cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
      if (g == 0) pmx[dh][16 * hg + c16] = cmax;
    }
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
    }
    __syncthreads();
    if (active) {
      // P for entries 0..31 (k-step 0) comes from dim half 0, 32..63 from half 1.
      const v8h p_own = pex[wave][lane], p_oth = pex[wave ^ 4][lane];
      const v8h p0 = dh == 0 ? p_own : p_oth, p1 = dh == 0 ? p_oth : p_own;
      if (!__all(alpha == 1.0f)) {
        float al[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) al[r] = __shfl(alpha, 4 * g + r, 64);
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          o[n][0] *= al[0]; o[n][1] *= al[1]; o[n][2] *= al[2]; o[n][3] *= al[3];
        }
      }
      // ---- O += P V over dims 256*dh ..; k-step j: entries 32j + {4g..4g+3, 16+4g..16+4g+3}.
      // V is read from the row-major K rows with the LDS transpose read: in each
      // 16-lane group, source lane s names entry (.. + s/4), dims 4(s%4)..+3, and
      // lane i receives dim i of those four entries.
      const int s16 = lane & 15;
      const _Float16* vbase = kt + (4 * g + (s16 >> 2)) * S::PITCH + 256 * dh + 4 * (s16 & 3);
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
        for (int jn = 0; jn < VB; ++jn) {
          o[n0 + jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p0, vf[jn][0], o[n0 + jn], 0, 0, 0);
          o[n0 + jn] = __builtin_amdgcn_mfma_f32_16x16x32_f16(p1, vf[jn][1], o[n0 + jn], 0, 0, 0);
        }
      }
    }
    // Next chunk into the other buffer (last read one iteration ago), then
    // the loads of the chunk after it.
    if (has_next) {
      store(kbuf[cur ^ 1]);
      if (c0 + 2 * kChunk < e_end) gather(c0 + 2 * kChunk);
    }
    __syncthreads();
  }

  // ---- partial results: l summed over the 4 lane groups and both dim halves
  float l_tot = l_run;
  l_tot += __shfl_xor(l_tot, 16, 64);
  l_tot += __shfl_xor(l_tot, 32, 64);
  if (active && g == 0) pmx[dh][16 * hg + c16] = l_tot;
  __syncthreads();
  if (!active) return;
  l_tot += pmx[dh ^ 1][16 * hg + c16];
  const int64_t pbase = (row * splits + split) * (int64_t)H;
  if (g == 0 && dh == 0) {
    part_ml[(pbase + head_b) * 2 + 0] = m_run;
    part_ml[(pbase + head_b) * 2 + 1] = l_tot;
  }
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      int h = 16 * hg + 4 * g + r;
      part_o[(pbase + h) * DV + 256 * dh + 16 * n + c16] = o[n][r];
    }
}

// Merge split partials: out = sum_s O_s 2^(m_s - M) / L, L = sum_s l_s 2^(m_s - M)
// (+ 2^(sink*log2e - M)), lse = (M + log2 L) ln 2.
template <int DV>
__global__ void __launch_bounds__(128)
sparse_attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits, int H,
                           const float* __restrict__ sink, float* __restrict__ out, float* __restrict__ lse) {
  const int64_t rh = blockIdx.x;            // row * H + h
  const int h = (int)(rh % H);
  const int64_t row = rh / H;
  float M = -__builtin_inff();
  const float sk = sink ? sink[h] * kLog2e : -__builtin_inff();
  for (int s = 0; s < splits; ++s) {
    float m = part_ml[((row * splits + s) * H + h) * 2];
    M = fmaxf(M, m);
  }
  M = fmaxf(M, sk);
  float L = 0.0f;
  float acc[DV / 128];
#pragma unroll
  for (int i = 0; i < DV / 128; ++i) acc[i] = 0.0f;
  if (M != -__builtin_inff()) {
    for (int s = 0; s < splits; ++s) {
      const int64_t pi = (row * splits + s) * H + h;
      float m = part_ml[pi * 2];
      if (m == -__builtin_inff()) continue;
      float wgt = __builtin_amdgcn_exp2f(m - M);
      L += part_ml[pi * 2 + 1] * wgt;
#pragma unroll
      for (int i = 0; i < DV / 128; ++i) acc[i] += part_o[pi * DV + threadIdx.x + 128 * i] * wgt;
    }
    if (sk != -__builtin_inff()) L += __builtin_amdgcn_exp2f(sk - M);
  }
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
#pragma unroll
  for (int i = 0; i < DV / 128; ++i) out[rh * DV + threadIdx.x + 128 * i] = acc[i] * inv;
  if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

int attn_num_splits(int64_t rows, int k_top, int W) {
  // One resident workgroup per compute unit (LDS and registers allow one).
  int E = k_top + W;
  int max_splits = (E + 63) / 64;
  int min_splits = (E + kMaxSpan - 1) / kMaxSpan;
  int64_t want = ((int64_t)device_cu_count() + rows - 1) / rows;
  int s = (int)(want < 1 ? 1 : (want > max_splits ? max_splits : want));
  if (s < min_splits) s = min_splits;
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
