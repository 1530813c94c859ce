// Sparse MLA attention over the Top-K FP4 main-KV rows plus the FP8 window.
//
// What it computes (DeepSeek-V4.1-Flash techniques map, "Checked in its
// code": multi-head latent attention with one latent KV head, and one
// trainable logit per head that enters only the softmax normaliser; fact
// sheet: one shared K=V entry per token, a 128-token window per layer; blog,
// CSA2 paragraph: attention runs over the indexer's Top-K entries of the FP4
// main cache): for each query row and head h, softmax over the selected
// entries (and the sink) of scale * q_h . k_e, applied to v_e = the first
// d_v channels of the same row.
//
// gfx950 mapping.  A workgroup holds one query row and a contiguous split of
// its entry list (Top-K rows, then the window rows); workgroups are numbered
// so that the splits of one row land on the same XCD and share its q in L2.
// Its 8 waves take two roles.  Chunks of 32 entries pass through three fp16
// K-row buffers in LDS: in iteration i the four S waves score chunk i, the
// four PV waves accumulate chunk i-1, and every wave dequantises its share of
// chunk i+1 (gathered into registers one iteration earlier) and issues the
// loads of chunk i+2; one barrier per iteration.  The PV waves dequantise
// before their products and the S waves after theirs, so that one role's
// VALU work overlaps the other's matrix products.  A gather task is one
// entry's 32-channel block, consecutive lanes taking consecutive 16-byte
// pieces of a row; the rows are dequantised with the gfx950 scaled converts
// (v_cvt_scalef32_pk_f16_fp4 / _fp8, which apply the power-of-two part of
// their scale; the E4M3 scales of a main row are converted to fp16 by the
// fp8 convert and applied as an fp16 multiply) -- exact, since E2M1 x E4M3
// has at most 6 significant bits within [2^-10, 2688].  q is read once per
// workgroup with coalesced loads, rounded to fp16 once and passed through
// LDS into the S waves' registers.  Per chunk,
//   S^T = K Q^T   on v_mfma_f32_16x16x32_f16: S wave w holds heads 16w .. +15
//                 (q in registers) and scores all 32 entries (two tiles of
//                 16), its K fragment reads running ahead of the products;
//   online softmax in fp32 (exp2 domain) with a lazily moved reference
//                 maximum: it moves only when a chunk exceeds it by more
//                 than 2^8 (log2 units), so P stays below 256, exact to
//                 fp16's relative precision, and O is rarely rescaled; P
//                 fragments and per-head rescale factors go to LDS;
//   O  += P V     on the same instruction: PV wave d holds all heads (four
//                 16-head tiles, 128 fp32 accumulator registers per lane) and
//                 output dims 128d .. +127, so every V fragment serves four
//                 head tiles.  P keeps the lane layout of the S^T
//                 accumulators (the A-operand layout once the k index is
//                 permuted identically for V), and V is read from the same
//                 fp16 rows with the LDS transpose read (ds_read_b64_tr_b16),
//                 so no transposed copy is stored.
// Splits write unnormalised partial (O, m, l); a combine kernel merges them
// with the log-sum-exp rule and adds the sink.  A row with a single split
// (4096-query prefill chunks) is normalised by the split kernel itself.

#include "common.h"
#include "internal.h"

namespace csa2 {

constexpr int kChunk = 32;           // entries per LDS chunk
constexpr float kLazy = 8.0f;        // move threshold of the reference maximum (log2 units)
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

// PAGED: main rows live in a page pool; a Top-K token id is translated to its
// pool row (block-table page, offset in the page) when the entry ids are
// staged, one iteration before the gather reads them.
template <int DQK, int DV, bool PAGED>
__global__ void __launch_bounds__(kAttnThreads)
sparse_attn_split_kernel(AttnArgs a, int prefill, int splits, int span,
                         float* __restrict__ part_o, float* __restrict__ part_ml) {
  using S = AttnShape<DQK>;
  constexpr int NT = DV / 64;                         // 16-dim output tiles per PV wave (a quarter of the dims)
  constexpr int NB = DQK / 32;                        // 32-channel blocks per row
  constexpr int NTASK = kChunk * NB;                  // (entry, block) tasks per chunk
  constexpr int QP = DQK + 8;                         // fp16 pitch of the staged q rows
  static_assert(64 * QP <= 2 * kChunk * S::PITCH, "q staging must fit two K buffers");
  constexpr int TPT = (NTASK + kAttnThreads - 1) / kAttnThreads;
  // K rows of three chunks: the one the S waves read, the one the PV waves
  // read as V, the one being dequantised.
  __shared__ __attribute__((aligned(16))) _Float16 kbuf[3][kChunk * S::PITCH];
  // Entry ids of four chunks (main: token id; window: window row; -1 = skip).
  __shared__ __attribute__((aligned(16))) int32_t eidc[4][kChunk];
  __shared__ __attribute__((aligned(16))) v8h pex[2][4][64];   // P fragments of the 4 S waves, 2 chunks
  __shared__ __attribute__((aligned(16))) float alf[2][64];     // per-head rescale factor, 2 chunks
  __shared__ __attribute__((aligned(16))) uint32_t mvf[2][4];   // per S wave: some factor is not 1, 2 chunks
  __shared__ float pml[2][64];                                  // epilogue: per-head (w, 1/L)

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
  const int64_t ring = a.swa_ring;
  if (ring > 0) {
    // Ring window: position x at row x % ring; the ring holds positions
    // swa_end - ring .. swa_end - 1.  The query at p sees the window
    // positions max(p - W + 1, swa_end - ring, 0) .. min(p, swa_end - 1).
    const int64_t p = a.q_pos ? (int64_t)a.q_pos[row] : ctx - 1;
    const int64_t end = a.swa_end[b];
    int64_t lo = p - a.W + 1;
    if (end - ring > lo) lo = end - ring;
    if (lo < 0) lo = 0;
    const int64_t hi = p < end - 1 ? p : end - 1;
    swa_r0 = lo;                      // first position
    n_swa = hi >= lo ? hi - lo + 1 : 0;
  } else if (prefill) {
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
    if (wv >= n_swa) return -1;
    return ring > 0 ? (int32_t)((swa_r0 + wv) % ring) : (int32_t)(swa_r0 + wv);
  };
  // Paged main rows: the block-table entry of a token (a load from a
  // clamped, in-range address) and the pool row it names; a token past the
  // block table or on a missing page (entry < 0 or >= n_pages) is skipped.
  const int32_t* bt_row = PAGED ? a.block_table + b * a.bt_stride : nullptr;
  auto page_of = [&](int ce, int32_t id) -> int32_t {
    const bool m = ce < K && id >= 0 && (int64_t)(id >> a.page_shift) < a.bt_stride;
    return bt_row[m ? (id >> a.page_shift) : 0];
  };
  auto pool_row = [&](int ce, int32_t id, int32_t pg) -> int32_t {
    if (ce >= K || id < 0) return id;   // window rows and skipped entries
    if ((int64_t)(id >> a.page_shift) >= a.bt_stride || pg < 0 || pg >= a.n_pages) return -1;
    return (pg << a.page_shift) | (id & ((1 << a.page_shift) - 1));
  };
  // Ids of the first three chunks (one entry per thread).
  static_assert(3 * kChunk <= kAttnThreads, "one entry per thread");
  const int ce0 = e_begin + (int)threadIdx.x;
  const int32_t ld0 = threadIdx.x < 3 * kChunk && ce0 < e_end && ce0 < K ? idx_row[ce0] : -1;
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
  if constexpr (PAGED) {
    if (threadIdx.x < 3 * kChunk) {
      const int32_t v0 = entry_id(ce0, ld0);
      eidc[threadIdx.x / kChunk][threadIdx.x % kChunk] = pool_row(ce0, v0, page_of(ce0, v0));
    }
  } else {
    if (threadIdx.x < 3 * kChunk) eidc[threadIdx.x / kChunk][threadIdx.x % kChunk] = entry_id(ce0, ld0);
  }

  // Roles: waves 0..3 are S waves (16 heads each, every entry of a chunk),
  // waves 4..7 PV waves (every head, a quarter of the output dims each).
  const bool s_wave = wave < 4;
  const int hg = wave & 3;
  const bool active = s_wave && 16 * hg < H;
  const int head_b = 16 * hg + c16;
  const float sl2 = a.softmax_scale * kLog2e;
  const uint8_t* codes_b = a.kv_codes + b * a.c_bstride;
  const uint8_t* scales_b = a.kv_scales + b * a.s_bstride;
  const uint8_t* sv_b = a.swa_vals ? a.swa_vals + b * a.sv_bstride : nullptr;
  const uint8_t* ss_b = a.swa_scales ? a.swa_scales + b * a.ss_bstride : nullptr;
  __syncthreads();

  const bool sc_pair = ((reinterpret_cast<uintptr_t>(a.kv_scales) | (uint64_t)a.s_bstride | (uint64_t)a.s_rstride) &
                        1u) == 0;
  // ---- gather: task = (entry e, 32-channel block j), j fastest, so that
  // consecutive lanes read consecutive 16-byte pieces of one row.
  RawTask raw[TPT];
  // Entry ids of this thread's tasks in chunk c0 (ring slot `slot`; -1 past
  // the split).  Read apart from the gather, at the top of an iteration, so
  // that the LDS round trip passes under that iteration's other work.
  auto task_ids = [&](int c0, int slot, int32_t(&idv)[TPT]) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = threadIdx.x + u * kAttnThreads;
      const int e = task < NTASK ? task / NB : 0;
      const int32_t v = eidc[slot][e];
      idv[u] = task < NTASK && c0 + e < e_end ? v : -1;
    }
  };
  auto gather_ids = [&](int c0, const int32_t(&idv)[TPT]) {
#pragma unroll
    for (int u = 0; u < TPT; ++u) {
      const int task = threadIdx.x + u * kAttnThreads;
      // A skipped task stages zero words: the main-row conversion turns
      // them into +0 halves, so the dequantisation has no third path.
      raw[u].kind = 0;
      raw[u].w[0] = 0u; raw[u].w[1] = 0u; raw[u].w[2] = 0u; raw[u].w[3] = 0u;
      raw[u].sc = 0u;
      if (task < NTASK) {
        const int e = task / NB;
        // The block's byte offsets are recomputed every chunk (an opaque j):
        // hoisted out of the loop, their 64-bit addresses held registers
        // across it and forced spills.
        int j = task - (task / NB) * NB;
        asm volatile("" : "+v"(j));
        const int ce = c0 + e;
        const int32_t id = idv[u];
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
  auto gather = [&](int c0, int slot) {
    int32_t idv[TPT];
    task_ids(c0, slot, idv);
    gather_ids(c0, idv);
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
      if (raw[u].kind == 2u) {
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
        // A main row, or a skipped task (zero words: +0 halves).
        // E2M1 -> fp16 in hardware (scale 1), then the E4M3 scale of each
        // 16-channel group (converted to fp16 by the fp8 convert) as an fp16
        // multiply; every step is exact (at most 6 significant bits).
        const v2h sc2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[u].sc, 1.0f, false);
#pragma unroll
        for (int hgp = 0; hgp < 2; ++hgp) {
          const v2h s2 = hgp ? __builtin_shufflevector(sc2, sc2, 1, 1) : __builtin_shufflevector(sc2, sc2, 0, 0);
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
      }
      uint4* dst = reinterpret_cast<uint4*>(kt + e * S::PITCH + 32 * j);
#pragma unroll
      for (int p = 0; p < 4; ++p) dst[p] = uint4{hv[4 * p], hv[4 * p + 1], hv[4 * p + 2], hv[4 * p + 3]};
    }
  };

  const int nch = e_end > e_begin ? (e_end - e_begin + kChunk - 1) / kChunk : 0;
  // Dequantise chunk it+1 into the buffer last read as V one iteration ago,
  // then issue the loads of chunk it+2 (every wave takes a share).
  auto advance = [&](int it, int c0, int kb_next, const int32_t(&idn)[TPT]) {
    if (it + 1 < nch) {
      store(kbuf[kb_next]);
      if (it + 2 < nch) gather_ids(c0 + 2 * kChunk, idn);
    }
  };

  // q of all heads through LDS (buffers 1 and 2 are free until the first
  // iterations refill them), rounded to fp16 once; the first chunk's loads
  // are issued before the wait for q.
  _Float16* qs = kbuf[1];
  if (nch > 0) gather(e_begin, 0);
  // Rotary channels of q rotated forward by the query position's angles
  // (fused RoPE of the pages' attention step), pairs (2i, 2i+1), in float32
  // before the fp16 rounding.
  const int r0 = DQK - a.rope_dim;
  const float* cs_row = a.rope_cs ? a.rope_cs + row * (int64_t)a.rope_dim : nullptr;
#pragma unroll
  for (int u = 0; u < QL; ++u) {
    const int i = (int)threadIdx.x + u * kAttnThreads;
    if (i < n4) {
      const int h = (4 * i) / DQK, d = 4 * i - h * DQK;
      if (a.rope_q && cs_row && d >= r0) {
        const float4 cs = *reinterpret_cast<const float4*>(cs_row + (d - r0));   // (cos, sin) of two pairs
        const float x0 = qv[u].x, y0 = qv[u].y, x1 = qv[u].z, y1 = qv[u].w;
        qv[u].x = x0 * cs.x - y0 * cs.y;
        qv[u].y = x0 * cs.y + y0 * cs.x;
        qv[u].z = x1 * cs.z - y1 * cs.w;
        qv[u].w = x1 * cs.w + y1 * cs.z;
      }
      v2h lo = {(_Float16)qv[u].x, (_Float16)qv[u].y}, hi = {(_Float16)qv[u].z, (_Float16)qv[u].w};
      *reinterpret_cast<uint2*>(qs + h * QP + d) =
          uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
    }
  }
  __syncthreads();

  // Iteration it: S waves score chunk it, PV waves accumulate chunk it-1,
  // every wave dequantises part of chunk it+1 and issues the loads of chunk
  // it+2; one barrier per iteration.  The two roles run separate copies of
  // the loop, so that each holds only its own state in registers.
  if (s_wave) {
    // ================================================================ S waves
    // Read by every S wave, active or not (rows past H are staged space,
    // never used): with the read under a branch, the compiler could not rule
    // out that these registers still awaited the q loads of the prologue and
    // made the products wait for every global load in flight, the next
    // chunk's gather included.
    v8h qf[S::KQ];
#pragma unroll
    for (int i = 0; i < S::KQ; ++i) qf[i] = *reinterpret_cast<const v8h*>(qs + head_b * QP + 32 * i + 8 * g);
    float m_run = -__builtin_inff();
    float l_run = 0.0f;
    if (nch > 0) store(kbuf[0]);
    if (nch > 1) gather(e_begin + kChunk, 1);
    __syncthreads();
    int kb = 0;
    for (int it = 0; it <= nch; ++it) {
      const int c0 = e_begin + it * kChunk;
      const int pb = it & 1;
      const int kb_next = kb == 2 ? 0 : kb + 1;
      int32_t idn[TPT];
      if (it + 2 < nch) task_ids(c0 + 2 * kChunk, (it + 2) & 3, idn);
      if (it < nch) {
        const _Float16* kt = kbuf[kb];
        float z[8];
        float cmax = -__builtin_inff();
        if (active) {
          // Two accumulator chains per entry tile (even / odd k-steps), and
          // the K fragment reads kept KA ahead of the products consuming them.
          v4f sa[2][2] = {{v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}},
                          {v4f{0.f, 0.f, 0.f, 0.f}, v4f{0.f, 0.f, 0.f, 0.f}}};
          const _Float16* krow0 = kt + c16 * S::PITCH + 8 * g;
          const _Float16* krow1 = krow0 + 16 * S::PITCH;
          v8h ka[S::KQ], kc[S::KQ];
#pragma unroll
          for (int i = 0; i < S::KQ; ++i) {
            ka[i] = *reinterpret_cast<const v8h*>(krow0 + 32 * i);
            kc[i] = *reinterpret_cast<const v8h*>(krow1 + 32 * i);
          }
#pragma unroll
          for (int i = 0; i < S::KQ; ++i) {
            sa[0][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ka[i], qf[i], sa[0][i & 1], 0, 0, 0);
            sa[1][i & 1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kc[i], qf[i], sa[1][i & 1], 0, 0, 0);
          }
          constexpr int KA = 12;
          __builtin_amdgcn_sched_group_barrier(0x100, KA, 0);
#pragma unroll
          for (int i = 0; i < 2 * S::KQ - KA; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          __builtin_amdgcn_sched_group_barrier(0x008, KA, 0);
          v4f st[2];
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) st[t][r] = sa[t][0][r] + sa[t][1][r];
          // st[t][r] = S^T[entry 16t + 4g + r][head c16]
          const int4 id0 = *reinterpret_cast<const int4*>(&eidc[it & 3][4 * g]);
          const int4 id1 = *reinterpret_cast<const int4*>(&eidc[it & 3][16 + 4 * g]);
          const int idv[8] = {id0.x, id0.y, id0.z, id0.w, id1.x, id1.y, id1.z, id1.w};
#pragma unroll
          for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float v = idv[4 * t + r] >= 0 ? st[t][r] * sl2 : -__builtin_inff();
              z[4 * t + r] = v;
              cmax = fmaxf(cmax, v);
            }
          // The head's maximum over the four lane groups matters only when
          // some value exceeds the reference by more than kLazy; otherwise
          // every lane keeps the reference (the same decision either way),
          // and the two cross-lane exchanges are skipped.
          if (__any(cmax > m_run + kLazy)) {
            cmax = fmaxf(cmax, __shfl_xor(cmax, 16, 64));
            cmax = fmaxf(cmax, __shfl_xor(cmax, 32, 64));
          }
        }
        float alpha = 1.0f;
        v8h pa;
#pragma unroll
        for (int i = 0; i < 8; ++i) pa[i] = (_Float16)0.0f;
        if (active) {
          // The reference maximum moves only when the chunk's maximum exceeds
          // it by more than kLazy (log2 units): P stays below 2^kLazy, exact
          // to fp16's relative precision, and the PV waves rescale O rarely.
          const float m_new = cmax > m_run + kLazy ? cmax : m_run;
          float psum = 0.0f;
          if (m_new != -__builtin_inff()) {
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
        }
        pex[pb][hg][lane] = pa;
        if (g == 0) alf[pb][16 * hg + c16] = alpha;
        // One flag per S wave tells the PV waves whether any of its heads'
        // reference maxima moved (the factors are then read and applied).
        const bool moved = __any(alpha != 1.0f);
        if (lane == 0) mvf[pb][hg] = moved ? 1u : 0u;
      }
      advance(it, c0, kb_next, idn);
      __syncthreads();
      kb = kb_next;
    }
    // per-head (m, l): l summed over the 4 lane groups
    float l_tot = l_run;
    l_tot += __shfl_xor(l_tot, 16, 64);
    l_tot += __shfl_xor(l_tot, 32, 64);
    if (splits == 1) {
      // The row's only split: normalise here, with the combine's operations
      // in its order (O * 2^(m - M), then * 1/L; L = l * 2^(m - M) +
      // 2^(sink - M)), and write out and lse; no partials, no combine launch.
      if (active && g == 0) {
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
        pml[0][head_b] = w;
        pml[1][head_b] = L > 0.0f ? 1.0f / L : 0.0f;
        if (a.lse) a.lse[row * H + head_b] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
      }
      __syncthreads();
      return;
    }
    if (active && g == 0) {
      const int64_t pbase = (row * splits + split) * (int64_t)H;
      part_ml[(pbase + head_b) * 2 + 0] = m_run;
      part_ml[(pbase + head_b) * 2 + 1] = l_tot;
    }
    return;
  }

  // ================================================================ PV waves
  // Wave dq owns all heads (4 tiles of 16) and output dims 128*dq .. +127.
  const int dq = wave & 3;
  v4f o[4][NT];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n) o[t][n] = v4f{0.f, 0.f, 0.f, 0.f};
  // Wave 4 keeps the raw ids of chunk it+3 in flight: issued before the
  // loads of chunk it+1, so the dequantisation's wait for those covers them,
  // and no wait for the gather is needed anywhere else in the loop.
  // Paged: the raw ids are loaded two chunks ahead, validated and their
  // block-table entries loaded one chunk ahead, and the pool rows staged.
  // (With no Top-K entries, k_top = 0, the window rows are still staged by
  // this lane; its raw id loads then read ctx_len[b], a valid address whose
  // value no window entry uses.)
  const bool id_lane = wave == 4 && lane < kChunk;
  auto raw_id = [&](int c) -> const int32_t* { return K > 0 ? idx_row + (c < K ? c : K - 1) : a.ctx_len + b; };
  int32_t ldn = 0, vn = -1, pgn = 0;
  if (id_lane) {
    const int ce = e_begin + 3 * kChunk + lane;
    if constexpr (PAGED) {
      const int32_t r3 = *raw_id(ce);
      const int c4 = ce + kChunk;
      ldn = *raw_id(c4);
      vn = entry_id(ce, r3);
      pgn = page_of(ce, vn);
    } else {
      ldn = *raw_id(ce);
    }
  }
  if (nch > 0) store(kbuf[0]);
  if (nch > 1) gather(e_begin + kChunk, 1);
  __syncthreads();
  int kb = 0;
  for (int it = 0; it <= nch; ++it) {
    const int c0 = e_begin + it * kChunk;
    const int pb = it & 1;
    const int kb_prev = kb == 0 ? 2 : kb - 1, kb_next = kb == 2 ? 0 : kb + 1;
    int32_t idn[TPT];
    if (it + 2 < nch) task_ids(c0 + 2 * kChunk, (it + 2) & 3, idn);
    // The dequantisation comes first here (the S waves end with it), so
    // that one role's VALU work overlaps the other's products.
    if (it + 1 < nch) {
      store(kbuf[kb_next]);
      if (id_lane) {
        const int ce = c0 + 3 * kChunk + lane;
        if constexpr (PAGED) {
          if (it + 3 < nch) eidc[(it + 3) & 3][lane] = pool_row(ce, vn, pgn);
          const int c4 = ce + kChunk;
          vn = entry_id(c4, ldn);
          pgn = page_of(c4, vn);
          const int c5 = c4 + kChunk;
          ldn = *raw_id(c5);
        } else {
          if (it + 3 < nch) eidc[(it + 3) & 3][lane] = entry_id(ce, ldn);
          const int cn = ce + kChunk;
          ldn = *raw_id(cn);
        }
      }
      if (it + 2 < nch) gather_ids(c0 + 2 * kChunk, idn);
    }
    if (it >= 1) {
      // O += P V for chunk it-1; k index: entries {4g..4g+3, 16+4g..16+4g+3},
      // the lane layout of the S^T accumulators.
      const _Float16* kt = kbuf[kb_prev];
      // V from the row-major K rows with the LDS transpose read: in each
      // 16-lane group, source lane s names entry (.. + s/4), dims
      // 4(s%4)..+3, and lane i receives dim i of those four entries.  Read
      // first: V does not depend on this chunk's P.
      const int s16 = lane & 15;
      const _Float16* vbase = kt + (4 * g + (s16 >> 2)) * S::PITCH + 128 * dq + 4 * (s16 & 3);
      typedef short v4s __attribute__((ext_vector_type(4)));
      typedef __attribute__((address_space(3))) v4s* lds_v4s;
      v8h vf[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const _Float16* vp = vbase + 16 * n;
        v4s lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vp));
        v4s hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s)(vp + 16 * S::PITCH));
        vf[n] = __builtin_bit_cast(v8h, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      }
      v8h pf[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) pf[t] = pex[pb ^ 1][t][lane];
      const uint4 mv = *reinterpret_cast<const uint4*>(&mvf[pb ^ 1][0]);
      if (__builtin_amdgcn_readfirstlane(mv.x | mv.y | mv.z | mv.w) != 0u) {
        float4 al[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) al[t] = *reinterpret_cast<const float4*>(&alf[pb ^ 1][16 * t + 4 * g]);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            o[t][n][0] *= al[t].x; o[t][n][1] *= al[t].y; o[t][n][2] *= al[t].z; o[t][n][3] *= al[t].w;
          }
      }
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int t = 0; t < 4; ++t) o[t][n] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pf[t], vf[n], o[t][n], 0, 0, 0);
    }
    __syncthreads();
    kb = kb_next;
  }
  if (splits == 1) {
    __syncthreads();   // the S waves' (w, 1/L)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (16 * t >= H) break;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * t + 4 * g + r;
        const float w = pml[0][h], inv = pml[1][h];
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          float v = (o[t][n][r] * w) * inv;
          const int dim = 128 * dq + 16 * n + c16;
          if (a.rope_cs && 128 * dq + 16 * n >= DV - a.rope_dim) {
            // inverse rotation of the rotary output channels: the pair's
            // other half sits in the neighbouring lane
            const float other = __shfl_xor(v, 1, 64);
            const int pr = (dim - (DV - a.rope_dim)) & ~1;
            const float c = a.rope_cs[row * (int64_t)a.rope_dim + pr], sn = a.rope_cs[row * (int64_t)a.rope_dim + pr + 1];
            v = (c16 & 1) ? v * c - other * sn : v * c + other * sn;
          }
          a.out[(row * H + h) * DV + dim] = v;
        }
      }
    }
    return;
  }
  const int64_t pbase = (row * splits + split) * (int64_t)H;
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    if (16 * t >= H) break;
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * t + 4 * g + r;
        part_o[(pbase + h) * DV + 128 * dq + 16 * n + c16] = o[t][n][r];
      }
  }
}

// Merge split partials: out = sum_s O_s 2^(m_s - M) / L, L = sum_s l_s 2^(m_s - M)
// (+ 2^(sink*log2e - M)), lse = (M + log2 L) ln 2.  One workgroup per
// (row, head) of G groups of DV/DPL threads (DPL output dims per thread):
// every wave reduces the split maxima itself, then group k accumulates
// splits k, k + G, ... with the loads of U of them in flight, and the
// groups' sums are added in group order through LDS.  G, U and DPL follow
// the split count, so that a row's splits are usually read in one round
// trip without padding loads.
template <int DV, int U, int DPL, int MAXG>
__global__ void __launch_bounds__(512)
sparse_attn_combine_kernel(const float* __restrict__ part_o, const float* __restrict__ part_ml, int splits, int H,
                           const float* __restrict__ sink, float* __restrict__ out, float* __restrict__ lse,
                           const float* __restrict__ rope_cs, int rope_dim) {
  constexpr int GT = DV / DPL;              // threads per group
  constexpr int NV = DPL / 4;               // float4 per thread and split
  static_assert(DPL % 4 == 0 && GT % 64 == 0, "whole waves of float4 columns");
  __shared__ float4 accs[(MAXG - 1) * GT * NV + 1];   // sums of groups 1..G-1 (G <= MAXG)
  __shared__ float lsum[MAXG];
  const int64_t rh = blockIdx.x;            // row * H + h
  const int h = (int)(rh % H);
  const int64_t row = rh / H;
  const int lane = threadIdx.x & 63;
  const int grp = threadIdx.x / GT, gl = threadIdx.x % GT;
  const int G = blockDim.x / GT;
  const float sk = sink ? sink[h] * kLog2e : -__builtin_inff();
  const float* mlb = part_ml + (row * splits * (int64_t)H + h) * 2;   // split s at mlb[2 * s * H]
  const float4* ob = reinterpret_cast<const float4*>(part_o + (row * splits * (int64_t)H + h) * DV) + NV * gl;
  // The first round's partials are requested before the split maxima are
  // reduced (their addresses do not depend on them), so that both loads
  // share one memory round trip.
  float2 ml[U];
  float4 ov[U][NV];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int sp = s0 + u * G < splits ? s0 + u * G : (s0 < splits ? s0 : 0);
      ml[u] = *reinterpret_cast<const float2*>(mlb + 2 * (int64_t)sp * H);
#pragma unroll
      for (int v = 0; v < NV; ++v) ov[u][v] = ob[(int64_t)sp * H * (DV / 4) + v];
    }
  };
  load_round(grp);
  float mx = -__builtin_inff();
  for (int sp = lane; sp < splits; sp += 64) mx = fmaxf(mx, mlb[2 * (int64_t)sp * H]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, 64));
  const float M = fmaxf(mx, sk);
  float4 acc[NV];
#pragma unroll
  for (int v = 0; v < NV; ++v) acc[v] = float4{0.f, 0.f, 0.f, 0.f};
  float L = 0.0f;
  if (M != -__builtin_inff()) {
    for (int s0 = grp; s0 < splits; s0 += G * U) {
      if (s0 != grp) load_round(s0);
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u * G >= splits || ml[u].x == -__builtin_inff()) continue;
        const float wgt = __builtin_amdgcn_exp2f(ml[u].x - M);
        L += ml[u].y * wgt;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
          acc[v].x += ov[u][v].x * wgt; acc[v].y += ov[u][v].y * wgt;
          acc[v].z += ov[u][v].z * wgt; acc[v].w += ov[u][v].w * wgt;
        }
      }
    }
  }
  if (MAXG > 1 && G > 1) {
    if (grp > 0) {
#pragma unroll
      for (int v = 0; v < NV; ++v) accs[((grp - 1) * NV + v) * GT + gl] = acc[v];
      if (gl == 0) lsum[grp] = L;
    }
    __syncthreads();
    if (grp > 0) return;
    for (int k = 1; k < G; ++k) {
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const float4 x = accs[((k - 1) * NV + v) * GT + gl];
        acc[v].x += x.x; acc[v].y += x.y; acc[v].z += x.z; acc[v].w += x.w;
      }
      L += lsum[k];
    }
  }
  if (M != -__builtin_inff() && sk != -__builtin_inff()) L += __builtin_amdgcn_exp2f(sk - M);
  const float inv = L > 0.0f ? 1.0f / L : 0.0f;
  float4* op = reinterpret_cast<float4*>(out + rh * DV) + NV * gl;
#pragma unroll
  for (int v = 0; v < NV; ++v) {
    float4 r = float4{acc[v].x * inv, acc[v].y * inv, acc[v].z * inv, acc[v].w * inv};
    const int d0 = 4 * (NV * gl + v);
    if (rope_cs && d0 >= DV - rope_dim) {   // inverse rotation of two rotary pairs
      const float4 cs = *reinterpret_cast<const float4*>(rope_cs + row * (int64_t)rope_dim + (d0 - (DV - rope_dim)));
      r = float4{r.x * cs.x + r.y * cs.y, r.y * cs.x - r.x * cs.y, r.z * cs.z + r.w * cs.w, r.w * cs.z - r.z * cs.w};
    }
    op[v] = r;
  }
  if (lse && threadIdx.x == 0) lse[rh] = L > 0.0f ? (M + __log2f(L)) * kLn2 : -__builtin_inff();
}

int attn_num_splits(int64_t rows, int k_top, int W) {
  // One resident workgroup per compute unit (LDS and registers allow one),
  // but at least 128 entries (four chunks) per split: with fewer rows than
  // compute units, shorter splits took no less time each and only added
  // partials for the combine.
  int E = k_top + W;
  int max_splits = (E + 127) / 128;
  int64_t want = ((int64_t)device_cu_count() + rows - 1) / rows;
  int s = (int)(want < 1 ? 1 : (want > max_splits ? max_splits : want));
  return s < 1 ? 1 : s;
}

size_t attn_ws_bytes(int64_t rows, int H, int d_v, int splits) {
  size_t po = sizeof(float) * (size_t)rows * splits * H * d_v;
  size_t pm = sizeof(float) * (size_t)rows * splits * H * 2;
  return ((po + 255) & ~(size_t)255) + ((pm + 255) & ~(size_t)255);
}

template <int DQK, int DV, bool PAGED>
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
  CSA2_LAUNCH("sparse_attn_split", (sparse_attn_split_kernel<DQK, DV, PAGED>), dim3(real_splits, (unsigned)rows),
              dim3(kAttnThreads), 0, s, a, prefill ? 1 : 0, real_splits, span, part_o, part_ml);
  if (real_splits > 1) {   // (a single split normalises and writes the output itself)
    // Up to 4 splits: one group of 128 threads (4 dims each) with every
    // split in flight; more: groups of 64 threads (8 dims each) over up to
    // 4 or 8 splits each.
    const dim3 grid((unsigned)(rows * a.H));
    if (real_splits <= 4) {
      CSA2_LAUNCH("sparse_attn_combine", (sparse_attn_combine_kernel<DV, 4, 4, 1>), grid, dim3(DV / 4), 0, s, part_o,
                  part_ml, real_splits, a.H, a.sink, a.out, a.lse, a.rope_cs, a.rope_dim);
    } else {
      const int U = real_splits <= 16 ? 4 : 8;
      int G = (real_splits + U - 1) / U;
      if (G > 8) G = 8;
      if (U == 4)
        CSA2_LAUNCH("sparse_attn_combine", (sparse_attn_combine_kernel<DV, 4, 8, 8>), grid, dim3(64 * G), 0, s, part_o,
                    part_ml, real_splits, a.H, a.sink, a.out, a.lse, a.rope_cs, a.rope_dim);
      else
        CSA2_LAUNCH("sparse_attn_combine", (sparse_attn_combine_kernel<DV, 8, 8, 8>), grid, dim3(64 * G), 0, s, part_o,
                    part_ml, real_splits, a.H, a.sink, a.out, a.lse, a.rope_cs, a.rope_dim);
    }
  }
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const AttnArgs& a, bool prefill, void* ws, hipStream_t s) {
  const bool paged = a.block_table != nullptr;
  if (a.d_qk == 576 && a.d_v == 512)
    return paged ? launch_attn_t<576, 512, true>(a, prefill, ws, s) : launch_attn_t<576, 512, false>(a, prefill, ws, s);
  if (a.d_qk == 512 && a.d_v == 512)
    return paged ? launch_attn_t<512, 512, true>(a, prefill, ws, s) : launch_attn_t<512, 512, false>(a, prefill, ws, s);
  return hipErrorInvalidValue;
}

}  // namespace csa2
