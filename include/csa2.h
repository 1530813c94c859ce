/*
 * csa2.h -- C ABI of the CSA2 (Compressed Sparse Attention 2) hot path for
 * AMD Instinct MI355X (gfx950).
 *
 * The path, as the DeepSeek-V4.1 pages describe it:
 *   - FP4 main KV cache: E2M1 values with one E4M3 scale per 16 channels,
 *     written after RoPE (DeepSeek-V4.1 blog, Introduction > DeepSeek-V4.1-
 *     Flash, CSA2 paragraph; DeepSeek-V4.1-Flash fact sheet, storage
 *     components of attn.kv_groups, main KV groups; techniques map, inference
 *     quantization: post-RoPE KV-cache quantization).
 *   - FP8 sliding-window cache of the last 128 tokens, E4M3 values with one
 *     E8M0 scale per 32 channels (fact sheet, SWA window group).
 *   - A lightning-style indexer scores every visible token and keeps the
 *     Top-K (techniques map, "Checked in its code", indexer-selected sparse
 *     attention; fact sheet, token selection).
 *   - Full / Reindex / Reuse layer modes share the main KV and indexer K and
 *     reuse Top-K indices; a hierarchical indexer restricts later layers to a
 *     candidate pool chosen by the first Full layer (blog, CSA2 paragraph;
 *     fact sheet, token selection: 2048-block x 8-position pool).
 *   - Sparse MLA attention with one shared latent K=V row per token; an
 *     optional extra logit per head joins only the softmax normaliser
 *     (techniques map: multi-head latent attention, learnable attention
 *     sink).
 *
 * Conventions shared by every entry point:
 *   - Every pointer is a caller-owned DEVICE buffer, except where noted.  The
 *     library never allocates, frees or synchronises; all work is enqueued on
 *     `stream` (a hipStream_t; NULL = the null stream).  Results are valid
 *     once the stream reaches that point.
 *   - Row-major layouts.  Cache strides are in BYTES.  Code / value arrays
 *     (and their strides) must be 4-byte aligned; scale arrays may have any
 *     stride.  This admits both the pages' interleaved entry (codes then
 *     scales in one row) and separate code/scale arrays.
 *   - Host-side validation of shapes, strides and pointers only; the data is
 *     not inspected.  NaN/Inf inputs are outside the contract.
 *   - Workspace: `ws` must hold at least the matching *_workspace_size()
 *     bytes, 256-byte aligned.  Its content on entry does not matter; it is
 *     scratch until the stream passes the call.  Calls that share one
 *     workspace must be ordered on one stream.
 *   - Return value: a csa2_status (0 = success).  Nothing is enqueued when a
 *     validation error is returned.
 *   - No global mutable state, except the optional per-thread kernel trace
 *     and the static scratch of csa2_index_score_topk_noalloc.
 */
#ifndef CSA2_H
#define CSA2_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum csa2_status {
  CSA2_OK = 0,
  CSA2_EINVAL = 1,       /* null required pointer, bad shape/stride/alignment */
  CSA2_EUNSUPPORTED = 2, /* valid arguments outside the compiled shape set */
  CSA2_EWORKSPACE = 3,   /* ws_bytes smaller than the *_workspace_size() */
  CSA2_EHIP = 4,         /* a HIP launch reported an error */
  CSA2_ESCRATCH = 5      /* inputs too large for csa2_index_score_topk_noalloc's static scratch */
};

/* Human-readable text of a status code (static storage, never NULL). */
const char* csa2_status_string(int status);

/* Library version string "major.minor.patch" (static storage). */
const char* csa2_version(void);

/*
 * kv_fp4_quantize -- main-KV write (blog, CSA2 paragraph; fact sheet, main KV
 * group: 256 data bytes + 32 scale bytes per 512-element entry).
 * Per row and per 16-channel group g:
 *   amax  = max |x| over the group (float32)
 *   scale = E4M3(float32(amax / 6)), round-to-nearest-even, saturating at 448
 *   code  = E2M1 value nearest |x| / scale (exact quotient), ties to the even
 *           code, saturating at 6; all zero when scale == 0; the sign bit is
 *           set only for a negative x with a non-zero magnitude.
 * x       [n_rows][d] float32, row stride x_row_stride ELEMENTS (>= d).
 * codes   [n_rows][d/2] bytes, channel 2i in the low nibble of byte i,
 *         row stride codes_row_stride BYTES.
 * scales  [n_rows][d/16] E4M3 bytes, row stride scales_row_stride BYTES.
 * d must be a positive multiple of 16.  n_rows == 0 is a no-op.
 */
int kv_fp4_quantize(const float* x, int64_t n_rows, int32_t d, int64_t x_row_stride,
                    uint8_t* codes, int64_t codes_row_stride,
                    uint8_t* scales, int64_t scales_row_stride, void* stream);

/*
 * swa_fp8_quantize -- sliding-window cache write (fact sheet, SWA window
 * group: E4M3 values with one E8M0 scale per 32 channels, 512 + 16 bytes).
 * Per row and 32-channel group: shared exponent e = floor(log2 amax) - 8,
 * E8M0 code clamp(e + 127, 0, 254) (127 when amax == 0); values are
 * E4M3(x / 2^e) with round-to-nearest-even and saturation at 448.
 * x [n_rows][d] float32 (row stride in elements); vals [n_rows][d] bytes;
 * scales [n_rows][d/32] bytes (row strides in bytes).  d % 32 == 0.
 */
int swa_fp8_quantize(const float* x, int64_t n_rows, int32_t d, int64_t x_row_stride,
                     uint8_t* vals, int64_t vals_row_stride,
                     uint8_t* scales, int64_t scales_row_stride, void* stream);

/*
 * idx_mxfp4_quantize -- indexer K write in the pages' format (fact sheet,
 * indexer K groups: MXFP4, E2M1 values with one E8M0 scale per 32 channels;
 * 64 code bytes + 4 scale bytes = 68 bytes per 128-channel entry).
 * Per row and 32-channel group: shared exponent e = floor(log2 amax) - 2,
 * E8M0 code clamp(e + 127, 0, 254) (127 when amax == 0); each element is the
 * E2M1 value nearest x / 2^e, ties to the even code, saturating at 6; the
 * sign bit only for a negative x with a non-zero magnitude.
 * x [n_rows][d] float32 (row stride in elements); codes [n_rows][d/2]
 * (channel 2i in the low nibble of byte i), scales [n_rows][d/32] (row
 * strides in bytes; code rows 4-byte aligned).  d % 32 == 0.
 */
int idx_mxfp4_quantize(const float* x, int64_t n_rows, int32_t d, int64_t x_row_stride,
                       uint8_t* codes, int64_t codes_row_stride,
                       uint8_t* scales, int64_t scales_row_stride, void* stream);

/*
 * csa2_index_score_topk -- indexer scoring + exact Top-K for Full and Reindex
 * layers (techniques map, indexer-selected sparse attention; blog, CSA2
 * paragraph), optionally also building the hierarchical candidate pool of
 * the first Full layer (blog, CSA2 paragraph; fact sheet, token selection).
 *
 * For query row (b, t) and visible token j (j < ctx_len[b] and, when q_pos
 * is given, j <= q_pos[b][t]):
 *   d_h = q_idx[b][t][h] . k_idx[b][j]  (exact for integer-valued E4M3 data
 *         whose partial sums stay below 2^24 in magnitude)
 *   s_j = sum over h = 0..H_I-1, in that order, of w[b][t][h] * max(d_h, 0),
 *         every float32 multiply and add rounded to nearest, no FMA.
 * Top-K: order (s desc, j asc); the first min(k_top, visible) tokens are
 * written to topk_idx[b][t][*] in ascending j, padded with -1; topk_score
 * (nullable) receives their scores (-inf for padding).
 *
 * q_idx    [B][Tq][H_I][D_I] E4M3 bytes.     w [B][Tq][H_I] float32.
 * k_idx    row j of sequence b at k_idx + b*k_batch_stride + j*k_row_stride
 *          (bytes), D_I E4M3 bytes per row; n_max rows are addressable.
 *          k_row_stride: a multiple of 8 (of 16 when D_I >= 128), below 4 MiB
 *          (CSA2_EUNSUPPORTED otherwise).
 * ctx_len  [B] int32 (values clamped to [0, n_max]).
 * q_pos    [B][Tq] int32 or NULL (NULL: every row sees the whole context).
 * topk_idx [B][Tq][k_top] int32 out; topk_score [B][Tq][k_top] float out or NULL.
 * Pool (pool_idx != NULL): blocks are [c*pool_block, (c+1)*pool_block) of the
 *   visible prefix; a block's score is the max of its tokens'; the top
 *   pool_nblocks blocks by (score desc, block asc) are expanded to their
 *   visible tokens: pool_idx [B][Tq][pool_nblocks*pool_block] int32 ascending,
 *   -1 padded; pool_len [B][Tq] int32 = number of valid entries.
 *   pool_block must be 1, 2, 4, 8 or 16.  The flat Top-K is a subset of the
 *   pool whenever pool_nblocks >= k_top.
 * Supported: D_I in {32, 64, 128, 256}; 1 <= H_I <= 32; k_top >= 1;
 * n_max <= 4,194,304 positions; B*Tq <= 65,535; k_row_stride < 4 MiB.
 *
 * Workspace: ws / ws_bytes, 256-byte aligned, of at least
 * csa2_index_score_topk_workspace_size() bytes.  Dense prefill chunks
 * (Tq >= 16, no pool, k_top <= 8192) select in one of two ways, with
 * identical results:
 *   - stored score keys, 4 bytes per (query row, visible position) plus
 *     per-tile histograms (csa2_index_score_topk_workspace_size_stored();
 *     13.4 GB for 4096 queries on 266,240 tokens), used whenever ws_bytes
 *     reaches that size: one scoring pass;
 *   - otherwise no score matrix at all: two passes that score one 16-key
 *     chunk in every eight build histograms of that sample and place each
 *     row's threshold in a narrow window, a full scoring pass emits the keys
 *     above the window and collects those inside it, and rows whose counts
 *     do not confirm the window (heavy ties, for instance) search exactly
 *     in further passes (radix digits of 12, 12 and 8 bits, then tie counts
 *     and tie emission in position order).  Query rows go in blocks of at
 *     most 1920; the workspace stays under 100 MB (10^8 bytes) for chunks
 *     up to 65,535 query rows and 4M positions.
 * csa2_index_score_topk_workspace_size() is the smaller of the two for such
 * chunks and the stored size for every other call.
 */
size_t csa2_index_score_topk_workspace_size(int32_t B, int32_t Tq, int64_t n_max, int32_t k_top,
                                            int32_t pool_block, int32_t pool_nblocks);
size_t csa2_index_score_topk_workspace_size_stored(int32_t B, int32_t Tq, int64_t n_max, int32_t k_top,
                                                   int32_t pool_block, int32_t pool_nblocks);
int csa2_index_score_topk(const uint8_t* q_idx, const float* w,
                          const uint8_t* k_idx, int64_t k_batch_stride, int64_t k_row_stride,
                          const int32_t* ctx_len, const int32_t* q_pos,
                          int32_t B, int32_t Tq, int32_t H_I, int32_t D_I, int64_t n_max, int32_t k_top,
                          int32_t* topk_idx, float* topk_score,
                          int32_t pool_block, int32_t pool_nblocks, int32_t* pool_idx, int32_t* pool_len,
                          void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_score_topk_mxfp4 -- csa2_index_score_topk over the pages' MXFP4
 * indexer keys (fact sheet, indexer K groups: E2M1 values, one E8M0 scale per
 * 32 channels, 68 bytes per 128-channel entry; idx_mxfp4_quantize writes them).
 * Same arguments, results, workspace (csa2_index_score_topk_workspace_size)
 * and pool option, with the key cache given as two arrays:
 *   k_codes  row j of b at k_codes + b*kc_batch_stride + j*kc_row_stride:
 *            D_I/2 bytes, channel 2i in the low nibble of byte i (pointer and
 *            strides multiples of 16; the pages' 68-byte entry therefore
 *            splits into a code array and a scale array).
 *   k_scales row j of b at k_scales + b*ks_batch_stride + j*ks_row_stride:
 *            D_I/32 E8M0 bytes (pointer and strides multiples of 4).
 *   d_h = q_idx[b][t][h] . dequant(k_j) on the scaled FP4 matrix cores; exact
 *   (hence bit-identical scores and indices) for integer-valued E4M3 queries
 *   in [-4, 4] whenever a key's four shared exponents span at most 11 binades.
 * Supported: D_I = 128, 1 <= H_I <= 32; prefill chunks (Tq >= 16) with
 * H_I <= 8 run as one dense product, longer head counts row by row.
 */
int csa2_index_score_topk_mxfp4(const uint8_t* q_idx, const float* w,
                                const uint8_t* k_codes, int64_t kc_batch_stride, int64_t kc_row_stride,
                                const uint8_t* k_scales, int64_t ks_batch_stride, int64_t ks_row_stride,
                                const int32_t* ctx_len, const int32_t* q_pos,
                                int32_t B, int32_t Tq, int32_t H_I, int32_t D_I, int64_t n_max, int32_t k_top,
                                int32_t* topk_idx, float* topk_score,
                                int32_t pool_block, int32_t pool_nblocks, int32_t* pool_idx, int32_t* pool_len,
                                void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_index_score_topk_noalloc -- csa2_index_score_topk for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same arguments, results and
 * kernels, minus ws / ws_bytes.  Its workspace is a static device array of
 * 64 MiB (64 << 20 bytes) inside the library, one per GPU, kept until the
 * process ends; the call allocates nothing, and what must start at zero is
 * cleared by a kernel on `stream`.  Inputs whose
 * csa2_index_score_topk_workspace_size() exceeds 64 MiB return
 * CSA2_ESCRATCH with nothing enqueued (e.g. 64 x 64K-token decode rows need
 * 48 MiB, 4 x 1M with the 2048 x 8 pool 55 MiB; a dense prefill chunk whose
 * stored keys exceed 64 MiB selects by scoring passes).  Every call on one
 * GPU uses that GPU's one array: calls that may overlap on one GPU (other
 * streams, other host threads) race and must be ordered by the caller.
 */
int csa2_index_score_topk_noalloc(const uint8_t* q_idx, const float* w,
                                  const uint8_t* k_idx, int64_t k_batch_stride, int64_t k_row_stride,
                                  const int32_t* ctx_len, const int32_t* q_pos,
                                  int32_t B, int32_t Tq, int32_t H_I, int32_t D_I, int64_t n_max, int32_t k_top,
                                  int32_t* topk_idx, float* topk_score,
                                  int32_t pool_block, int32_t pool_nblocks, int32_t* pool_idx, int32_t* pool_len,
                                  void* stream);

/*
 * csa2_hier_pool_topk -- later hierarchical-indexer layers (blog, CSA2
 * paragraph: later indexing layers are restricted to the candidate pool of
 * the first Full layer).  Scores only the pool tokens pool_idx[b][t][0 ..
 * pool_len-1] (ascending token ids, as csa2_index_score_topk writes them)
 * with this layer's q_idx / w, and keeps the Top-K by (s desc, token id asc).
 * Output as csa2_index_score_topk: ascending token ids, -1 padded.
 * ctx_len  [B] int32: pool ids id with 0 <= id < ctx_len[b] name tokens; any
 *          other entry (-1 padding, a stale or out-of-range id) is skipped,
 *          never read.  ctx_len[b] must not exceed the rows k_idx holds for
 *          sequence b.
 * pool_idx [B][Tq][pool_cap] ascending among its valid entries;
 * pool_len [B][Tq] (clamped to [0, pool_cap]).
 */
size_t csa2_hier_pool_topk_workspace_size(int32_t B, int32_t Tq, int32_t pool_cap, int32_t k_top);
int csa2_hier_pool_topk(const uint8_t* q_idx, const float* w,
                        const uint8_t* k_idx, int64_t k_batch_stride, int64_t k_row_stride,
                        const int32_t* ctx_len, const int32_t* pool_idx, const int32_t* pool_len, int32_t pool_cap,
                        int32_t B, int32_t Tq, int32_t H_I, int32_t D_I, int32_t k_top,
                        int32_t* topk_idx, float* topk_score,
                        void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_hier_pool_topk_mxfp4 -- csa2_hier_pool_topk over MXFP4 indexer keys
 * (key arrays as in csa2_index_score_topk_mxfp4; workspace
 * csa2_hier_pool_topk_workspace_size).
 */
int csa2_hier_pool_topk_mxfp4(const uint8_t* q_idx, const float* w,
                              const uint8_t* k_codes, int64_t kc_batch_stride, int64_t kc_row_stride,
                              const uint8_t* k_scales, int64_t ks_batch_stride, int64_t ks_row_stride,
                              const int32_t* ctx_len, const int32_t* pool_idx, const int32_t* pool_len,
                              int32_t pool_cap, int32_t B, int32_t Tq, int32_t H_I, int32_t D_I, int32_t k_top,
                              int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_decode -- sparse MLA decode attention over the Top-K FP4
 * main-KV rows plus the FP8 window (techniques map: MLA with one latent KV
 * head, learnable sink; fact sheet: one shared K=V entry, 128-token window
 * per layer).  Used by Full, Reindex and Reuse layers alike: a Reuse layer
 * passes another layer's topk_idx.
 * For row b and head h, with entry set E = {valid topk rows} U {window rows
 * 0 .. swa_len[b]-1}:
 *   k_e = dequantised row (d_qk channels), v_e = its first d_v channels
 *   z_e = softmax_scale * (q[b][h] . k_e)
 *   out[b][h] = sum_e softmax(z, sink_h)_e v_e; lse[b][h] = log-sum-exp of z
 *   (and sink_h), natural log.  Empty E without sink: out = 0, lse = -inf.
 * Index entries < 0 or >= ctx_len[b] are skipped.
 * q        [B][H][d_qk] float32.
 * kv_codes row j of b at kv_codes + b*c_batch_stride + j*c_row_stride (d_qk/2 bytes);
 * kv_scales row j of b at kv_scales + b*s_batch_stride + j*s_row_stride (d_qk/16 bytes).
 * topk_idx [B][k_top] int32 (NULL allowed when k_top = 0: the window alone).  ctx_len [B].
 * swa_vals  row w of b at swa_vals + b*sv_batch_stride + w*sv_row_stride (d_qk bytes E4M3);
 * swa_scales row w of b at swa_scales + b*ss_batch_stride + w*ss_row_stride (d_qk/32 bytes E8M0);
 * swa_len  [B] int32 (clamped to [0, W]); swa pointers may be NULL when W == 0.
 * sink     [H] float32 or NULL.  out [B][H][d_v] float32; lse [B][H] or NULL.
 * Supported: (d_qk, d_v) in {(576, 512), (512, 512)}; H % 16 == 0, H <= 64
 * (CSA2_EUNSUPPORTED otherwise).
 * Arithmetic: dequantised K/V rows and q enter fp16 matrix cores with fp32
 * accumulation; softmax and the output reduction are fp32.
 * Accuracy: main rows (E2M1 x E4M3: at most 6 significant bits within
 * [2^-10, 2688]) are exact in fp16; window values are exact while every
 * block's E8M0 code lies in [112, 134] (scales 2^-15 .. 2^7) and are rounded
 * to fp16 (subnormals below 2^-14, zero below 2^-24, overflow above 65504)
 * outside it.  q and the softmax weights are rounded to fp16 once (relative
 * 2^-11), so each logit moves by about softmax_scale * |q_h| |k_e| * 2^-12.
 * With unit-variance q and rows this keeps every (row, head) output within
 * 2e-3 relative (max error / max |out|) up to softmax_scale = 4 / sqrt(576);
 * at larger logit spreads the error grows with that product (about 5e-3 on
 * outputs and 7e-3 on lse at 12 / sqrt(576)).
 */
size_t csa2_sparse_attn_decode_workspace_size(int32_t B, int32_t H, int32_t d_v, int32_t k_top, int32_t W);
int csa2_sparse_attn_decode(const float* q,
                            const uint8_t* kv_codes, int64_t c_batch_stride, int64_t c_row_stride,
                            const uint8_t* kv_scales, int64_t s_batch_stride, int64_t s_row_stride,
                            const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len,
                            const uint8_t* swa_vals, int64_t sv_batch_stride, int64_t sv_row_stride,
                            const uint8_t* swa_scales, int64_t ss_batch_stride, int64_t ss_row_stride,
                            const int32_t* swa_len, int32_t W, const float* sink,
                            int32_t B, int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                            float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_decode_rope -- csa2_sparse_attn_decode over the pages'
 * 512-wide K = V row (fact sheet, attention facts: head dim 512 = nope +
 * rope, one shared K = V entry; partial RoPE on the last 64 dims of Q and KV
 * with an inverse rotation on the attention output; techniques map, inference
 * kernel: a fused RoPE-attention-RoPE-cast kernel) with the rotary steps
 * fused around it.  d_qk = d_v = d = 512.  rope_cs [B][rope_dim] float32
 * (16-byte aligned): for the query position of row b, the cosine and sine of
 * the angle of each channel pair (2i, 2i+1) of the last rope_dim channels,
 * (cos_i, sin_i) at [b][2i], [b][2i+1] (the angles -- RoPE base, YaRN -- are
 * the caller's).  When rotate_q, q's last rope_dim channels are rotated
 * forward, (a, b) -> (a cos - b sin, a sin + b cos), before the products
 * (else q arrives rotated); out's last rope_dim channels are always rotated
 * back, (a, b) -> (a cos + b sin, b cos - a sin).  The output stays float32.
 * rope_dim a positive multiple of 4, at most d.  Other arguments as in
 * csa2_sparse_attn_decode (workspace: csa2_sparse_attn_decode_workspace_size).
 */
int csa2_sparse_attn_decode_rope(const float* q,
                                 const uint8_t* kv_codes, int64_t c_batch_stride, int64_t c_row_stride,
                                 const uint8_t* kv_scales, int64_t s_batch_stride, int64_t s_row_stride,
                                 const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len,
                                 const uint8_t* swa_vals, int64_t sv_batch_stride, int64_t sv_row_stride,
                                 const uint8_t* swa_scales, int64_t ss_batch_stride, int64_t ss_row_stride,
                                 const int32_t* swa_len, int32_t W, const float* sink,
                                 int32_t B, int32_t H, int32_t d, float softmax_scale,
                                 const float* rope_cs, int32_t rope_dim, int32_t rotate_q,
                                 float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_prefill -- the same attention for a causal chunk of Tq
 * query tokens per sequence, each with its own Top-K list and its own window:
 * the query at position p = q_pos[b][t] sees window positions
 * max(p - W + 1, swa_pos0[b]) .. p, where window-array row i of sequence b
 * holds position swa_pos0[b] + i (rows 0 .. swa_rows-1).
 * q [B][Tq][H][d_qk]; topk_idx [B][Tq][k_top]; q_pos [B][Tq];
 * swa_vals / swa_scales rows as in decode with swa_rows rows per sequence;
 * swa_pos0 [B]; out [B][Tq][H][d_v]; lse [B][Tq][H] or NULL.
 */
size_t csa2_sparse_attn_prefill_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d_v,
                                               int32_t k_top, int32_t W);
int csa2_sparse_attn_prefill(const float* q,
                             const uint8_t* kv_codes, int64_t c_batch_stride, int64_t c_row_stride,
                             const uint8_t* kv_scales, int64_t s_batch_stride, int64_t s_row_stride,
                             const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len,
                             const int32_t* q_pos,
                             const uint8_t* swa_vals, int64_t sv_batch_stride, int64_t sv_row_stride,
                             const uint8_t* swa_scales, int64_t ss_batch_stride, int64_t ss_row_stride,
                             const int32_t* swa_pos0, int32_t swa_rows, int32_t W, const float* sink,
                             int32_t B, int32_t Tq, int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                             float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * csa2_sparse_attn_paged -- the same attention over a serving-cache layout
 * (techniques map, technique tree: KV cache management; fact sheet: every
 * layer keeps its own 128-token window): the main KV rows of all sequences
 * live in one page pool, and each sequence's window is a ring.  Decode (Tq =
 * 1) and multi-query decode / prefill chunks (Tq > 1, one Top-K list per
 * query row).
 *   Page pool: rows 0 .. n_pages*page_size-1, row r at kv_codes +
 *     r*c_row_stride (d_qk/2 bytes) and kv_scales + r*s_row_stride (d_qk/16
 *     bytes).  Token j of sequence b is pool row
 *     block_table[b*bt_stride + j/page_size] * page_size + j % page_size.
 *     page_size: a power of two; n_pages * page_size < 2^31.  A Top-K id < 0
 *     or >= ctx_len[b], past the block table (j/page_size >= bt_stride) or
 *     on a block-table entry outside [0, n_pages) is skipped, never read.
 *   Ring window: swa_vals / swa_scales hold swa_ring rows per sequence (batch
 *     and row strides in bytes); window position x is ring row x % swa_ring,
 *     and swa_end[b] is one past the newest position written, so the ring
 *     holds positions swa_end[b]-swa_ring .. swa_end[b]-1.  The query at
 *     position p (q_pos[b][t]; NULL only when Tq == 1, then p =
 *     ctx_len[b]-1) sees window positions max(p-W+1, swa_end[b]-swa_ring, 0)
 *     .. min(p, swa_end[b]-1).
 * q [B][Tq][H][d_qk]; topk_idx [B][Tq][k_top] (token ids); out
 * [B][Tq][H][d_v]; lse [B][Tq][H] or NULL.  Supported shapes and accuracy
 * as csa2_sparse_attn_decode; the result equals that of the linear layouts
 * holding the same rows.
 */
size_t csa2_sparse_attn_paged_workspace_size(int32_t B, int32_t Tq, int32_t H, int32_t d_v, int32_t k_top,
                                             int32_t W);
int csa2_sparse_attn_paged(const float* q,
                           const uint8_t* kv_codes, int64_t c_row_stride,
                           const uint8_t* kv_scales, int64_t s_row_stride,
                           const int32_t* block_table, int64_t bt_stride, int32_t page_size, int32_t n_pages,
                           const int32_t* topk_idx, int32_t k_top, const int32_t* ctx_len, const int32_t* q_pos,
                           const uint8_t* swa_vals, int64_t sv_batch_stride, int64_t sv_row_stride,
                           const uint8_t* swa_scales, int64_t ss_batch_stride, int64_t ss_row_stride,
                           int32_t swa_ring, const int32_t* swa_end, int32_t W, const float* sink,
                           int32_t B, int32_t Tq, int32_t H, int32_t d_qk, int32_t d_v, float softmax_scale,
                           float* out, float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * Kernel trace for measurement harnesses.  While a trace is attached to the
 * calling host thread, each kernel the library launches from that thread
 * carries events[2*i] and events[2*i+1] as the start and stop events of its
 * dispatch (hipExtLaunchKernelGGL; the elapsed time between them is the
 * kernel's execution, and no separate event record is put on the stream) for
 * the i-th launch (HOST array of hipEvent_t created by the caller), and
 * names[i] (HOST array, nullable) receives the kernel's static name.
 * Launches past `capacity` are counted but not recorded.
 * csa2_trace_detach returns the number of launches since attach through
 * *n_launches (nullable) and stops recording.
 */
int csa2_trace_attach(void** events, const char** names, int32_t capacity);
/*
 * Restrict the attached trace of the calling thread to launches whose static
 * kernel name equals kernel_name (at most 63 characters; NULL = every
 * launch again); other launches are neither recorded nor counted.  Returns
 * CSA2_EINVAL when no trace is attached or the name is too long.
 */
int csa2_trace_only(const char* kernel_name);
int csa2_trace_detach(int32_t* n_launches);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H */
