/*
 * Host-side driver of the C ABI for the sanitizer build (AddressSanitizer +
 * UndefinedBehaviorSanitizer on the host code only).  It exercises the
 * validation of every entry point (null pointers, shapes, strides,
 * alignment, workspace sizes, unsupported shapes) and the workspace-size
 * arithmetic at the largest supported sizes.  With no GPU visible, calls
 * whose arguments pass validation stop at their first HIP launch and return
 * CSA2_EHIP; those calls are made only when the runtime reports no device,
 * since their pointers are host memory.
 *
 * Exit status 0 when every status matches; the sanitizers abort on a report.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "csa2.h"

int hipGetDeviceCount(int* count);   /* from the HIP runtime */

static int g_fail = 0, g_n = 0;

#define EXPECT(call, want)                                                             \
  do {                                                                                 \
    int got_ = (call);                                                                 \
    ++g_n;                                                                             \
    if (got_ != (want)) {                                                              \
      fprintf(stderr, "line %d: %s -> %d (%s), expected %d\n", __LINE__, #call, got_, \
              csa2_status_string(got_), (int)(want));                                  \
      ++g_fail;                                                                        \
    }                                                                                  \
  } while (0)

#define EXPECT_TRUE(cond)                                            \
  do {                                                               \
    ++g_n;                                                           \
    if (!(cond)) {                                                   \
      fprintf(stderr, "line %d: %s is false\n", __LINE__, #cond);    \
      ++g_fail;                                                      \
    }                                                                \
  } while (0)

static void* buf(size_t n) {
  void* p = aligned_alloc(256, (n + 255) / 256 * 256);
  if (!p) {
    fprintf(stderr, "host allocation failed\n");
    exit(2);
  }
  memset(p, 0, (n + 255) / 256 * 256);
  return p;
}

int main(void) {
  int n_dev = -1;
  const int no_device = hipGetDeviceCount(&n_dev) != 0 || n_dev == 0;
  const int launch = no_device ? CSA2_EHIP : -1;   /* expected status of a valid call */

  /* status strings and version */
  for (int s = -2; s < 9; ++s) EXPECT_TRUE(csa2_status_string(s) != NULL && strlen(csa2_status_string(s)) > 0);
  EXPECT_TRUE(strcmp(csa2_status_string(CSA2_OK), "ok") == 0);
  EXPECT_TRUE(csa2_version() != NULL);

  /* ------------------------------------------------------------ quantisers */
  float* x = (float*)buf(4 * 576 * 4);
  uint8_t* c8 = (uint8_t*)buf(4 * 576);
  uint8_t* s8 = (uint8_t*)buf(4 * 64);
  EXPECT(kv_fp4_quantize(x, 0, 576, 576, c8, 288, s8, 36, NULL), CSA2_OK);
  EXPECT(kv_fp4_quantize(x, -1, 576, 576, c8, 288, s8, 36, NULL), CSA2_EINVAL);
  EXPECT(kv_fp4_quantize(x, 4, 8, 576, c8, 288, s8, 36, NULL), CSA2_EINVAL);
  EXPECT(kv_fp4_quantize(NULL, 4, 576, 576, c8, 288, s8, 36, NULL), CSA2_EINVAL);
  EXPECT(kv_fp4_quantize(x, 4, 576, 575, c8, 288, s8, 36, NULL), CSA2_EINVAL);
  EXPECT(kv_fp4_quantize(x, 4, 576, 576, c8 + 1, 288, s8, 36, NULL), CSA2_EINVAL);
  EXPECT(kv_fp4_quantize(x, 4, 576, 576, c8, 290, s8, 36, NULL), CSA2_EINVAL);
  EXPECT(kv_fp4_quantize(x, 4, 576, 576, c8, 288, s8, 35, NULL), CSA2_EINVAL);
  EXPECT(swa_fp8_quantize(x, 4, 48, 576, c8, 576, s8, 18, NULL), CSA2_EINVAL);
  EXPECT(swa_fp8_quantize(x, 4, 576, 576, c8, 575, s8, 18, NULL), CSA2_EINVAL);
  EXPECT(swa_fp8_quantize(x, 0, 576, 576, NULL, 576, NULL, 18, NULL), CSA2_OK);
  EXPECT(idx_mxfp4_quantize(x, 4, 128, 128, c8, 64, s8, 3, NULL), CSA2_EINVAL);
  EXPECT(idx_mxfp4_quantize(x, 4, 112, 128, c8, 64, s8, 4, NULL), CSA2_EINVAL);
  EXPECT(idx_mxfp4_quantize(x, 4, 128, 128, c8, 64, NULL, 4, NULL), CSA2_EINVAL);
  if (no_device) {
    EXPECT(kv_fp4_quantize(x, 4, 576, 576, c8, 288, s8, 36, NULL), launch);
    EXPECT(swa_fp8_quantize(x, 4, 576, 576, c8, 576, s8, 18, NULL), launch);
    EXPECT(idx_mxfp4_quantize(x, 4, 128, 128, c8, 64, s8, 4, NULL), launch);
  }

  /* -------------------------------------------------- workspace arithmetic */
  const int64_t sizes[] = {0, 1, 63, 64, 65, 4096, 65536, 65537, 131072, 266240, 1 << 20, 4 << 20};
  for (size_t i = 0; i < sizeof(sizes) / sizeof(sizes[0]); ++i) {
    const int64_t n = sizes[i];
    const size_t a = csa2_index_score_topk_workspace_size(64, 1, n, 2048, 0, 0);
    const size_t b = csa2_index_score_topk_workspace_size(64, 1, n + 1, 2048, 0, 0);
    const size_t p = csa2_index_score_topk_workspace_size(4, 1, n, 2048, 8, 2048);
    EXPECT_TRUE(a >= (size_t)64 * 4 * (size_t)n && p >= (size_t)4 * 4 * (size_t)n);
    EXPECT_TRUE(b + 4096 * 64 * 4 >= a);   /* the longer-row layout may drop the per-tile histograms */
  }
  for (size_t i = 0; i < sizeof(sizes) / sizeof(sizes[0]); ++i) {
    const int64_t n = sizes[i];
    const size_t full = csa2_index_score_topk_workspace_size_stored(1, 4096, n, 2048, 0, 0);
    const size_t bnd = csa2_index_score_topk_workspace_size(1, 4096, n, 2048, 0, 0);
    EXPECT_TRUE(bnd <= full && bnd < (size_t)100000000);
    EXPECT_TRUE(csa2_index_score_topk_workspace_size_stored(64, 1, n, 2048, 0, 0) ==
                csa2_index_score_topk_workspace_size(64, 1, n, 2048, 0, 0));
  }
  EXPECT_TRUE(csa2_index_score_topk_workspace_size_stored(-1, 16, 10, 1, 0, 0) == 0);
  EXPECT_TRUE(csa2_index_score_topk_workspace_size(-1, 1, 10, 1, 0, 0) == 0);
  EXPECT_TRUE(csa2_index_score_topk_workspace_size(1, 1, -10, 1, 0, 0) == 0);
  EXPECT_TRUE(csa2_hier_pool_topk_workspace_size(4, 1, 16384, 2048) >= (size_t)4 * 16384 * 4);
  EXPECT_TRUE(csa2_hier_pool_topk_workspace_size(-4, 1, 16384, 2048) == 0);
  EXPECT_TRUE(csa2_sparse_attn_decode_workspace_size(64, 64, 512, 2048, 128) >= (size_t)64 * 64 * 512 * 4);
  EXPECT_TRUE(csa2_sparse_attn_decode_workspace_size(64, 0, 512, 2048, 128) == 0);
  EXPECT_TRUE(csa2_sparse_attn_prefill_workspace_size(1, 4096, 64, 512, 2048, 128) > 0);
  EXPECT_TRUE(csa2_sparse_attn_paged_workspace_size(65535, 1, 64, 512, 2048, 128) > 0);

  /* --------------------------------------------------------- index scoring */
  const int B = 2, Tq = 1, HI = 8, DI = 128, K = 64;
  const int64_t N = 1000;
  uint8_t* q = (uint8_t*)buf(B * Tq * HI * DI);
  float* w = (float*)buf(B * Tq * HI * 4);
  uint8_t* k = (uint8_t*)buf(B * N * DI);
  int32_t* ctx = (int32_t*)buf(B * 4);
  int32_t* idx = (int32_t*)buf(B * Tq * 4096 * 4);
  int32_t* pidx = (int32_t*)buf(B * Tq * 4096 * 4);
  int32_t* plen = (int32_t*)buf(B * Tq * 4);
  size_t wsz = csa2_index_score_topk_workspace_size(B, Tq, N, K, 8, 64);
  void* ws = buf(wsz + 512);
  const int64_t rs = DI, bs = N * DI;
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, 0, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                               NULL), CSA2_OK);
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, 0, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                               NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk(NULL, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws,
                               wsz, NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL,
                               (char*)ws + 16, wsz, NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk(q, w, k, bs, 120, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                               NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk(q, w, k, bs, 136, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                               NULL), CSA2_EINVAL);   /* not 16-byte rows at D_I = 128 */
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, 33, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                               NULL), CSA2_EUNSUPPORTED);
  EXPECT(csa2_index_score_topk(q, w, k, bs, 96, ctx, NULL, B, Tq, HI, 96, N, K, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                               NULL), CSA2_EUNSUPPORTED);
  EXPECT(csa2_index_score_topk(q, w, k, bs, (int64_t)1 << 22, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL,
                               NULL, ws, wsz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws,
                               csa2_index_score_topk_workspace_size(B, Tq, N, K, 0, 0) - 1, NULL), CSA2_EWORKSPACE);
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 3, 64, pidx, plen, ws, wsz,
                               NULL), CSA2_EINVAL);   /* pool block not a power of two <= 16 */
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 8, 64, pidx, NULL, ws, wsz,
                               NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, 65536, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws,
                               wsz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(csa2_index_score_topk_noalloc(q, w, k, bs, rs, ctx, NULL, 64, 1, HI, DI, (int64_t)1 << 20, K, idx, NULL, 0,
                                       0, NULL, NULL, NULL), CSA2_ESCRATCH);
  /* MXFP4 keys: 16-byte code rows, 4-byte scale rows, D_I = 128 */
  uint8_t* kc = (uint8_t*)buf(B * N * 64);
  uint8_t* ks = (uint8_t*)buf(B * N * 4);
  EXPECT(csa2_index_score_topk_mxfp4(q, w, kc, N * 64, 64, NULL, N * 4, 4, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL,
                                     0, 0, NULL, NULL, ws, wsz, NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk_mxfp4(q, w, kc + 4, N * 64, 64, ks, N * 4, 4, ctx, NULL, B, Tq, HI, DI, N, K, idx,
                                     NULL, 0, 0, NULL, NULL, ws, wsz, NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk_mxfp4(q, w, kc, N * 64, 64, ks + 1, N * 4, 4, ctx, NULL, B, Tq, HI, DI, N, K, idx,
                                     NULL, 0, 0, NULL, NULL, ws, wsz, NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk_mxfp4(q, w, kc, N * 64, 64, ks, N * 4, 2, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL,
                                     0, 0, NULL, NULL, ws, wsz, NULL), CSA2_EINVAL);
  EXPECT(csa2_index_score_topk_mxfp4(q, w, kc, N * 32, 32, ks, N * 4, 4, ctx, NULL, B, Tq, HI, 64, N, K, idx, NULL,
                                     0, 0, NULL, NULL, ws, wsz, NULL), CSA2_EUNSUPPORTED);
  if (no_device) {
    EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 0, 0, NULL, NULL, ws, wsz,
                                 NULL), launch);
    EXPECT(csa2_index_score_topk(q, w, k, bs, rs, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL, 8, 64, pidx, plen, ws,
                                 wsz, NULL), launch);
    EXPECT(csa2_index_score_topk_mxfp4(q, w, kc, N * 64, 64, ks, N * 4, 4, ctx, NULL, B, Tq, HI, DI, N, K, idx, NULL,
                                       0, 0, NULL, NULL, ws, wsz, NULL), launch);
  }

  /* ------------------------------------------------------------ pool layer */
  const int cap = 512;
  size_t psz = csa2_hier_pool_topk_workspace_size(B, Tq, cap, K);
  void* pws = buf(psz);
  EXPECT(csa2_hier_pool_topk(q, w, k, bs, rs, ctx, NULL, plen, cap, B, Tq, HI, DI, K, idx, NULL, pws, psz, NULL),
         CSA2_EINVAL);
  EXPECT(csa2_hier_pool_topk(q, w, k, bs, rs, ctx, pidx, plen, cap, B, Tq, HI, DI, K, idx, NULL, pws, psz - 1, NULL),
         CSA2_EWORKSPACE);
  EXPECT(csa2_hier_pool_topk(q, w, k, bs, rs, ctx, pidx, plen, -1, B, Tq, HI, DI, K, idx, NULL, pws, psz, NULL),
         CSA2_EINVAL);
  EXPECT(csa2_hier_pool_topk_mxfp4(q, w, kc, N * 64, 128, ks, N * 4, 8, ctx, pidx, plen, cap, B, Tq, HI, 256, K, idx,
                                   NULL, pws, psz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(csa2_hier_pool_topk_mxfp4(q, w, kc, N * 64, 64, ks, N * 4, 4, ctx, pidx, plen, cap, B, Tq, HI, 256, K, idx,
                                   NULL, pws, psz, NULL), CSA2_EINVAL);   /* code rows below D_I / 2 */
  if (no_device) {
    EXPECT(csa2_hier_pool_topk(q, w, k, bs, rs, ctx, pidx, plen, cap, B, Tq, HI, DI, K, idx, NULL, pws, psz, NULL),
           launch);
    EXPECT(csa2_hier_pool_topk_mxfp4(q, w, kc, N * 64, 64, ks, N * 4, 4, ctx, pidx, plen, cap, B, Tq, HI, DI, K, idx,
                                     NULL, pws, psz, NULL), launch);
  }

  /* ------------------------------------------------------------- attention */
  const int H = 64, d = 576, dv = 512, W = 128, Ka = 256, R = 64;
  float* qa = (float*)buf((size_t)B * 4 * H * d * 4);
  uint8_t* cache = (uint8_t*)buf((size_t)B * R * 324 + 1024);
  uint8_t* sv = (uint8_t*)buf((size_t)B * W * d);
  uint8_t* ss = (uint8_t*)buf((size_t)B * W * 18);
  int32_t* swl = (int32_t*)buf(B * 4);
  int32_t* qpos = (int32_t*)buf(B * 4 * 4);
  int32_t* bt = (int32_t*)buf(B * 16 * 4);
  float* out = (float*)buf((size_t)B * 4 * H * dv * 4);
  float* lse = (float*)buf((size_t)B * 4 * H * 4);
  float* cs = (float*)buf((size_t)B * 64 * 4);
  size_t asz = csa2_sparse_attn_prefill_workspace_size(B, 4, H, dv, Ka, W);
  size_t dsz = csa2_sparse_attn_decode_workspace_size(B, H, dv, Ka, W);
  void* aws = buf(asz > dsz ? asz : dsz);
  const int64_t cb = R * 324;
#define DEC(...) csa2_sparse_attn_decode(__VA_ARGS__)
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, 0, H,
             d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_OK);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, 40,
             d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, 128,
             d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, H,
             640, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);   /* row strides below 640 channels */
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, H,
             d, 256, 0.04f, out, lse, aws, dsz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(DEC(qa, cache, cb, 322, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, H,
             d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  EXPECT(DEC(qa, cache + 2, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL,
             B, H, d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, NULL, W * d, d, ss, W * 18, 18, swl, W, NULL, B,
             H, d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, NULL, W, NULL, B, H,
             d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, 0, ctx, sv, W * d, d, ss, W * 18, 18, swl, 0, NULL, B, H,
             d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);   /* no entries at all */
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, NULL, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B,
             H, d, dv, 0.04f, out, lse, aws, dsz, NULL), CSA2_EINVAL);   /* Top-K entries without ids */
  if (no_device)   /* the window alone: no Top-K ids needed */
    EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, NULL, 0, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B,
               H, d, dv, 0.04f, out, lse, aws, dsz, NULL), launch);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, H,
             d, dv, 0.04f, out, lse, (char*)aws + 64, dsz, NULL), CSA2_EINVAL);
  EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B, H,
             d, dv, 0.04f, out, lse, aws, dsz - 1, NULL), CSA2_EWORKSPACE);
  /* the pages' K = V row with the RoPE steps */
#define ROPE(...) csa2_sparse_attn_decode_rope(__VA_ARGS__)
  EXPECT(ROPE(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B,
              H, 576, 0.04f, cs, 64, 1, out, lse, aws, dsz, NULL), CSA2_EUNSUPPORTED);   /* only the 512 row */
  EXPECT(ROPE(qa, cache, cb, 288, cache + 256, cb, 288, idx, Ka, ctx, sv, W * 512, 512, ss, W * 16, 16, swl, W, NULL,
              B, H, 576, 0.04f, cs, 64, 1, out, lse, aws, dsz, NULL), CSA2_EINVAL);   /* window rows too short */
  EXPECT(ROPE(qa, cache, cb, 288, cache + 256, cb, 288, idx, Ka, ctx, sv, W * 512, 512, ss, W * 16, 16, swl, W, NULL,
              B, H, 512, 0.04f, cs, 62, 1, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  EXPECT(ROPE(qa, cache, cb, 288, cache + 256, cb, 288, idx, Ka, ctx, sv, W * 512, 512, ss, W * 16, 16, swl, W, NULL,
              B, H, 512, 0.04f, cs + 1, 64, 1, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  EXPECT(ROPE(qa, cache, cb, 288, cache + 256, cb, 288, idx, Ka, ctx, sv, W * 512, 512, ss, W * 16, 16, swl, W, NULL,
              B, H, 512, 0.04f, NULL, 64, 1, out, lse, aws, dsz, NULL), CSA2_EINVAL);
  /* prefill */
#define PRE(...) csa2_sparse_attn_prefill(__VA_ARGS__)
  EXPECT(PRE(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, qpos, W, W,
             NULL, B, 4, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);   /* q_pos required */
  EXPECT(PRE(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, qpos, sv, W * d, d, ss, W * 18, 18, NULL, W, W,
             NULL, B, 4, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);   /* window origin required */
  EXPECT(PRE(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, qpos, sv, W * d, d, ss, W * 18, 18, qpos, W, W,
             NULL, B, 40000, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(PRE(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, qpos, sv, W * d, d, ss, W * 18, 18, qpos, W, W,
             NULL, B, 4, H, d, dv, 0.04f, out, lse, aws, asz - 1, NULL), CSA2_EWORKSPACE);
  /* paged */
#define PAG(...) csa2_sparse_attn_paged(__VA_ARGS__)
  EXPECT(PAG(qa, cache, 324, cache + 288, 324, bt, 16, 48, 8, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, W,
             swl, W, NULL, B, 1, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);   /* page not 2^k */
  EXPECT(PAG(qa, cache, 324, cache + 288, 324, NULL, 16, 64, 8, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, W,
             swl, W, NULL, B, 1, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);
  EXPECT(PAG(qa, cache, 324, cache + 288, 324, bt, 16, 64, 0, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, W,
             swl, W, NULL, B, 1, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);
  EXPECT(PAG(qa, cache, 324, cache + 288, 324, bt, 16, 1 << 20, 4096, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18,
             18, W, swl, W, NULL, B, 1, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EUNSUPPORTED);
  EXPECT(PAG(qa, cache, 324, cache + 288, 324, bt, 16, 64, 8, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, W,
             swl, W, NULL, B, 2, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);   /* Tq > 1 needs q_pos */
  EXPECT(PAG(qa, cache, 324, cache + 288, 324, bt, 16, 64, 8, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, 0,
             swl, W, NULL, B, 1, H, d, dv, 0.04f, out, lse, aws, asz, NULL), CSA2_EINVAL);   /* empty ring */
  if (no_device) {
    EXPECT(DEC(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, sv, W * d, d, ss, W * 18, 18, swl, W, NULL, B,
               H, d, dv, 0.04f, out, lse, aws, dsz, NULL), launch);
    EXPECT(ROPE(qa, cache, cb, 288, cache + 256, cb, 288, idx, Ka, ctx, sv, W * 512, 512, ss, W * 16, 16, swl, W,
                NULL, B, H, 512, 0.04f, cs, 64, 1, out, lse, aws, dsz, NULL), launch);
    EXPECT(PRE(qa, cache, cb, 324, cache + 288, cb, 324, idx, Ka, ctx, qpos, sv, W * d, d, ss, W * 18, 18, qpos, W, W,
               NULL, B, 4, H, d, dv, 0.04f, out, lse, aws, asz, NULL), launch);
    EXPECT(PAG(qa, cache, 324, cache + 288, 324, bt, 16, 64, 8, idx, Ka, ctx, NULL, sv, W * d, d, ss, W * 18, 18, W,
               swl, W, NULL, B, 1, H, d, dv, 0.04f, out, lse, aws, asz, NULL), launch);
  }

  /* ----------------------------------------------------------------- trace */
  void* events[8] = {0};
  const char* names[4] = {0};
  int32_t nl = -1;
  EXPECT(csa2_trace_only("index_score"), CSA2_EINVAL);   /* nothing attached */
  EXPECT(csa2_trace_attach(events, names, 4), CSA2_OK);
  char longname[80];
  memset(longname, 'a', sizeof(longname) - 1);
  longname[sizeof(longname) - 1] = 0;
  EXPECT(csa2_trace_only(longname), CSA2_EINVAL);
  EXPECT(csa2_trace_only("index_score"), CSA2_OK);
  EXPECT(csa2_trace_only(NULL), CSA2_OK);
  EXPECT(csa2_trace_detach(&nl), CSA2_OK);
  EXPECT_TRUE(nl == 0);

  printf("host ABI driver: %d checks, %d failed, device calls %s\n", g_n, g_fail,
         no_device ? "checked (no device)" : "skipped (device present)");
  free(x); free(c8); free(s8); free(q); free(w); free(k); free(ctx); free(idx); free(pidx); free(plen); free(ws);
  free(kc); free(ks); free(pws); free(qa); free(cache); free(sv); free(ss); free(swl); free(qpos); free(bt); free(out);
  free(lse); free(cs); free(aws);
  return g_fail ? 1 : 0;
}
