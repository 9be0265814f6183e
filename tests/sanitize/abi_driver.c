/*
 * Drives the argument validation of libsparse_attn's C ABI (include/sparse_attn.h)
 * in a build whose host code carries AddressSanitizer and
 * UndefinedBehaviorSanitizer.  Every call here must be refused before the
 * library touches a device (no GPU is needed): null pointers, bad shapes,
 * misalignment, bad enums, NaN parameters, malformed segment lists, oversize
 * workspaces.  The error text is read back after each call, and the workspace
 * size query, which is pure host arithmetic, is checked on valid shapes.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "sparse_attn.h"

static int g_fail = 0;

static void expect(int32_t got, int32_t want, const char* what) {
  const char* msg = sa_last_error();
  if (got != want) {
    fprintf(stderr, "%s: status %d, expected %d (%s)\n", what, got, want, msg);
    g_fail = 1;
  } else if (want != SA_OK && (msg == NULL || strlen(msg) == 0)) {
    fprintf(stderr, "%s: no error text\n", what);
    g_fail = 1;
  }
}

static sa_dims dims(int B, int H, int Lq, int Lkv, int d, int lqv, int lkvv, int Lv) {
  sa_dims x = {B, H, Lq, Lkv, d, lqv, lkvv, Lv};
  return x;
}

static sa_route_params params(float thr, int G, int prefix, int kb, int ksr, int vsr, int mkb, int rule, float sp,
                              int nseg, const sa_segment* seg) {
  sa_route_params p;
  memset(&p, 0, sizeof p);
  p.threshold = thr;
  p.centroids_per_block = G;
  p.prefix_tokens = prefix;
  p.kblock = kb;
  p.k_scale_rows = ksr;
  p.v_scale_rows = vsr;
  p.map_kblock = mkb;
  p.rule = rule;
  p.sparsity = sp;
  p.n_segments = nseg;
  p.segments_host = seg;
  return p;
}

int main(void) {
  void* P = (void*)(uintptr_t)4096;       /* never dereferenced: every call below is refused first */
  void* odd = (void*)(uintptr_t)4104;     /* 8 bytes off a 16-byte boundary */
  if (sa_abi_version() != SA_ABI_VERSION) {
    fprintf(stderr, "ABI version mismatch\n");
    return 1;
  }
  /* quantize */
  expect(quantize_qk_int8(NULL, 0, 0, 128, 1, 1, 128, 128, 128, 128, P, P, NULL, 32, NULL), SA_E_NULL, "q null");
  expect(quantize_qk_int8(P, 0, 0, 128, 1, 1, 128, 96, 128, 128, P, P, NULL, 32, NULL), SA_E_SHAPE, "q d");
  expect(quantize_qk_int8(P, 0, 0, 128, 1, 1, 128, 128, 128, 32, P, P, NULL, 32, NULL), SA_E_VALUE, "q R");
  expect(quantize_qk_int8(P, 0, 0, 128, 1, 1, 100, 128, 100, 64, P, P, NULL, 32, NULL), SA_E_SHAPE, "q L");
  expect(quantize_qk_int8(P, 0, 0, 128, 1, 1, 128, 128, 129, 64, P, P, NULL, 32, NULL), SA_E_SHAPE, "q valid");
  expect(quantize_qk_int8(odd, 0, 0, 128, 1, 1, 128, 128, 128, 64, P, P, NULL, 32, NULL), SA_E_ALIGN, "q align");
  expect(quantize_qk_int8(P, 0, 0, 100, 1, 1, 128, 128, 128, 64, P, P, NULL, 32, NULL), SA_E_ALIGN, "q stride");
  expect(quantize_qk_int8(P, 0, 0, 128, 1, 1, 128, 128, 128, 64, P, P, odd, 32, NULL), SA_E_ALIGN, "q sums align");
  expect(quantize_qk_int8(P, 0, 0, 128, 1, 1, 128, 128, 128, 64, P, P, P, 48, NULL), SA_E_VALUE, "q sum_rows");
  /* cache append */
  expect(kv_cache_append_int8(P, 0, 0, 128, 1, 1, 256, 128, 256, 128, P, P, 1, 0, NULL), SA_E_SHAPE, "c slots");
  expect(kv_cache_append_int8(P, 0, 0, 128, 1, 1, 128, 128, 128, 128, P, P, 4, 4, NULL), SA_E_VALUE, "c first");
  /* route */
  {
    sa_dims dm = dims(1, 2, 256, 512, 128, 256, 500, 512);
    sa_route_params p = params(1.0f, 1, 0, 64, 64, 128, 64, SA_RULE_THRESHOLD, 0.0f, 0, NULL);
    const size_t ws = sparse_attn_route_workspace_size(&dm, &p, 0);
    if (ws != (size_t)(2 * 2 * 2 * 128 + 2 * 8 * 2 * 128)) {
      fprintf(stderr, "workspace size %zu\n", ws);
      g_fail = 1;
    }
    if (sparse_attn_route_workspace_size(&dm, &p, 1) != 0) g_fail = 1;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, 16, NULL),
           SA_E_WORKSPACE, "r workspace small");
    expect(sparse_attn_route(NULL, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws,
                             NULL),
           SA_E_NULL, "r q null");
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, odd, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_ALIGN, "r ksums align");
    p.threshold = NAN;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_VALUE, "r nan");
    p.threshold = 1.0f;
    p.rule = SA_RULE_TOPK;
    p.sparsity = 1.5f;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_VALUE, "r sparsity");
    p.rule = 7;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_VALUE, "r rule");
    p.rule = SA_RULE_THRESHOLD;
    const sa_segment bad1[2] = {{0, 64, 0}, {100, 64, 1}};
    const sa_segment bad2[2] = {{0, 100, 0}, {64, 64, 1}};
    sa_segment many[SA_MAX_SEGMENTS + 1];
    for (int x = 0; x <= SA_MAX_SEGMENTS; ++x) many[x] = (sa_segment){64 * x, 1, 0};
    p.n_segments = 2;
    p.segments_host = bad1;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_VALUE, "r seg start");
    p.segments_host = bad2;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_VALUE, "r seg overlap");
    p.n_segments = SA_MAX_SEGMENTS + 1;
    p.segments_host = many;
    expect(sparse_attn_route(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &dm, &p, NULL, P, P, P, P, NULL, P, ws, NULL),
           SA_E_VALUE, "r seg count");
    p.n_segments = 0;
    p.segments_host = NULL;
    /* oversize for the library-owned workspace */
    sa_dims big = dims(1, 128, 32768, 32768, 128, 32768, 32768, 32768);
    expect(sparse_attn_route_noalloc(P, P, P, P, SA_BF16, NULL, NULL, NULL, NULL, &big, &p, NULL, P, P, P, P, NULL,
                                     NULL),
           SA_E_WORKSPACE, "noalloc size");
  }
  /* forward */
  {
    sa_dims dm = dims(1, 2, 256, 512, 96, 256, 512, 512);
    sa_route_params p = params(1.0f, 1, 0, 64, 64, 128, 64, SA_RULE_THRESHOLD, 0.0f, 0, NULL);
    expect(sparse_attn_fwd(P, P, P, P, P, SA_BF16, NULL, NULL, &dm, &p, P, P, P, P, 0.125f, P, SA_F32, NULL, NULL),
           SA_E_SHAPE, "f d");
    dm.d = 128;
    expect(sparse_attn_fwd(P, P, P, P, P, SA_BF16, NULL, NULL, &dm, &p, P, P, P, P, -1.0f, P, SA_F32, NULL, NULL),
           SA_E_VALUE, "f sm");
    expect(sparse_attn_fwd(P, P, P, P, P, SA_INT8, NULL, NULL, &dm, &p, P, P, P, P, 0.125f, P, SA_F32, NULL, NULL),
           SA_E_NULL, "f vscale");
    expect(sparse_attn_fwd(P, P, P, P, P, SA_BF16, NULL, NULL, &dm, &p, P, NULL, P, P, 0.125f, P, SA_F32, NULL, NULL),
           SA_E_NULL, "f centroids");
    expect(sparse_attn_fwd(P, P, P, P, P, SA_BF16, NULL, NULL, &dm, &p, P, P, P, P, 0.125f, P, 9, NULL, NULL),
           SA_E_VALUE, "f out dtype");
    expect(sparse_attn_fwd_float(P, P, odd, NULL, &dm, &p, P, P, P, P, 0.125f, P, SA_F32, NULL, NULL), SA_E_ALIGN,
           "ff align");
  }
  /* virtual-KV gather */
  {
    const int32_t src[3] = {0, 1, 2};
    expect(gather_virtual_kv(P, 1, 1, 128, 2, 128, src, 3, P, P, 0, 16, 64, P, P, P, NULL), SA_E_VALUE, "g src");
    expect(gather_virtual_kv(P, 1, 1, 100, 2, 128, src, 2, P, P, 0, 16, 64, P, P, P, NULL), SA_E_SHAPE, "g rows");
    expect(gather_virtual_kv(P, 1, 1, 128, 2, 128, src, 2, P, P, 1, 16, 64, P, P, P, NULL), SA_E_VALUE, "g rot");
  }
  if (g_fail) return 1;
  printf("abi driver: every invalid call refused with a message\n");
  return 0;
}
