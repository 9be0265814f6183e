/*
 * Runs every entry point of the CPU oracle (oracle/oracle.c) on small ragged
 * inputs in buffers of exactly the documented sizes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: any read or write past a
 * buffer, use of freed memory, signed overflow or misaligned access aborts
 * the run.  The numbers themselves are checked by the Python pins; this only
 * checks the memory and arithmetic behaviour of the code paths: quantization
 * with padding, the streaming cache with wrap-around, routing under both rules
 * with a prefix, with segments and with explicit maps (G = 0, 1, 2; 64- and
 * 128-row key blocks; INT8 V through a virtual-KV block table), the forward on
 * the INT8 and floating paths, and the virtual-KV gather.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_quantize(const uint16_t* x, int64_t sB, int64_t sH, int64_t sL, int B, int H, int L, int d, int valid_len,
                  int R, int8_t* q, float* scale);
int orc_cache_append(const uint16_t* x, int64_t sB, int64_t sH, int64_t sL, int B, int H, int rows, int d,
                     int valid_len, int R, int8_t* cache_q, float* cache_scale, int slots, int first_slot);
int orc_route(const int8_t* q, const int8_t* k, const float* k_scale, int k_scale_rows, const uint16_t* v_bf16,
              const int8_t* v_i8, const float* v_scale, int v_scale_rows, const int32_t* v_block_src, int Lv, int B,
              int H, int Lq, int Lkv, int d, int lq_valid, int lkv_valid, int rule, double tau, double sparsity, int G,
              int prefix, int kblock, const int32_t* seg, int nseg, const uint8_t* explicit_map, int map_kblock,
              uint8_t* map, double* kbar, double* vbar, double* count, double* stats, uint8_t* tie);
void orc_forward(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale, int k_scale_rows,
                 const uint16_t* v_bf16, const int8_t* v_i8, const float* v_scale, int v_scale_rows,
                 const int32_t* v_block_src, int Lv, int B, int H, int Lq, int Lkv, int d, int lq_valid, int lkv_valid,
                 int kblock, const int32_t* seg, int nseg, int G, const uint8_t* map, const double* kbar,
                 const double* vbar, const double* count, double sm_scale, const int64_t* sel, int nsel, double* out,
                 double* lse, const uint16_t* q_bf16, const uint16_t* k_bf16);
void orc_materialize_virtual_k(const uint16_t* k_phys, int B, int H, int S, int n_phys, int d, const int32_t* src,
                               int n_logical, const float* cosv, const float* sinv, int rot_offset, int d_rot,
                               uint16_t* k_log);
void orc_gather_virtual_kv(const uint16_t* k_phys, int B, int H, int S, int n_phys, int d, const int32_t* src,
                           int n_logical, const float* cosv, const float* sinv, int rot_offset, int d_rot, int R,
                           int8_t* k_q, float* k_scale, int32_t* v_block_src);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static uint32_t next_u32(void) {
  g_state ^= g_state << 13;
  g_state ^= g_state >> 7;
  g_state ^= g_state << 17;
  return (uint32_t)(g_state >> 16);
}

/* bf16 bits of a value in [-2, 2) */
static uint16_t rand_bf16(void) {
  float f = ((float)(next_u32() & 0xFFFF) / 32768.0f - 1.0f) * 2.0f;
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)(u >> 16);
}

static void* xmalloc(size_t n) {
  void* p = malloc(n ? n : 1);
  if (!p) {
    fprintf(stderr, "out of memory\n");
    exit(2);
  }
  return p;
}

static uint16_t* rand_tensor(size_t n) {
  uint16_t* x = (uint16_t*)xmalloc(n * sizeof(uint16_t));
  for (size_t i = 0; i < n; ++i) x[i] = rand_bf16();
  return x;
}

#define CHECK(c)                                             \
  do {                                                       \
    if (!(c)) {                                              \
      fprintf(stderr, "check failed: %s (line %d)\n", #c, __LINE__); \
      exit(1);                                               \
    }                                                        \
  } while (0)

/* One routing + forward case: B = 1, H = 2, d; query and key lengths Lq,
 * Lkv (multiples of 128) with valid lengths; kblock; G; rule or explicit map;
 * optional segments; V bf16 or INT8 (optionally through a block table over a
 * shorter physical V); the INT8 or floating QK forward. */
static void run_case(int d, int Lq, int Lkv, int lq_valid, int lkv_valid, int kblock, int G, int rule, int explicit,
                     const int32_t* seg, int nseg, int prefix, int v_int8, int virt, int qk_float) {
  const int B = 1, H = 2;
  const int Lv = virt ? Lkv / 2 : Lkv;
  const int nQB = Lq / 128, nKB = Lkv / kblock, Gs = G > 0 ? G : 1;
  const int ksr = kblock, vsr = 128;
  uint16_t* q = rand_tensor((size_t)B * H * Lq * d);
  uint16_t* k = rand_tensor((size_t)B * H * Lkv * d);
  uint16_t* v = rand_tensor((size_t)B * H * Lv * d);
  int8_t* q8 = (int8_t*)xmalloc((size_t)B * H * Lq * d);
  float* qs = (float*)xmalloc(sizeof(float) * B * H * nQB);
  int8_t* k8 = (int8_t*)xmalloc((size_t)B * H * Lkv * d);
  float* ks = (float*)xmalloc(sizeof(float) * B * H * (Lkv / ksr));
  orc_quantize(q, (int64_t)H * Lq * d, (int64_t)Lq * d, d, B, H, Lq, d, lq_valid, 128, q8, qs);
  orc_quantize(k, (int64_t)H * Lkv * d, (int64_t)Lkv * d, d, B, H, Lkv, d, lkv_valid, ksr, k8, ks);
  int8_t* v8 = NULL;
  float* vs = NULL;
  if (v_int8) {
    v8 = (int8_t*)xmalloc((size_t)B * H * Lv * d);
    vs = (float*)xmalloc(sizeof(float) * B * H * (Lv / vsr));
    orc_quantize(v, (int64_t)H * Lv * d, (int64_t)Lv * d, d, B, H, Lv, d, Lv, vsr, v8, vs);
  }
  int32_t* vbs = NULL;
  if (virt) {
    vbs = (int32_t*)xmalloc(sizeof(int32_t) * (Lkv / 64));
    for (int j = 0; j < Lkv / 64; ++j) vbs[j] = (int32_t)(next_u32() % (uint32_t)(Lv / 64));
  }
  uint8_t* em = NULL;
  const int mk = kblock;
  if (explicit) {
    em = (uint8_t*)xmalloc((size_t)B * H * nQB * (Lkv / mk));
    for (size_t i = 0; i < (size_t)B * H * nQB * (Lkv / mk); ++i) em[i] = (uint8_t)(next_u32() % 4); /* incl. 3 */
  }
  uint8_t* map = (uint8_t*)xmalloc((size_t)B * H * nQB * nKB);
  uint8_t* tie = (uint8_t*)xmalloc((size_t)B * H * nQB * nKB);
  double* kbar = (double*)xmalloc(sizeof(double) * B * H * nKB * Gs * d);
  double* vbar = (double*)xmalloc(sizeof(double) * B * H * nKB * Gs * d);
  double* cnt = (double*)xmalloc(sizeof(double) * B * H * nKB * Gs);
  double* stats = (double*)xmalloc(sizeof(double) * B * H * nQB * 2);
  int rc = orc_route(q8, k8, ks, ksr, v_int8 ? NULL : v, v8, vs, vsr, vbs, Lv, B, H, Lq, Lkv, d, lq_valid, lkv_valid,
                     rule, 0.5, 0.6, G, prefix, kblock, seg, nseg, em, mk, map, kbar, vbar, cnt, stats, tie);
  CHECK(rc == 0);
  for (size_t i = 0; i < (size_t)B * H * nQB * nKB; ++i) CHECK(map[i] <= 2);
  const int nsel = B * H * nQB;
  int64_t* sel = (int64_t*)xmalloc(sizeof(int64_t) * nsel);
  for (int i = 0; i < nsel; ++i) sel[i] = i;
  double* out = (double*)xmalloc(sizeof(double) * nsel * 128 * d);
  double* lse = (double*)xmalloc(sizeof(double) * nsel * 128);
  orc_forward(q8, qs, k8, ks, ksr, v_int8 ? NULL : v, v8, vs, vsr, vbs, Lv, B, H, Lq, Lkv, d, lq_valid, lkv_valid,
              kblock, seg, nseg, G, map, kbar, vbar, cnt, 1.0 / sqrt((double)d), sel, nsel, out, lse,
              qk_float ? q : NULL, qk_float ? k : NULL);
  for (size_t i = 0; i < (size_t)nsel * 128 * d; ++i) CHECK(!isnan(out[i]));
  free(q); free(k); free(v); free(q8); free(qs); free(k8); free(ks); free(v8); free(vs); free(vbs); free(em);
  free(map); free(tie); free(kbar); free(vbar); free(cnt); free(stats); free(sel); free(out); free(lse);
}

int main(void) {
  /* routing rules, prefix, ragged ends, both key-block sizes, both d */
  run_case(64, 256, 512, 250, 500, 64, 1, 0, 0, NULL, 0, 0, 0, 0, 0);
  run_case(128, 384, 640, 300, 577, 64, 2, 0, 0, NULL, 0, 128, 0, 0, 0);
  run_case(128, 256, 768, 256, 700, 128, 1, 1, 0, NULL, 0, 0, 0, 0, 0);
  run_case(64, 256, 512, 200, 512, 64, 0, 1, 0, NULL, 0, 64, 0, 0, 0);
  run_case(128, 256, 512, 256, 512, 64, 2, 1, 0, NULL, 0, 0, 0, 0, 1); /* floating QK */
  /* segments: dense, padding gaps, routed */
  {
    const int32_t seg[] = {0, 77, 0, 128, 100, 1, 256, 190, 1};
    run_case(128, 512, 512, 500, 446, 64, 2, 0, 0, seg, 3, 0, 0, 0, 0);
    run_case(64, 512, 512, 512, 446, 64, 1, 1, 0, seg, 3, 0, 0, 0, 1);
  }
  /* explicit maps over an INT8 V cache, G = 0 and 2, and through a block table */
  run_case(128, 256, 512, 256, 512, 128, 0, 0, 1, NULL, 0, 0, 1, 0, 0);
  run_case(64, 256, 512, 256, 480, 64, 2, 0, 1, NULL, 0, 0, 1, 1, 0);
  run_case(128, 256, 512, 256, 512, 64, 2, 0, 1, NULL, 0, 0, 0, 1, 0);

  /* streaming cache: chunks with wrap-around and a partial last slab */
  {
    const int H = 2, d = 64, R = 128, slots = 5;
    int8_t* cq = (int8_t*)xmalloc((size_t)H * slots * R * d);
    float* cs = (float*)xmalloc(sizeof(float) * H * slots);
    int first = 0;
    for (int chunk = 0; chunk < 4; ++chunk) {
      const int rows = R * (1 + chunk % 3), valid = rows - (chunk == 3 ? 37 : 0);
      uint16_t* x = rand_tensor((size_t)H * rows * d);
      CHECK(orc_cache_append(x, (int64_t)H * rows * d, (int64_t)rows * d, d, 1, H, rows, d, valid, R, cq, cs, slots,
                             first) == 0);
      first = (first + rows / R) % slots;
      free(x);
    }
    free(cq);
    free(cs);
  }
  /* virtual-KV gather and its conservative materialization */
  {
    const int H = 2, S = 128, n_phys = 2, n_log = 5, d = 64, d_rot = 16;
    uint16_t* kp = rand_tensor((size_t)H * S * n_phys * d);
    const int32_t src[5] = {0, 1, 1, 0, 1};
    float* cs = (float*)xmalloc(sizeof(float) * n_log * d_rot / 2);
    float* sn = (float*)xmalloc(sizeof(float) * n_log * d_rot / 2);
    for (int i = 0; i < n_log * d_rot / 2; ++i) {
      cs[i] = cosf(0.1f * (float)i);
      sn[i] = sinf(0.1f * (float)i);
    }
    uint16_t* kl = (uint16_t*)xmalloc(sizeof(uint16_t) * H * S * n_log * d);
    orc_materialize_virtual_k(kp, 1, H, S, n_phys, d, src, n_log, cs, sn, 2, d_rot, kl);
    int8_t* k8 = (int8_t*)xmalloc((size_t)H * S * n_log * d);
    float* ks = (float*)xmalloc(sizeof(float) * H * S * n_log / 64);
    int32_t* vbs = (int32_t*)xmalloc(sizeof(int32_t) * S * n_log / 64);
    orc_gather_virtual_kv(kp, 1, H, S, n_phys, d, src, n_log, cs, sn, 2, d_rot, 64, k8, ks, vbs);
    for (int j = 0; j < S * n_log / 64; ++j) CHECK(vbs[j] >= 0 && vbs[j] < S * n_phys / 64);
    free(kp); free(cs); free(sn); free(kl); free(k8); free(ks); free(vbs);
  }
  printf("oracle driver: all cases ran\n");
  return 0;
}
