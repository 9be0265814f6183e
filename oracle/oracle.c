/*
 * CPU oracle for block-sparse INT8 video attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in __graft_entry__.py
 * and the cpu_baseline leg of bench.py may load this library.  The GPU path
 * (block_sparse_int8_amd) never calls, links or includes anything here, and this
 * file includes nothing of the GPU path.
 *
 * What it computes follows the pages' statement of the method:
 *   - Configure Sol Sparse Attention, "How it works": per 128-token query block,
 *     each 64-token K/V block is rated by an inexpensive proxy taken from the
 *     INT8 Q/K that the exact tiles also use; blocks rated above
 *     mean + routing_threshold * std are not computed exactly but become one 64-token
 *     centroid (1x64) or two 32-token centroids (2x32) that still enter the
 *     online softmax.
 *   - Configure Sol Sparse Attention, "The inputs that matter": routing_threshold
 *     (default 1.0) and a manually protected leading token prefix.
 *   - FlashVSR Sparge Attention, "How it works": routing on logical blocks,
 *     converted to the physical block geometry afterwards.
 *   - FlashVSR Kitchen Sparse Attention, opening section: K/V kept as an INT8
 *     cache in bounded 128-row slabs.
 *   - Configure H3 Static Virtual KV, mode list: seven logical K slices re-read
 *     from two physical bf16 slices through a source map, each with its own
 *     temporal rotary phase, materialized only as INT8.
 *
 * Arithmetic: attention logits, softmax and centroids in float64; the INT8 code
 * of each element is decided in float32 exactly as the GPU kernel decides it
 * (one IEEE division for 127/amax, one multiply, round-half-even); routing
 * proxies are exact integers turned into float64 with one multiply and one
 * divide.  Plain loops; OpenMP only across independent (batch, head) or query
 * blocks.  Compile with -ffp-contract=off so no product is fused behind our back.
 *
 * Parity status of each function is listed beside it ("pinned by" names the
 * kind of test that pins it; the proxy's relation to the real Sol proxy is
 * "parity unpinned" because the pages do not define the proxy).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_DROP 0
#define ORC_EXACT 1
#define ORC_CENTROID 2
#define QBLOCK 128

static float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, 4);
  return f;
}

static uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

/* ------------------------------------------------------------------------- */
/* Per-block symmetric INT8 quantization.                                     */
/* Configure Sol Sparse Attention, "How it works" (prequantized INT8 Q/K);    */
/* FlashVSR Kitchen Sparse Attention, opening section (128-row INT8 slabs).  */
/* For each block of R rows: amax over the valid rows; scale = amax/127;     */
/* code = round-half-even(x * (127/amax)) clamped to [-127, 127]; an all-zero */
/* block gets scale 0 and codes 0; rows at or past valid_len get code 0.     */
/* Pinned by: hand examples (round-half-even cases), error bound, range.     */
/* ------------------------------------------------------------------------- */
void orc_quantize(const uint16_t* x, int64_t sB, int64_t sH, int64_t sL, int B, int H, int L,
                  int d, int valid_len, int R, int8_t* q, float* scale) {
  int nblk = (L + R - 1) / R;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      for (int blk = 0; blk < nblk; ++blk) {
        int r0 = blk * R, r1 = r0 + R < L ? r0 + R : L;
        float amax = 0.0f;
        for (int r = r0; r < r1 && r < valid_len; ++r)
          for (int c = 0; c < d; ++c) {
            float v = fabsf(bf16_to_f32(x[b * sB + h * sH + r * sL + c]));
            if (v > amax) amax = v;
          }
        float s = 0.0f, inv = 0.0f;
        if (amax > 0.0f) {
          s = amax / 127.0f;
          inv = 127.0f / amax;
        }
        scale[((int64_t)b * H + h) * nblk + blk] = s;
        for (int r = r0; r < r1; ++r)
          for (int c = 0; c < d; ++c) {
            int8_t code = 0;
            if (r < valid_len && amax > 0.0f) {
              float y = rintf(bf16_to_f32(x[b * sB + h * sH + r * sL + c]) * inv);
              if (y > 127.0f) y = 127.0f;
              if (y < -127.0f) y = -127.0f;
              code = (int8_t)y;
            }
            q[(((int64_t)b * H + h) * L + r) * d + c] = code;
          }
      }
    }
}

/* Dequantized value of V at logical row r, channel c (bf16 or INT8 cache).
 * With a block source table, logical 64-row block r/64 reads physical block
 * v_block_src[r/64] (Configure H3 Static Virtual KV, mode list: V is never
 * copied, only re-read); an INT8 V takes the scale of the physical row.
 * Pinned by: route and forward through the table equal SDPA and numpy means on
 * a V materialized by concatenating the physical slices in source-map order,
 * and, for INT8 V with 64- and 128-row physical scales, the results on a
 * materialized INT8 V. */
typedef struct {
  const uint16_t* v_bf16;
  const int8_t* v_i8;
  const float* v_scale;
  int v_scale_rows;
  const int32_t* v_block_src;
  int Lv;
  int H;
  int d;
} orc_vsrc;

static double v_at(const orc_vsrc* s, int b, int h, int r, int c) {
  int pr = s->v_block_src ? s->v_block_src[r / 64] * 64 + (r % 64) : r;
  int64_t idx = (((int64_t)b * s->H + h) * s->Lv + pr) * s->d + c;
  if (s->v_bf16) return (double)bf16_to_f32(s->v_bf16[idx]);
  int nvb = (s->Lv + s->v_scale_rows - 1) / s->v_scale_rows;
  return (double)s->v_i8[idx] * (double)s->v_scale[((int64_t)b * s->H + h) * nvb + pr / s->v_scale_rows];
}

/* ------------------------------------------------------------------------- */
/* Streaming INT8 K/V cache (FlashVSR Kitchen Sparse Attention, opening      */
/* section: in streaming use each block holds the recent K/V history as    */
/* INT8, bounded, in 128-row slabs).  The cache is a ring of                 */
/* `slots` slabs of R rows per (b, h).  A chunk of `rows` new rows is        */
/* quantized per slab of R rows exactly as orc_quantize does (rows at or     */
/* past valid_len are padding), and slab s of the chunk replaces ring slot   */
/* (first_slot + s) mod slots, evicting what that slot held; other slots are */
/* left as they are.                                                          */
/* Pinned by: a stream appended in several chunks leaves the ring equal to   */
/* one quantization of the whole stream, slab g in slot g mod slots, for the */
/* last `slots` slabs; untouched slots keep their contents.                  */
/* Returns 0, or -1 on bad arguments.                                         */
/* ------------------------------------------------------------------------- */
int orc_cache_append(const uint16_t* x, int64_t sB, int64_t sH, int64_t sL, int B, int H, int rows, int d,
                     int valid_len, int R, int8_t* cache_q, float* cache_scale, int slots, int first_slot) {
  if (rows % R || rows / R > slots || first_slot < 0 || first_slot >= slots) return -1;
  int nblk = rows / R;
  int8_t* q = (int8_t*)malloc((size_t)B * H * (rows > 0 ? rows : 1) * d);
  float* sc = (float*)malloc(sizeof(float) * (size_t)B * H * (nblk > 0 ? nblk : 1));
  orc_quantize(x, sB, sH, sL, B, H, rows, d, valid_len, R, q, sc);
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      int64_t bh = (int64_t)b * H + h;
      for (int s = 0; s < nblk; ++s) {
        int slot = (first_slot + s) % slots;
        memcpy(cache_q + (bh * slots + slot) * (int64_t)R * d, q + (bh * rows + (int64_t)s * R) * d,
               (size_t)R * d);
        cache_scale[bh * slots + slot] = sc[bh * nblk + s];
      }
    }
  free(q);
  free(sc);
  return 0;
}

/* ------------------------------------------------------------------------- */
/* Key layout.  Ref2VA VSA, two-stage attention patch: the geometry mapper    */
/* gives the text, reference-image and reference-audio tokens tiles of their */
/* own, which stay dense, and only the generated-video key tiles are pruned; */
/* Configure Sol Sparse Attention, "The inputs that matter": a long reference */
/* video may be sparsified while images and audio stay exact, and the auto   */
/* prefix policy follows the model's own layout.                             */
/* seg holds nseg (start, rows, routed) triplets in increasing start, each   */
/* start a multiple of the key block, so no key block spans two segments.   */
/* Key row u is valid when it lies in [start, start + rows) of a segment and */
/* below lkv_valid; the rest (a segment's padding up to the next start) is   */
/* excluded like the padding at the end.  Key block j is routed when the     */
/* segment holding its first row is.  Without segments (nseg = 0) the rows   */
/* below lkv_valid are valid and blocks at or after the protected prefix are */
/* routed.                                                                    */
/* ------------------------------------------------------------------------- */
typedef struct {
  const int32_t* seg;
  int nseg, lkv_valid, prefix, kblock;
} orc_layout;

/* Segment holding row u (the last with start <= u), or -1. */
static int orc_seg_of(const orc_layout* L, int u) {
  int s = -1;
  for (int x = 0; x < L->nseg; ++x)
    if (L->seg[3 * x] <= u) s = x;
  return s;
}

static int orc_key_valid(const orc_layout* L, int u) {
  if (u >= L->lkv_valid) return 0;
  if (L->nseg == 0) return 1;
  int s = orc_seg_of(L, u);
  return s >= 0 && u < L->seg[3 * s] + L->seg[3 * s + 1];
}

static int orc_block_routed(const orc_layout* L, int j) {
  if (L->nseg == 0) return j * L->kblock >= L->prefix;
  int s = orc_seg_of(L, j * L->kblock);
  return s >= 0 && L->seg[3 * s + 2] != 0;
}

/* ------------------------------------------------------------------------- */
/* Routing: block map, centroids, statistics.                                 */
/*                                                                            */
/* Sums (integer): Qsum_i = sum of INT8 Q codes over the valid rows of query */
/* block i; Ksum_j likewise over key block j; n_j = valid rows of key block. */
/*                                                                            */
/* Candidates of a query block: routed key blocks (see the key layout) with */
/* at least one valid row (Configure Sol Sparse Attention, "The inputs that */
/* matter"; Ref2VA VSA, two-stage attention patch: only video key tiles are */
/* pruned).  Other blocks with valid rows are always exact (the protected   */
/* prefix, dense segments); blocks without valid rows are dropped.          */
/*                                                                            */
/* Proxy: the dot product of the dequantized block means, q_mean . k_mean.   */
/* Dividing out the positive per-row factor a_i / n_i leaves                 */
/*   s_ij = (Qsum_i . Ksum_j) * b_j / n_j                                     */
/* which ranks and standardizes identically; the dot is an exact integer.    */
/* Rule (Configure Sol Sparse Attention, "How it works"): with mu and sigma  */
/* the mean and population standard deviation of s_ij over the candidates,   */
/* a candidate becomes a centroid when s_ij > mu + tau*sigma, else exact.    */
/* tau = +inf, sigma = 0 or no candidates: every candidate exact.            */
/* tie[i,j] = 1 when |s_ij - (mu + tau*sigma)| <= 1e-6 * sigma.              */
/*                                                                            */
/* Fixed-sparsity rule (rule = 1; Ref2VA VSA, two-stage attention patch:     */
/* top-k pruning of the video key tiles only, at a set sparsity such as      */
/* 0.75, with 0.50-0.70 suggested as a start): of the N candidates of a query */
/* block, floor(sparsity * N) are pruned (the product taken in float64) and  */
/* the other N - floor(sparsity * N) stay exact: those with the largest      */
/* s_ij, equal values ordered by lower key-block index first.  Pruned blocks */
/* become centroids when centroids are kept (G > 0) and are dropped when     */
/* G = 0.  Prefix blocks stay exact, empty blocks dropped; stats are NaN.    */
/*                                                                            */
/* Explicit maps (FlashVSR Sparge Attention, "How it works"): a map on       */
/* logical blocks of map_kblock keys; physical block j takes the state of    */
/* logical block j*kblock/map_kblock.  Values above 2 count as exact, and so */
/* does a centroid request when no centroids are kept (G = 0).  Prefix       */
/* blocks are exact and empty blocks dropped here too.                        */
/*                                                                            */
/* Centroids (Configure Sol Sparse Attention, "How it works": one 64-token   */
/* centroid, or two 32-token ones): for group g of block j (G groups of      */
/* kblock/G contiguous rows), n_jg valid rows, kbar = mean of the dequantized */
/* INT8 keys, vbar = mean of V, weight n_jg.  An empty group has weight 0.   */
/*                                                                            */
/* Pinned by: brute force on tiny inputs, closed-form outlier example,       */
/* tau = +/-inf cases, nesting in tau, scale invariance, 1x64 map == 2x32    */
/* map, LCSA block count; for the fixed-sparsity rule a hand-ordered        */
/* example, brute force, equal-score ordering, kept counts and nesting in    */
/* the sparsity.  The proxy itself: parity unpinned (the pages do not        */
/* define it).                                                                */
/* Returns 0, or -1 on bad arguments.                                         */
/* ------------------------------------------------------------------------- */
typedef struct {
  double s;
  int j;
} orc_scored;

/* Larger score first; equal scores by lower block index. */
static int orc_rank_cmp(const void* pa, const void* pb) {
  const orc_scored* a = (const orc_scored*)pa;
  const orc_scored* b = (const orc_scored*)pb;
  if (a->s > b->s) return -1;
  if (a->s < b->s) return 1;
  return (a->j > b->j) - (a->j < b->j);
}

int orc_route(const int8_t* q, const int8_t* k, const float* k_scale, int k_scale_rows,
              const uint16_t* v_bf16, const int8_t* v_i8, const float* v_scale, int v_scale_rows,
              const int32_t* v_block_src, int Lv, int B, int H, int Lq, int Lkv, int d, int lq_valid,
              int lkv_valid, int rule, double tau, double sparsity, int G, int prefix, int kblock,
              const int32_t* seg, int nseg,
              const uint8_t* explicit_map, int map_kblock, uint8_t* map, double* kbar,
              double* vbar, double* count, double* stats, uint8_t* tie) {
  int nQB = (Lq + QBLOCK - 1) / QBLOCK;
  int nKB = (Lkv + kblock - 1) / kblock;
  int nKS = (Lkv + k_scale_rows - 1) / k_scale_rows;
  int nMB = explicit_map ? (Lkv + map_kblock - 1) / map_kblock : 0;
  if (G < 0 || G > 2 || (G > 0 && kblock % G)) return -1;
  if (!explicit_map && k_scale_rows != kblock) return -1;
  if (!explicit_map && rule == 0 && (G == 0 || isnan(tau))) return -1;
  if (!explicit_map && rule == 1 && !(sparsity >= 0.0 && sparsity <= 1.0)) return -1;
  if (!explicit_map && rule != 0 && rule != 1) return -1;
  orc_vsrc vs = {v_bf16, v_i8, v_scale, v_scale_rows, v_block_src, Lv, H, d};
  orc_layout lay = {seg, nseg, lkv_valid, prefix, kblock};
  int ok = 0;
  for (int x = 0; x < nseg; ++x) {
    if (seg[3 * x] % kblock || seg[3 * x + 1] < 0) return -1;
    if (x > 0 && seg[3 * x] < seg[3 * (x - 1)] + seg[3 * (x - 1) + 1]) return -1;
  }
  if (nseg > 0 && prefix != 0) return -1;

#pragma omp parallel for collapse(2) schedule(dynamic)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h) {
      int64_t bh = (int64_t)b * H + h;
      const int8_t* qh = q + bh * Lq * d;
      const int8_t* kh = k + bh * Lkv * d;
      int64_t* Qs = (int64_t*)calloc((size_t)nQB * d, sizeof(int64_t));
      int64_t* Ks = (int64_t*)calloc((size_t)nKB * d, sizeof(int64_t));
      int* nk = (int*)calloc((size_t)nKB, sizeof(int));
      double* s = (double*)malloc(sizeof(double) * (size_t)nKB);
      orc_scored* ranked = (orc_scored*)malloc(sizeof(orc_scored) * (size_t)nKB);
      for (int i = 0; i < nQB; ++i)
        for (int t = i * QBLOCK; t < (i + 1) * QBLOCK && t < Lq && t < lq_valid; ++t)
          for (int c = 0; c < d; ++c) Qs[(int64_t)i * d + c] += qh[(int64_t)t * d + c];
      for (int j = 0; j < nKB; ++j)
        for (int u = j * kblock; u < (j + 1) * kblock && u < Lkv; ++u) {
          if (!orc_key_valid(&lay, u)) continue;
          nk[j] += 1;
          for (int c = 0; c < d; ++c) Ks[(int64_t)j * d + c] += kh[(int64_t)u * d + c];
        }

      /* Centroids per group. */
      if (G > 0) {
        int gr = kblock / G;
        for (int j = 0; j < nKB; ++j)
          for (int g = 0; g < G; ++g) {
            int64_t o = ((bh * nKB + j) * G + g);
            int n = 0;
            for (int c = 0; c < d; ++c) {
              kbar[o * d + c] = 0.0;
              vbar[o * d + c] = 0.0;
            }
            for (int u = j * kblock + g * gr; u < j * kblock + (g + 1) * gr && u < Lkv; ++u) {
              if (!orc_key_valid(&lay, u)) continue;
              ++n;
              double ks = (double)k_scale[bh * nKS + u / k_scale_rows];
              for (int c = 0; c < d; ++c) {
                kbar[o * d + c] += (double)kh[(int64_t)u * d + c] * ks;
                vbar[o * d + c] += v_at(&vs, b, h, u, c);
              }
            }
            for (int c = 0; c < d; ++c) {
              kbar[o * d + c] = n ? kbar[o * d + c] / n : 0.0;
              vbar[o * d + c] = n ? vbar[o * d + c] / n : 0.0;
            }
            count[o] = (double)n;
          }
      }

      for (int i = 0; i < nQB; ++i) {
        uint8_t* mrow = map + (bh * nQB + i) * nKB;
        uint8_t* trow = tie ? tie + (bh * nQB + i) * nKB : NULL;
        double mu = NAN, sigma = NAN;
        if (trow) memset(trow, 0, (size_t)nKB);
        if (explicit_map) {
          const uint8_t* erow = explicit_map + (bh * nQB + i) * nMB;
          for (int j = 0; j < nKB; ++j) {
            int st = erow[(int64_t)j * kblock / map_kblock];
            if (st > ORC_CENTROID || (st == ORC_CENTROID && G == 0)) st = ORC_EXACT;
            if (!orc_block_routed(&lay, j)) st = ORC_EXACT;
            if (nk[j] == 0) st = ORC_DROP;
            mrow[j] = (uint8_t)st;
          }
        } else {
          int N = 0;
          for (int j = 0; j < nKB; ++j) {
            int cand = nk[j] > 0 && orc_block_routed(&lay, j);
            if (!cand) {
              mrow[j] = nk[j] > 0 ? ORC_EXACT : ORC_DROP;
              continue;
            }
            int64_t D = 0;
            for (int c = 0; c < d; ++c) D += Qs[(int64_t)i * d + c] * Ks[(int64_t)j * d + c];
            s[j] = (double)D * (double)k_scale[bh * nKS + j] / (double)nk[j];
            ++N;
          }
          if (rule == 1) {
            /* fixed sparsity: keep the N - floor(sparsity * N) best-scored */
            int n = 0;
            for (int j = 0; j < nKB; ++j)
              if (nk[j] > 0 && orc_block_routed(&lay, j)) {
                ranked[n].s = s[j];
                ranked[n].j = j;
                ++n;
              }
            qsort(ranked, (size_t)n, sizeof(orc_scored), orc_rank_cmp);
            int keep = N - (int)floor(sparsity * (double)N);
            for (int r = 0; r < n; ++r) mrow[ranked[r].j] = r < keep ? ORC_EXACT : (G > 0 ? ORC_CENTROID : ORC_DROP);
            if (stats) {
              stats[(bh * nQB + i) * 2] = NAN;
              stats[(bh * nQB + i) * 2 + 1] = NAN;
            }
            continue;
          }
          if (N > 0) {
            double sum = 0.0;
            for (int j = 0; j < nKB; ++j)
              if (nk[j] > 0 && orc_block_routed(&lay, j)) sum += s[j];
            mu = sum / N;
            double ss = 0.0;
            for (int j = 0; j < nKB; ++j)
              if (nk[j] > 0 && orc_block_routed(&lay, j)) ss += (s[j] - mu) * (s[j] - mu);
            sigma = sqrt(ss / N);
          }
          int keep_all = N == 0 || (isinf(tau) && tau > 0) || sigma == 0.0;
          double thr = keep_all ? INFINITY : mu + tau * sigma;
          for (int j = 0; j < nKB; ++j) {
            if (!(nk[j] > 0 && orc_block_routed(&lay, j))) continue;
            mrow[j] = (!keep_all && s[j] > thr) ? ORC_CENTROID : ORC_EXACT;
            if (trow && !keep_all && isfinite(thr) && fabs(s[j] - thr) <= 1e-6 * sigma) trow[j] = 1;
          }
        }
        if (stats) {
          stats[(bh * nQB + i) * 2] = mu;
          stats[(bh * nQB + i) * 2 + 1] = sigma;
        }
      }
      free(Qs);
      free(Ks);
      free(nk);
      free(s);
      free(ranked);
    }
  return ok;
}

/* ------------------------------------------------------------------------- */
/* Forward pass over one set of query blocks.                                 */
/* Configure Sol Sparse Attention, "How it works": exact blocks use the INT8 */
/* Q/K (integer dot times both scales); skipped blocks add their centroids   */
/* to the same softmax (Configure H3 Static Virtual KV, mode list: "residual"*/
/* puts the centroids into the same online softmax as the exact blocks).     */
/* For a valid query row t of block i (scale a_i):                           */
/*   x_tu = sm * a_i * b(u) * (q_t . k_u)        for valid keys u of EXACT blocks */
/*   c_tg = sm * a_i * (q_t . kbar_g)            for centroid groups with n_g > 0  */
/*   o_t  = (sum_u e^x v_u + sum_g n_g e^c vbar_g) / (sum_u e^x + sum_g n_g e^c)    */
/*   lse_t = log of that denominator (with the max subtracted and added back) */
/* Rows with nothing to attend, and rows past lq_valid, give 0 and -inf.     */
/* sel lists query blocks as (b*H + h)*nQB + i; out is [nsel][128][d],       */
/* lse [nsel][128].                                                           */
/* Floating QK path (q_bf16, k_bf16 given; Configure Sol Sparse Attention,  */
/* "How it works": with a floating dense backend the exact blocks run in    */
/* floating point instead of W8A8): x_tu = sm * (q_t . k_u) and              */
/* c_tg = sm * (q_t . kbar_g) on the bf16 values; the block map and the     */
/* centroids are the same (routed on the INT8 codes).                        */
/* Pinned by: all-exact map == textbook softmax attention (library SDPA in   */
/* float64), LCSA map == masked dense attention, single-block centroid       */
/* closed forms, identical-key blocks (centroid == exact, count weighting);  */
/* the floating path: all-exact == SDPA on the bf16 inputs, a single        */
/* centroid block gives vbar, and a mix of exact keys and 2x32 centroid      */
/* columns equals a softmax over explicitly listed columns (bf16 query      */
/* against kbar, 1/sqrt(d), ln(count) bias).                                  */
/* ------------------------------------------------------------------------- */
void orc_forward(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale,
                 int k_scale_rows, const uint16_t* v_bf16, const int8_t* v_i8, const float* v_scale,
                 int v_scale_rows, const int32_t* v_block_src, int Lv, int B, int H, int Lq, int Lkv,
                 int d, int lq_valid, int lkv_valid, int kblock, const int32_t* seg, int nseg, int G,
                 const uint8_t* map,
                 const double* kbar, const double* vbar, const double* count, double sm_scale,
                 const int64_t* sel, int nsel, double* out, double* lse, const uint16_t* q_bf16,
                 const uint16_t* k_bf16) {
  int nQB = (Lq + QBLOCK - 1) / QBLOCK;
  int nKB = (Lkv + kblock - 1) / kblock;
  int nKS = (Lkv + k_scale_rows - 1) / k_scale_rows;
  int maxcols = Lkv + nKB * (G > 0 ? G : 0);
  orc_vsrc vs = {v_bf16, v_i8, v_scale, v_scale_rows, v_block_src, Lv, H, d};
  orc_layout lay = {seg, nseg, lkv_valid, 0, kblock};
  (void)B;

#pragma omp parallel
  {
    double* x = (double*)malloc(sizeof(double) * (size_t)(maxcols > 0 ? maxcols : 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(maxcols > 0 ? maxcols : 1));
    int* col = (int*)malloc(sizeof(int) * (size_t)(maxcols > 0 ? maxcols : 1)); /* key row, or -1-centroid index */
    double* acc = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic)
    for (int e = 0; e < nsel; ++e) {
      int64_t id = sel[e];
      int i = (int)(id % nQB);
      int64_t bh = id / nQB;
      int b = (int)(bh / H), h = (int)(bh % H);
      const uint8_t* mrow = map + (bh * nQB + i) * nKB;
      double a = (double)q_scale[bh * nQB + i];
      for (int r = 0; r < QBLOCK; ++r) {
        int t = i * QBLOCK + r;
        double* o = out + ((int64_t)e * QBLOCK + r) * d;
        for (int c = 0; c < d; ++c) o[c] = 0.0;
        lse[(int64_t)e * QBLOCK + r] = -INFINITY;
        if (t >= Lq || t >= lq_valid) continue;
        const int8_t* qt = q + (bh * Lq + t) * d;
        const uint16_t* qf = q_bf16 ? q_bf16 + (bh * Lq + t) * d : NULL;
        int n = 0;
        for (int j = 0; j < nKB; ++j) {
          if (mrow[j] == ORC_EXACT) {
            for (int u = j * kblock; u < (j + 1) * kblock && u < Lkv; ++u) {
              if (!orc_key_valid(&lay, u)) continue;
              if (qf) {
                const uint16_t* kf = k_bf16 + (bh * Lkv + u) * d;
                double dotf = 0.0;
                for (int c = 0; c < d; ++c) dotf += (double)bf16_to_f32(qf[c]) * (double)bf16_to_f32(kf[c]);
                x[n] = sm_scale * dotf;
                w[n] = 1.0;
                col[n] = u;
                ++n;
                continue;
              }
              const int8_t* ku = k + (bh * Lkv + u) * d;
              int64_t dot = 0;
              for (int c = 0; c < d; ++c) dot += (int64_t)qt[c] * ku[c];
              x[n] = sm_scale * a * (double)k_scale[bh * nKS + u / k_scale_rows] * (double)dot;
              w[n] = 1.0;
              col[n] = u;
              ++n;
            }
          } else if (mrow[j] == ORC_CENTROID && G > 0) {
            for (int g = 0; g < G; ++g) {
              int64_t ci = (bh * nKB + j) * G + g;
              if (count[ci] <= 0.0) continue;
              double dot = 0.0;
              if (qf) {
                for (int c = 0; c < d; ++c) dot += (double)bf16_to_f32(qf[c]) * kbar[ci * d + c];
              } else {
                for (int c = 0; c < d; ++c) dot += a * (double)qt[c] * kbar[ci * d + c];
              }
              x[n] = sm_scale * dot;
              w[n] = count[ci];
              col[n] = (int)(-1 - ci);
              ++n;
            }
          }
        }
        if (n == 0) continue;
        double m = -INFINITY;
        for (int u = 0; u < n; ++u)
          if (x[u] > m) m = x[u];
        double l = 0.0;
        for (int c = 0; c < d; ++c) acc[c] = 0.0;
        for (int u = 0; u < n; ++u) {
          double p = w[u] * exp(x[u] - m);
          l += p;
          if (col[u] >= 0) {
            for (int c = 0; c < d; ++c) acc[c] += p * v_at(&vs, b, h, col[u], c);
          } else {
            int64_t ci = -1 - (int64_t)col[u];
            for (int c = 0; c < d; ++c) acc[c] += p * vbar[ci * d + c];
          }
        }
        for (int c = 0; c < d; ++c) o[c] = acc[c] / l;
        lse[(int64_t)e * QBLOCK + r] = m + log(l);
      }
    }
    free(x);
    free(w);
    free(col);
    free(acc);
  }
}

/* ------------------------------------------------------------------------- */
/* Virtual KV, conservative materialization (Configure H3 Static Virtual KV, */
/* mode list: "conservative" builds the exact seven-slice K context).        */
/* Logical slice l, row r reads physical slice src[l], row r, and rotates    */
/* channel pairs (off + 2p, off + 2p + 1), p < d_rot/2, by slice l's phase:  */
/*   y0 = fma(x0, cos, -(x1 * sin)),  y1 = fma(x0, sin, x1 * cos)            */
/* in float32, then rounds to bf16 (the model's K dtype).  Other channels    */
/* are copied.                                                                */
/* Pinned by: zero phase == plain copy, quarter-turn phase == exact pair     */
/* swap with negation, norm preservation to rounding.                         */
/* ------------------------------------------------------------------------- */
void orc_materialize_virtual_k(const uint16_t* k_phys, int B, int H, int S, int n_phys, int d,
                               const int32_t* src, int n_logical, const float* cosv,
                               const float* sinv, int rot_offset, int d_rot, uint16_t* k_log) {
  int Lp = S * n_phys, Ll = S * n_logical, np2 = d_rot / 2;
#pragma omp parallel for collapse(2) schedule(static)
  for (int b = 0; b < B; ++b)
    for (int h = 0; h < H; ++h)
      for (int l = 0; l < n_logical; ++l)
        for (int r = 0; r < S; ++r) {
          const uint16_t* xr = k_phys + (((int64_t)b * H + h) * Lp + (int64_t)src[l] * S + r) * d;
          uint16_t* yr = k_log + (((int64_t)b * H + h) * Ll + (int64_t)l * S + r) * d;
          for (int c = 0; c < d; ++c) yr[c] = xr[c];
          for (int p = 0; p < np2; ++p) {
            int c0 = rot_offset + 2 * p;
            float x0 = bf16_to_f32(xr[c0]), x1 = bf16_to_f32(xr[c0 + 1]);
            float cs = cosv[l * np2 + p], sn = sinv[l * np2 + p];
            float t1 = x1 * sn, t2 = x1 * cs;
            float y0 = fmaf(x0, cs, -t1);
            float y1 = fmaf(x0, sn, t2);
            yr[c0] = f32_to_bf16_rne(y0);
            yr[c0 + 1] = f32_to_bf16_rne(y1);
          }
        }
}

/* Virtual KV, "fast" mode (Configure H3 Static Virtual KV, mode list): the    */
/* same logical keys, produced only as INT8 containers with one scale per R    */
/* logical rows, plus the V block source table: logical 64-row block j reads  */
/* physical V block src[j / (S/64)] * (S/64) + j % (S/64).  Defined as the     */
/* conservative materialization followed by the quantizer, which is exactly    */
/* the pages' claim that nothing is approximated.                              */
void orc_gather_virtual_kv(const uint16_t* k_phys, int B, int H, int S, int n_phys, int d,
                           const int32_t* src, int n_logical, const float* cosv, const float* sinv,
                           int rot_offset, int d_rot, int R, int8_t* k_q, float* k_scale,
                           int32_t* v_block_src) {
  int64_t Ll = (int64_t)S * n_logical;
  uint16_t* tmp = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)B * H * Ll * d);
  orc_materialize_virtual_k(k_phys, B, H, S, n_phys, d, src, n_logical, cosv, sinv, rot_offset,
                            d_rot, tmp);
  orc_quantize(tmp, (int64_t)H * Ll * d, Ll * d, d, B, H, (int)Ll, d, (int)Ll, R, k_q, k_scale);
  free(tmp);
  int bps = S / 64;
  for (int j = 0; j < n_logical * bps; ++j) v_block_src[j] = src[j / bps] * bps + j % bps;
}

int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
