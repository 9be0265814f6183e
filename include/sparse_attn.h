/*
 * sparse_attn.h — C ABI of the MI355X (gfx950) block-sparse INT8 video attention
 * library (libsparse_attn.so).
 *
 * The method (Configure Sol Sparse Attention, "How it works"): Q and K are
 * quantized to INT8 per block; within each 128-token query block every 64-token
 * key/value block is rated by an inexpensive proxy on those INT8 tensors; a block whose
 * score exceeds mean + routing_threshold * std over the query block's candidates
 * is skipped, standing in as a single 64-token centroid (1x64) or two 32-token
 * centroids (2x32) that still enter the online softmax; the other blocks are
 * computed exactly (INT8 QK^T, fp32 online softmax, bf16 PV).  A leading prefix
 * of conditioning tokens can be exempted (Configure Sol Sparse Attention, "The
 * inputs that matter"; Ref2VA VSA, two-stage attention patch section).  An
 * explicit block map — e.g. FlashVSR's local-causal LCSA mask on logical
 * 128x128 blocks (FlashVSR Sparge Attention, opening section and "How it
 * works") — can replace the routing rule.  Virtual K/V contexts are gathered
 * from physical slices (Configure H3 Static Virtual KV, mode list).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Device pointers unless a name ends in _host.  The caller allocates and owns
 *    every buffer; the library allocates no device memory and keeps no state
 *    beyond a per-device architecture check and the thread-local error text
 *    (sparse_attn_route_noalloc aside: its workspace is a static array of the
 *    library's device code).
 *  - Work is queued on `stream` (a hipStream_t passed as void*; NULL = the
 *    default stream) and never synchronizes the host.  Arguments are validated
 *    before anything is queued: a non-zero status means nothing was launched.
 *  - On failure a status below is returned and sa_last_error() describes it.
 *    No exception, abort or exit crosses this boundary.
 *  - Tensors named [B,H,L,d] are dense with d contiguous, unless strides are
 *    passed.  bf16 is IEEE bfloat16 as uint16 bits.  INT8 and bf16 tensors
 *    must be 16-byte aligned.
 *  - Query blocks are 128 rows.  Lq must be a multiple of 128 and Lkv a
 *    multiple of 128; the ragged end of a sequence is expressed with
 *    lq_valid / lkv_valid (rows at or past them are padding: excluded from
 *    scales, sums, centroids and softmax; padded output rows are written as 0
 *    with lse = -inf).
 *  - A segmented key layout (sa_segment) also pads each segment to a key-block
 *    boundary.  Route and forward exclude those rows from counts, centroids and
 *    the softmax; quantize_qk_int8 does not know the layout, so padding rows
 *    should hold zeros (they then code to 0 and leave a block's scale as it
 *    would be without them).  Query rows inside the layout's padding are
 *    computed like any other row below lq_valid.
 *  - Only gfx950 devices are accepted; others give SA_E_UNSUPPORTED.
 *  - The forward passes address one head's K and V with 32-bit offsets: each
 *    must be below 4 GiB (SA_E_SHAPE otherwise).
 */
#ifndef SPARSE_ATTN_H
#define SPARSE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SA_ABI_VERSION 7

enum sa_status {
  SA_OK = 0,
  SA_E_NULL = 1,        /* a required pointer is NULL */
  SA_E_SHAPE = 2,       /* a size is out of range or inconsistent */
  SA_E_ALIGN = 3,       /* a pointer or stride breaks the 16-byte rule */
  SA_E_VALUE = 4,       /* a scalar parameter is invalid (NaN threshold, bad enum) */
  SA_E_UNSUPPORTED = 5, /* the current device is not gfx950 */
  SA_E_DEVICE = 6,      /* no usable HIP device */
  SA_E_LAUNCH = 7,      /* a kernel launch failed */
  SA_E_WORKSPACE = 8    /* workspace missing or too small */
};

/* Block-map states (one uint8 per (query block, key block)). */
enum sa_block_state { SA_DROP = 0, SA_EXACT = 1, SA_CENTROID = 2 };

/* Routing rules used when no explicit map is given. */
enum sa_route_rule {
  SA_RULE_THRESHOLD = 0, /* Sol: centroid iff proxy > mean + threshold * std */
  SA_RULE_TOPK = 1       /* fixed sparsity: keep the best-scored candidates */
};

/* Element types for V and the attention output. */
enum sa_dtype { SA_BF16 = 0, SA_INT8 = 1, SA_F32 = 2 };

typedef struct sa_dims {
  int32_t B, H;                /* batch, heads (>= 1) */
  int32_t Lq, Lkv;             /* allocated query rows, logical key rows (multiples of 128) */
  int32_t d;                   /* head dimension: 64 or 128 */
  int32_t lq_valid, lkv_valid; /* 0 <= valid <= allocated */
  int32_t Lv;                  /* physical rows of V: == Lkv, or the physical length when
                                  v_block_src remaps 64-row V blocks (virtual KV) */
} sa_dims;

/* One segment of the key sequence (Ref2VA VSA, two-stage attention patch:
 * text, reference-image and reference-audio tokens get key tiles of their own
 * that stay dense, and only generated-video key tiles are pruned; Configure
 * Sol Sparse Attention, "The inputs that matter": a reference video may be
 * routed as well, and the auto prefix policy follows the model's layout). */
typedef struct sa_segment {
  int32_t start;               /* first key row: a multiple of kblock, so that no key
                                  block spans two segments */
  int32_t rows;                /* valid rows (>= 0); rows from start + rows up to the
                                  next segment's start are padding */
  int32_t routed;              /* nonzero: its key blocks are routing candidates;
                                  zero: dense (always SA_EXACT) */
} sa_segment;

#define SA_MAX_SEGMENTS 16

typedef struct sa_route_params {
  float threshold;             /* routing_threshold tau (Sol rule); +inf keeps every block
                                  exact, -inf makes every candidate a centroid; NaN is
                                  rejected when the Sol rule is used */
  int32_t centroids_per_block; /* G: 1 (1x64), 2 (2x32); 0 only with an explicit map and
                                  means "no centroids" */
  int32_t prefix_tokens;       /* multiple of kblock; key blocks inside it are always exact
                                  and are not routing candidates */
  int32_t kblock;              /* key block rows: 64 or 128 */
  int32_t k_scale_rows;        /* rows per K scale: 64 or 128 (== kblock for the Sol rule) */
  int32_t v_scale_rows;        /* rows per V scale when V is INT8: 64 or 128 */
  int32_t map_kblock;          /* key rows per entry of an explicit map: a multiple of kblock */
  int32_t rule;                /* SA_RULE_THRESHOLD or SA_RULE_TOPK (ignored with an explicit map) */
  float sparsity;              /* SA_RULE_TOPK: fraction of the candidates pruned per query
                                  block, in [0, 1]; NaN or outside is rejected */
  int32_t n_segments;          /* 0: the key layout is the prefix (dense) then routed rows
                                  up to lkv_valid; 1..SA_MAX_SEGMENTS: segments_host
                                  describes it (prefix_tokens must then be 0) */
  const sa_segment* segments_host; /* host array of n_segments, in increasing start,
                                  non-overlapping, start + rows <= lkv_valid; read during
                                  the call only */
} sa_route_params;

/* ABI version of this build (SA_ABI_VERSION).  A caller compiled against another
 * version must not call anything else (FlashVSR Kitchen Sparse Attention, "When
 * it bites": the loader checks the ABI version and fails fast). */
int32_t sa_abi_version(void);

/* Text of the last error on the calling thread; valid until the next call on
 * this thread.  Never NULL. */
const char* sa_last_error(void);

/* SA_OK when `device` is a gfx950 GPU, SA_E_UNSUPPORTED for another GPU,
 * SA_E_DEVICE when it does not exist (FlashVSR Kitchen Sparse Attention, "When
 * it bites": unsupported runtimes are rejected outright rather than run). */
int32_t sa_device_check(int32_t device);

/* Per-block symmetric INT8 quantization (Configure Sol Sparse Attention, "How it
 * works": Q and K are prequantized to INT8 and the same codes serve routing and
 * the exact path; FlashVSR Kitchen Sparse Attention, opening section: an INT8
 * K/V cache in 128-row slabs).
 *   x_bf16   bf16, element (b,h,l,c) at x_bf16 + b*sB + h*sH + l*sL + c
 *            (strides in elements, multiples of 8; channel stride 1)
 *   L        rows (multiple of rows_per_block), d in {64,128}
 *   valid_len rows at or past it are padding (code 0, not in amax)
 *   rows_per_block 64 or 128
 *   x_q      out int8 [B,H,L,d] dense
 *   scale    out fp32 [B,H,L/rows_per_block]: amax/127 of the block (0 if all
 *            zero); code = clamp(round-half-even(x * (127/amax)), -127, 127)
 *   col_sums optional out int16 [B,H,L/sum_rows,d] (NULL: not written): the
 *            column sums of the written codes over each chunk of sum_rows
 *            rows (32, or rows_per_block; ignored when col_sums is NULL).
 *            Handed to sparse_attn_route as q_sums (Q, sum_rows 128) and k_sums
 *            (K, sum_rows 32) they spare the route a second read of the codes.
 * Bit-exact with a plain IEEE float32 evaluation of that rule. */
int32_t quantize_qk_int8(const void* x_bf16, int64_t sB, int64_t sH, int64_t sL, int32_t B,
                         int32_t H, int32_t L, int32_t d, int32_t valid_len,
                         int32_t rows_per_block, int8_t* x_q, float* scale, int16_t* col_sums,
                         int32_t sum_rows, void* stream);

/* Streaming INT8 K/V cache append (FlashVSR Kitchen Sparse Attention, opening
 * section: in streaming use each block holds the recent K/V history as INT8,
 * bounded, in 128-row slabs).  The cache of one tensor (K
 * or V) is a ring of `slots` slabs of rows_per_slab rows per (b, h).  The new
 * chunk is quantized per slab exactly as quantize_qk_int8 quantizes blocks, and
 * slab s of it replaces ring slot (first_slot + s) mod slots, evicting the slab
 * there; other slots are not touched.  The caller tracks which slot holds which
 * slab: route and forward see the ring in slot order, so maps and segments
 * passed with it refer to slot order (attention is order-free over keys).
 *   x_bf16       bf16 chunk, element (b,h,l,c) at x_bf16 + b*sB + h*sH + l*sL + c
 *                (strides in elements, multiples of 8; channel stride 1)
 *   rows         chunk rows, a multiple of rows_per_slab, rows/rows_per_slab <= slots
 *   valid_len    rows at or past it are padding (code 0, not in amax)
 *   rows_per_slab 64 or 128
 *   cache_q      int8 [B,H,slots*rows_per_slab,d]; cache_scale fp32 [B,H,slots]
 *   first_slot   in [0, slots)
 * Bit-exact with quantizing the chunk and copying its slabs into the ring. */
int32_t kv_cache_append_int8(const void* x_bf16, int64_t sB, int64_t sH, int64_t sL, int32_t B, int32_t H,
                             int32_t rows, int32_t d, int32_t valid_len, int32_t rows_per_slab, int8_t* cache_q,
                             float* cache_scale, int32_t slots, int32_t first_slot, void* stream);

/* Bytes of device workspace sparse_attn_route needs for these arguments (0 when
 * an explicit map is given).  Returns 0 and sets the error text on bad input. */
size_t sparse_attn_route_workspace_size(const sa_dims* dims, const sa_route_params* p,
                                        int32_t has_explicit_map);

/* Routing pass: block map plus centroids (Configure Sol Sparse Attention, "How
 * it works"; FlashVSR Sparge Attention, "How it works" for explicit maps on
 * logical blocks converted to the physical key-block size).
 *   q         int8 [B,H,Lq,d] (quantized with 128-row blocks)
 *   k         int8 [B,H,Lkv,d], k_scale fp32 [B,H,Lkv/k_scale_rows]
 *   q_sums, k_sums  optional int16 [B,H,Lq/128,d] and [B,H,Lkv/32,d]: the
 *             col_sums quantize_qk_int8 wrote with q (sum_rows 128) and k
 *             (sum_rows 32).  When given, the
 *             block sums come from them and q (resp. k) is not read and may be
 *             NULL.  They count every row of a chunk, which equals the sum over
 *             the valid rows because padding rows are coded 0 (past the valid
 *             length always; inside a segmented layout when they hold zeros, as
 *             required above).
 *   v         [B,H,Lv,d] bf16 (v_dtype SA_BF16) or int8 (SA_INT8, with v_scale
 *             fp32 [B,H,Lv/v_scale_rows]); logical key row r reads V row
 *             v_block_src[r/64]*64 + r%64 when v_block_src (int32 [Lkv/64]) is
 *             given, else row r.  Table entries outside [0, Lv/64) are clamped.
 *   explicit_map NULL: Sol rule.  Else uint8 [B,H,Lq/128,Lkv/map_kblock]; values
 *             above 2, and centroid entries when G = 0, are taken as SA_EXACT.
 *   block_map out uint8 [B,H,Lq/128,Lkv/kblock]:
 *             Candidates are routed key blocks with a valid row: at or after
 *             the prefix, or in a routed segment; proxy s_ij = (sum of INT8 Q codes of query block i) .
 *             (sum of INT8 K codes of key block j) * b_j / n_j (n_j valid rows,
 *             b_j the block's K scale) — the dot of the dequantized block means
 *             up to a positive per-query-block factor, exact in float64.
 *             SA_RULE_THRESHOLD: mu, sigma = mean and population std of s_ij
 *             over the candidates (float64); SA_CENTROID iff
 *             s_ij > mu + threshold*sigma, else SA_EXACT (all SA_EXACT if there
 *             are no candidates or sigma = 0).
 *             SA_RULE_TOPK (Ref2VA VSA, two-stage attention patch: top-k
 *             pruning of the video key tiles at a set sparsity): with N
 *             candidates, the N - floor(sparsity * N) of largest s_ij (the
 *             product in float64; equal s_ij ordered by lower block index) are
 *             SA_EXACT, the others SA_CENTROID when G > 0 and SA_DROP when G = 0.
 *             Prefix blocks and blocks of dense segments SA_EXACT; key blocks
 *             without valid rows SA_DROP (also for maps).
 *   k_centroid, v_centroid out fp32 [B,H,Lkv/kblock,G,d]; count out fp32
 *             [B,H,Lkv/kblock,G]: group g covers rows [g*kblock/G,(g+1)*kblock/G)
 *             of the block; kbar = mean of the dequantized INT8 keys, vbar =
 *             mean of V, count = valid rows (0 for an empty group).  Written for
 *             every block when G > 0; may be NULL when G = 0.
 *   row_stats optional out float64 [B,H,Lq/128,2] = (mu, sigma); NaN for maps
 *             and for SA_RULE_TOPK.
 *   workspace device memory of sparse_attn_route_workspace_size() bytes.
 * Threshold decisions are bit-exact with a float64 evaluation except where s_ij
 * lies within 1e-6*sigma of the threshold (summation order of mu, sigma);
 * SA_RULE_TOPK decisions are bit-exact. */
int32_t sparse_attn_route(const int8_t* q, const int8_t* k, const float* k_scale, const void* v,
                          int32_t v_dtype, const float* v_scale, const int32_t* v_block_src,
                          const int16_t* q_sums, const int16_t* k_sums,
                          const sa_dims* dims, const sa_route_params* p,
                          const uint8_t* explicit_map, uint8_t* block_map, float* k_centroid,
                          float* v_centroid, float* count, double* row_stats, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Bytes of library-owned route workspace per device (sparse_attn_route_noalloc). */
#define SA_ROUTE_SCRATCH_BYTES (16u << 20)

/* sparse_attn_route for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, results and errors as sparse_attn_route, without the
 * workspace: the block sums live in a library-owned device array of
 * SA_ROUTE_SCRATCH_BYTES (16 MiB), one per device, allocated with the library's
 * device code when a device first uses it and held until the process ends.
 * Calls whose sparse_attn_route_workspace_size() exceeds it (more than 85
 * heads of L = 32768, d = 128, kblock = 64) fail with SA_E_WORKSPACE before anything is
 * queued.  Nothing is allocated, freed or cleared by the call.  Every call on
 * one device shares that array: calls that can overlap in time on one device
 * (other streams, other host threads) race, and the caller must order them.
 * The array keeps the last call's contents, which no later call reads. */
int32_t sparse_attn_route_noalloc(const int8_t* q, const int8_t* k, const float* k_scale, const void* v,
                                  int32_t v_dtype, const float* v_scale, const int32_t* v_block_src,
                                  const int16_t* q_sums, const int16_t* k_sums,
                                  const sa_dims* dims, const sa_route_params* p,
                                  const uint8_t* explicit_map, uint8_t* block_map, float* k_centroid,
                                  float* v_centroid, float* count, double* row_stats, void* stream);

/* Forward pass over one block map (Configure Sol Sparse Attention, "How it
 * works"; Configure H3 Static Virtual KV, mode list, "residual": centroids share
 * the online softmax with the exact blocks).  For valid query row t of block i
 * (scale a_i = q_scale[b,h,i]):
 *   exact keys u (valid rows of SA_EXACT blocks):
 *       logit = sm_scale * a_i * b(u) * (q_t . k_u)   (INT8 dot, exact in int32)
 *   centroid groups g (count n_g > 0) of SA_CENTROID blocks:
 *       logit = sm_scale * a_i * (q_t . kbar_g) + ln(n_g), value vbar_g
 *   out_t = softmax-weighted sum of the values; lse_t = ln(sum of exp(logit)).
 * Softmax in fp32 (online, base 2), P rounded to bf16 for the PV product (bf16
 * MFMA with fp32 accumulation); kbar/vbar enter as bf16 hi+lo pairs.
 *   q, q_scale  int8 [B,H,Lq,d], fp32 [B,H,Lq/128]
 *   k, k_scale, v, v_dtype, v_scale, v_block_src: as for sparse_attn_route
 *   p           kblock, k_scale_rows, v_scale_rows, centroids_per_block and the
 *               key layout (segments, lkv_valid) are used; the routing fields
 *               are ignored
 *   block_map   uint8 [B,H,Lq/128,Lkv/kblock] (values > 2 are taken as SA_DROP)
 *   k_centroid, v_centroid, count: route outputs (may be NULL when G = 0)
 *   out         [B,H,Lq,d] fp32 (SA_F32) or bf16 (SA_BF16)
 *   lse         optional fp32 [B,H,Lq] (natural log)
 * Rows with nothing to attend and padded rows get 0 and lse = -inf. */
int32_t sparse_attn_fwd(const int8_t* q, const float* q_scale, const int8_t* k,
                        const float* k_scale, const void* v, int32_t v_dtype, const float* v_scale,
                        const int32_t* v_block_src, const sa_dims* dims, const sa_route_params* p,
                        const uint8_t* block_map, const float* k_centroid, const float* v_centroid,
                        const float* count, float sm_scale, void* out, int32_t out_dtype, float* lse,
                        void* stream);

/* Forward pass with a floating QK^T (Configure Sol Sparse Attention, "How it
 * works": with a floating dense backend the kept blocks are computed in
 * floating point rather than on the W8A8 path; the block map and centroids
 * are the same, routed on the INT8 codes).  As sparse_attn_fwd, except:
 *   exact keys u:       logit = sm_scale * (q_t . k_u)       on the bf16 values
 *   centroid groups g:  logit = sm_scale * (q_t . kbar_g) + ln(n_g)
 * with q_t the bf16 query (fp32 accumulation of bf16 products).
 *   q_bf16  bf16 [B,H,Lq,d], k_bf16 bf16 [B,H,Lkv,d], v_bf16 bf16 [B,H,Lv,d],
 *           dense; v_block_src as for sparse_attn_fwd
 *   p       kblock, centroids_per_block and the key layout are used
 *   block_map, k_centroid, v_centroid, count, sm_scale, out, out_dtype, lse:
 *           as for sparse_attn_fwd */
int32_t sparse_attn_fwd_float(const void* q_bf16, const void* k_bf16, const void* v_bf16,
                              const int32_t* v_block_src, const sa_dims* dims, const sa_route_params* p,
                              const uint8_t* block_map, const float* k_centroid, const float* v_centroid,
                              const float* count, float sm_scale, void* out, int32_t out_dtype, float* lse,
                              void* stream);

/* Virtual-KV gather, "fast" mode (Configure H3 Static Virtual KV, mode list):
 * logical slice l (of n_logical, at most 16) re-reads physical slice
 * src_map_host[l] (of n_phys), rotates channel pairs (rot_offset + 2p,
 * rot_offset + 2p + 1), p < d_rot/2, by slice l's phase
 *     y0 = fma(x0, cos, -(x1*sin)),  y1 = fma(x0, sin, x1*cos)   (fp32)
 * rounds to bf16 and quantizes per k_rows_per_block logical rows as
 * quantize_qk_int8 does.  Only the INT8 keys are materialized; V is not
 * copied, the returned table maps logical 64-row blocks to physical ones.
 *   k_phys_bf16   bf16 [B,H,n_phys*rows_per_slice,d] dense
 *   rows_per_slice multiple of k_rows_per_block and of 64
 *   src_map_host  host int32 [n_logical], values in [0, n_phys)
 *   rope_cos/sin  fp32 [n_logical, d_rot/2] (device)
 *   rot_offset, d_rot even, rot_offset + d_rot <= d
 *   k_logical     out int8 [B,H,n_logical*rows_per_slice,d]
 *   k_scale       out fp32 [B,H,n_logical*rows_per_slice/k_rows_per_block]
 *   v_block_src   out int32 [n_logical*rows_per_slice/64]:
 *                 src_map[j/(S/64)]*(S/64) + j%(S/64)
 * Bit-exact with materializing the seven-slice bf16 keys ("conservative")
 * and quantizing them. */
int32_t gather_virtual_kv(const void* k_phys_bf16, int32_t B, int32_t H, int32_t rows_per_slice,
                          int32_t n_phys, int32_t d, const int32_t* src_map_host,
                          int32_t n_logical, const float* rope_cos, const float* rope_sin,
                          int32_t rot_offset, int32_t d_rot, int32_t k_rows_per_block,
                          int8_t* k_logical, float* k_scale, int32_t* v_block_src, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPARSE_ATTN_H */
