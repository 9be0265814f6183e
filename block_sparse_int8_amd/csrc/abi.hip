// C ABI of libsparse_attn: argument validation, device check, dispatch.
//
// Every entry point validates all of its arguments before queueing anything,
// returns a status code, and records a message in a thread-local buffer
// (FlashVSR Kitchen Sparse Attention, "When it bites": fail at once with a
// clear message; unsupported runtimes are rejected outright).
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/sparse_attn.h"
#include "sa_launch.h"

namespace {

thread_local char g_err[512] = "";

int32_t fail(int32_t code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

int32_t ok() {
  g_err[0] = '\0';
  return SA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Per-device result of the architecture check: 0 unknown, 1 gfx950, 2 other.
constexpr int kMaxDev = 64;
int g_arch[kMaxDev] = {0};
std::mutex g_arch_mu;

int32_t check_device(int dev) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return fail(SA_E_DEVICE, "no HIP device is visible");
  }
  if (dev < 0 || dev >= count || dev >= kMaxDev) return fail(SA_E_DEVICE, "device %d does not exist (%d visible)", dev, count);
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_arch[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return fail(SA_E_DEVICE, "hipGetDeviceProperties failed for device %d", dev);
    }
    g_arch[dev] = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    if (g_arch[dev] == 2)
      return fail(SA_E_UNSUPPORTED, "device %d is %s; this library only runs on gfx950 (MI355X)", dev,
                  prop.gcnArchName);
  }
  if (g_arch[dev] != 1) return fail(SA_E_UNSUPPORTED, "device %d is not gfx950", dev);
  return SA_OK;
}

// Compute units of device dev, read once per device (256 on MI355X).
int g_cus[kMaxDev] = {0};

int device_cus(int dev) {
  if (dev < 0 || dev >= kMaxDev) return 256;
  std::lock_guard<std::mutex> lk(g_arch_mu);
  if (g_cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
      (void)hipGetLastError();
      n = 256;
    }
    g_cus[dev] = n;
  }
  return g_cus[dev];
}

int32_t check_current_device(int* dev_out = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SA_E_DEVICE, "no current HIP device");
  }
  if (dev_out) *dev_out = dev;
  return check_device(dev);
}

int32_t launched(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(SA_E_LAUNCH, "%s launch failed: %s", what, hipGetErrorString(e));
  return ok();
}

bool pos(int x) { return x > 0; }

// Shared validation of dims / params for route and fwd.
int32_t check_dims(const sa_dims* dm, const sa_route_params* p, bool has_vbs) {
  if (!dm || !p) return fail(SA_E_NULL, "dims and params must not be NULL");
  if (!pos(dm->B) || !pos(dm->H)) return fail(SA_E_SHAPE, "B and H must be >= 1 (got %d, %d)", dm->B, dm->H);
  if (dm->d != 64 && dm->d != 128) return fail(SA_E_SHAPE, "d must be 64 or 128 (got %d)", dm->d);
  if (dm->Lq < 0 || dm->Lq % 128) return fail(SA_E_SHAPE, "Lq must be a non-negative multiple of 128 (got %d)", dm->Lq);
  if (dm->Lkv < 0 || dm->Lkv % 128) return fail(SA_E_SHAPE, "Lkv must be a non-negative multiple of 128 (got %d)", dm->Lkv);
  if (dm->lq_valid < 0 || dm->lq_valid > dm->Lq) return fail(SA_E_SHAPE, "lq_valid %d outside [0, %d]", dm->lq_valid, dm->Lq);
  if (dm->lkv_valid < 0 || dm->lkv_valid > dm->Lkv)
    return fail(SA_E_SHAPE, "lkv_valid %d outside [0, %d]", dm->lkv_valid, dm->Lkv);
  if (p->kblock != 64 && p->kblock != 128) return fail(SA_E_VALUE, "kblock must be 64 or 128 (got %d)", p->kblock);
  if (p->k_scale_rows != 64 && p->k_scale_rows != 128)
    return fail(SA_E_VALUE, "k_scale_rows must be 64 or 128 (got %d)", p->k_scale_rows);
  if (p->centroids_per_block < 0 || p->centroids_per_block > 2)
    return fail(SA_E_VALUE, "centroids_per_block must be 0, 1 or 2 (got %d)", p->centroids_per_block);
  if (p->prefix_tokens < 0 || p->prefix_tokens % p->kblock)
    return fail(SA_E_VALUE, "prefix_tokens must be a non-negative multiple of kblock (got %d)", p->prefix_tokens);
  if (has_vbs) {
    if (dm->Lv <= 0 || dm->Lv % 64) return fail(SA_E_SHAPE, "Lv must be a positive multiple of 64 with v_block_src (got %d)", dm->Lv);
  } else if (dm->Lv != dm->Lkv) {
    return fail(SA_E_SHAPE, "Lv (%d) must equal Lkv (%d) without v_block_src", dm->Lv, dm->Lkv);
  }
  if (dm->Lkv / p->kblock > 65535 * 2) return fail(SA_E_SHAPE, "Lkv too long");
  return SA_OK;
}

// Key layout from the segment list, or from the prefix and the valid length.
int32_t build_layout(const sa_dims* dm, const sa_route_params* p, sa::KvLayout* lay) {
  *lay = sa::KvLayout{};
  lay->kblock = p->kblock;
  if (p->n_segments == 0) {
    lay->n = 2;
    lay->start[0] = 0;
    lay->end[0] = p->prefix_tokens < dm->lkv_valid ? p->prefix_tokens : dm->lkv_valid;
    lay->start[1] = p->prefix_tokens;
    lay->end[1] = dm->lkv_valid;
    lay->routed = 2u;
    return SA_OK;
  }
  if (p->n_segments < 0 || p->n_segments > SA_MAX_SEGMENTS)
    return fail(SA_E_VALUE, "n_segments must be in [0, %d] (got %d)", SA_MAX_SEGMENTS, p->n_segments);
  if (!p->segments_host) return fail(SA_E_NULL, "segments_host is required when n_segments > 0");
  if (p->prefix_tokens != 0) return fail(SA_E_VALUE, "prefix_tokens must be 0 when segments are given");
  int prev_end = 0;
  for (int x = 0; x < p->n_segments; ++x) {
    const sa_segment& g = p->segments_host[x];
    if (g.start < 0 || g.start % p->kblock)
      return fail(SA_E_VALUE, "segment %d: start %d is not a non-negative multiple of kblock", x, g.start);
    if (g.rows < 0 || g.start + g.rows > dm->lkv_valid)
      return fail(SA_E_VALUE, "segment %d: rows %d outside [0, lkv_valid - start]", x, g.rows);
    if (x > 0 && g.start < prev_end)
      return fail(SA_E_VALUE, "segment %d starts at %d, inside the previous segment", x, g.start);
    prev_end = g.start + g.rows;
    lay->start[x] = g.start;
    lay->end[x] = g.start + g.rows;
    if (g.routed) lay->routed |= 1u << x;
  }
  lay->n = p->n_segments;
  return SA_OK;
}

// The forward kernels address one head's K and V through 32-bit buffer
// offsets: each must stay below 4 GiB.
int32_t check_head_bytes(const sa_dims* dm, int k_bytes_per_elt, int v_bytes_per_elt, const char* who) {
  const int64_t kb = (int64_t)dm->Lkv * dm->d * k_bytes_per_elt, vb = (int64_t)dm->Lv * dm->d * v_bytes_per_elt;
  if (kb >= (int64_t)1 << 32 || vb >= (int64_t)1 << 32)
    return fail(SA_E_SHAPE, "%s: one head's K or V exceeds 4 GiB (%lld, %lld bytes)", who, (long long)kb, (long long)vb);
  return SA_OK;
}

int32_t check_v(int32_t v_dtype, const void* v, const float* v_scale, const sa_dims* dm, const sa_route_params* p) {
  if (v_dtype != SA_BF16 && v_dtype != SA_INT8) return fail(SA_E_VALUE, "v_dtype must be SA_BF16 or SA_INT8");
  if (!v) return fail(SA_E_NULL, "v must not be NULL");
  if (!aligned16(v)) return fail(SA_E_ALIGN, "v must be 16-byte aligned");
  if (v_dtype == SA_INT8) {
    if (!v_scale) return fail(SA_E_NULL, "v_scale is required for INT8 V");
    if (p->v_scale_rows != 64 && p->v_scale_rows != 128)
      return fail(SA_E_VALUE, "v_scale_rows must be 64 or 128 (got %d)", p->v_scale_rows);
    if (dm->Lv % p->v_scale_rows) return fail(SA_E_SHAPE, "Lv must be a multiple of v_scale_rows");
  }
  return SA_OK;
}

}  // namespace

extern "C" {

int32_t sa_abi_version(void) { return SA_ABI_VERSION; }

const char* sa_last_error(void) { return g_err; }

int32_t sa_device_check(int32_t device) {
  const int32_t rc = check_device(device);
  return rc == SA_OK ? ok() : rc;
}

int32_t quantize_qk_int8(const void* x_bf16, int64_t sB, int64_t sH, int64_t sL, int32_t B, int32_t H,
                         int32_t L, int32_t d, int32_t valid_len, int32_t rows_per_block, int8_t* x_q,
                         float* scale, int16_t* col_sums, int32_t sum_rows, void* stream) {
  if (!x_bf16 || !x_q || !scale) return fail(SA_E_NULL, "quantize_qk_int8: x, x_q and scale must not be NULL");
  if (B < 1 || H < 1 || L < 0) return fail(SA_E_SHAPE, "quantize_qk_int8: bad B/H/L (%d, %d, %d)", B, H, L);
  if (d != 64 && d != 128) return fail(SA_E_SHAPE, "quantize_qk_int8: d must be 64 or 128 (got %d)", d);
  if (rows_per_block != 64 && rows_per_block != 128)
    return fail(SA_E_VALUE, "quantize_qk_int8: rows_per_block must be 64 or 128 (got %d)", rows_per_block);
  if (L % rows_per_block) return fail(SA_E_SHAPE, "quantize_qk_int8: L (%d) must be a multiple of rows_per_block", L);
  if (valid_len < 0 || valid_len > L) return fail(SA_E_SHAPE, "quantize_qk_int8: valid_len %d outside [0, %d]", valid_len, L);
  if (!aligned16(x_bf16) || !aligned16(x_q)) return fail(SA_E_ALIGN, "quantize_qk_int8: x and x_q must be 16-byte aligned");
  if (sB % 8 || sH % 8 || sL % 8 || sL < d)
    return fail(SA_E_ALIGN, "quantize_qk_int8: strides must be multiples of 8 elements and sL >= d");
  if (col_sums && !aligned16(col_sums)) return fail(SA_E_ALIGN, "quantize_qk_int8: col_sums must be 16-byte aligned");
  if (col_sums && sum_rows != 32 && sum_rows != rows_per_block)
    return fail(SA_E_VALUE, "quantize_qk_int8: sum_rows must be 32 or rows_per_block (got %d)", sum_rows);
  if (const int32_t rc = check_current_device()) return rc;
  if (L == 0) return ok();
  sa::QuantizeArgs a{static_cast<const uint16_t*>(x_bf16), sB, sH, sL, B, H, L, d, valid_len, rows_per_block, x_q, scale,
                     L / rows_per_block, 0, col_sums, col_sums ? sum_rows : 32};
  return launched(sa::launch_quantize(a, static_cast<hipStream_t>(stream)), "quantize");
}

int32_t kv_cache_append_int8(const void* x_bf16, int64_t sB, int64_t sH, int64_t sL, int32_t B, int32_t H,
                             int32_t rows, int32_t d, int32_t valid_len, int32_t rows_per_slab, int8_t* cache_q,
                             float* cache_scale, int32_t slots, int32_t first_slot, void* stream) {
  if (!x_bf16 || !cache_q || !cache_scale)
    return fail(SA_E_NULL, "kv_cache_append_int8: x, cache_q and cache_scale must not be NULL");
  if (B < 1 || H < 1 || rows < 0) return fail(SA_E_SHAPE, "kv_cache_append_int8: bad B/H/rows (%d, %d, %d)", B, H, rows);
  if (d != 64 && d != 128) return fail(SA_E_SHAPE, "kv_cache_append_int8: d must be 64 or 128 (got %d)", d);
  if (rows_per_slab != 64 && rows_per_slab != 128)
    return fail(SA_E_VALUE, "kv_cache_append_int8: rows_per_slab must be 64 or 128 (got %d)", rows_per_slab);
  if (rows % rows_per_slab) return fail(SA_E_SHAPE, "kv_cache_append_int8: rows (%d) must be a multiple of rows_per_slab", rows);
  if (slots < 1 || rows / rows_per_slab > slots)
    return fail(SA_E_SHAPE, "kv_cache_append_int8: %d slabs do not fit a ring of %d slots", rows / rows_per_slab, slots);
  if (first_slot < 0 || first_slot >= slots)
    return fail(SA_E_VALUE, "kv_cache_append_int8: first_slot %d outside [0, %d)", first_slot, slots);
  if (valid_len < 0 || valid_len > rows) return fail(SA_E_SHAPE, "kv_cache_append_int8: valid_len %d outside [0, %d]", valid_len, rows);
  if (!aligned16(x_bf16) || !aligned16(cache_q)) return fail(SA_E_ALIGN, "kv_cache_append_int8: x and cache_q must be 16-byte aligned");
  if (sB % 8 || sH % 8 || sL % 8 || sL < d)
    return fail(SA_E_ALIGN, "kv_cache_append_int8: strides must be multiples of 8 elements and sL >= d");
  if (const int32_t rc = check_current_device()) return rc;
  if (rows == 0) return ok();
  sa::QuantizeArgs a{static_cast<const uint16_t*>(x_bf16), sB, sH, sL, B, H, rows, d, valid_len, rows_per_slab, cache_q,
                     cache_scale, slots, first_slot, nullptr, 32};
  return launched(sa::launch_quantize(a, static_cast<hipStream_t>(stream)), "kv_cache_append_int8");
}

size_t sparse_attn_route_workspace_size(const sa_dims* dims, const sa_route_params* p, int32_t has_explicit_map) {
  if (check_dims(dims, p, false) != SA_OK && check_dims(dims, p, true) != SA_OK) return 0;
  if (has_explicit_map) return 0;
  return sa::route_workspace_bytes(dims->B, dims->H, dims->Lq / 128, dims->Lkv / p->kblock, dims->d);
}

}  // extern "C"

namespace {

// The routing pass behind sparse_attn_route (workspace from the caller) and
// sparse_attn_route_noalloc (library-owned workspace: `noalloc` set, and
// workspace / workspace_bytes ignored).
int32_t route_impl(const int8_t* q, const int8_t* k, const float* k_scale, const void* v, int32_t v_dtype,
                   const float* v_scale, const int32_t* v_block_src, const int16_t* q_sums, const int16_t* k_sums,
                   const sa_dims* dims, const sa_route_params* p,
                   const uint8_t* explicit_map, uint8_t* block_map, float* k_centroid, float* v_centroid,
                   float* count, double* row_stats, void* workspace, size_t workspace_bytes, bool noalloc,
                   void* stream) {
  if (const int32_t rc = check_dims(dims, p, v_block_src != nullptr)) return rc;
  sa::KvLayout lay;
  if (const int32_t rc = build_layout(dims, p, &lay)) return rc;
  if ((!q && !q_sums) || (!k && !k_sums) || !k_scale || !block_map)
    return fail(SA_E_NULL, "sparse_attn_route: q (or q_sums), k (or k_sums), k_scale and block_map are required");
  if ((q && !aligned16(q)) || (k && !aligned16(k)) || (q_sums && !aligned16(q_sums)) || (k_sums && !aligned16(k_sums)))
    return fail(SA_E_ALIGN, "sparse_attn_route: q, k, q_sums and k_sums must be 16-byte aligned");
  const int G = p->centroids_per_block;
  const bool sol = explicit_map == nullptr;
  if (sol) {
    if (p->rule != SA_RULE_THRESHOLD && p->rule != SA_RULE_TOPK)
      return fail(SA_E_VALUE, "sparse_attn_route: rule must be SA_RULE_THRESHOLD or SA_RULE_TOPK (got %d)", p->rule);
    if (p->rule == SA_RULE_THRESHOLD) {
      if (G == 0) return fail(SA_E_VALUE, "sparse_attn_route: the threshold rule needs centroids_per_block 1 or 2");
      if (isnan(p->threshold)) return fail(SA_E_VALUE, "sparse_attn_route: threshold is NaN");
    } else if (!(p->sparsity >= 0.0f && p->sparsity <= 1.0f)) {
      return fail(SA_E_VALUE, "sparse_attn_route: sparsity must lie in [0, 1]");
    }
    if (p->k_scale_rows != p->kblock)
      return fail(SA_E_VALUE, "sparse_attn_route: routing rules need one K scale per key block (k_scale_rows == kblock)");
    if ((size_t)(dims->Lkv / p->kblock) * 8 > 49152)
      return fail(SA_E_SHAPE, "sparse_attn_route: at most 6144 key blocks per row for the routing rules");
  } else {
    if (p->map_kblock < p->kblock || p->map_kblock % p->kblock || dims->Lkv % p->map_kblock)
      return fail(SA_E_VALUE, "sparse_attn_route: map_kblock (%d) must be a multiple of kblock dividing Lkv", p->map_kblock);
  }
  if (G > 0) {
    if (!k_centroid || !v_centroid || !count) return fail(SA_E_NULL, "sparse_attn_route: centroid outputs are required when G > 0");
    if (!aligned16(k_centroid) || !aligned16(v_centroid)) return fail(SA_E_ALIGN, "sparse_attn_route: centroids must be 16-byte aligned");
    if (const int32_t rc = check_v(v_dtype, v, v_scale, dims, p)) return rc;
  }
  size_t need = 0;
  if (sol) {
    need = sa::route_workspace_bytes(dims->B, dims->H, dims->Lq / 128, dims->Lkv / p->kblock, dims->d);
    if (noalloc) {
      if (need > sa::kRouteScratchBytes)
        return fail(SA_E_WORKSPACE,
                    "sparse_attn_route_noalloc: these shapes need %zu bytes of workspace, more than the %zu the "
                    "library holds per device (SA_ROUTE_SCRATCH_BYTES); call sparse_attn_route with a workspace",
                    need, (size_t)sa::kRouteScratchBytes);
    } else {
      if (!workspace || workspace_bytes < need)
        return fail(SA_E_WORKSPACE, "sparse_attn_route: workspace of %zu bytes required (got %zu)", need,
                    workspace_bytes);
      if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return fail(SA_E_ALIGN, "sparse_attn_route: workspace must be 256-byte aligned");
    }
  }
  int dev = 0;
  if (const int32_t rc = check_current_device(&dev)) return rc;
  if (dims->Lq == 0 || dims->Lkv == 0) return ok();
  if (sol && noalloc) {
    const hipError_t e = sa::route_scratch(dev, &workspace);
    if (e != hipSuccess)
      return fail(SA_E_DEVICE, "sparse_attn_route_noalloc: no address for the library workspace on device %d: %s",
                  dev, hipGetErrorString(e));
  }
  sa::RouteArgs a{};
  a.lay = lay;
  a.q = q; a.k = k; a.k_scale = k_scale; a.v = v; a.v_int8 = v_dtype == SA_INT8; a.v_scale = v_scale;
  a.v_block_src = v_block_src;
  a.B = dims->B; a.H = dims->H; a.Lq = dims->Lq; a.Lkv = dims->Lkv; a.Lv = dims->Lv; a.d = dims->d;
  a.lq_valid = dims->lq_valid; a.lkv_valid = dims->lkv_valid;
  a.nQB = dims->Lq / 128; a.nKB = dims->Lkv / p->kblock; a.kblock = p->kblock; a.G = G;
  a.prefix = p->prefix_tokens; a.k_scale_rows = p->k_scale_rows; a.v_scale_rows = p->v_scale_rows;
  a.map_kblock = sol ? p->kblock : p->map_kblock; a.tau = p->threshold;
  a.rule = p->rule == SA_RULE_TOPK ? sa::kRuleTopK : sa::kRuleThreshold; a.sparsity = p->sparsity;
  a.explicit_map = explicit_map; a.map = block_map; a.kc = k_centroid; a.vc = v_centroid; a.cnt = count;
  a.stats = row_stats;
  a.q_sums = q_sums; a.k_sums = k_sums;
  a.num_cus = device_cus(dev);
  if (sol) {
    char* ws = static_cast<char*>(workspace);
    const size_t qbytes = ((size_t)a.B * a.H * a.nQB * 2 * a.d + 255) & ~(size_t)255;
    a.qdig = reinterpret_cast<int8_t*>(ws);
    a.kdig = reinterpret_cast<int8_t*>(ws + qbytes);
  }
  return launched(sa::launch_route(a, static_cast<hipStream_t>(stream)), "route");
}

}  // namespace

extern "C" {

int32_t sparse_attn_route(const int8_t* q, const int8_t* k, const float* k_scale, const void* v, int32_t v_dtype,
                          const float* v_scale, const int32_t* v_block_src, const int16_t* q_sums,
                          const int16_t* k_sums, const sa_dims* dims, const sa_route_params* p,
                          const uint8_t* explicit_map, uint8_t* block_map, float* k_centroid, float* v_centroid,
                          float* count, double* row_stats, void* workspace, size_t workspace_bytes, void* stream) {
  return route_impl(q, k, k_scale, v, v_dtype, v_scale, v_block_src, q_sums, k_sums, dims, p, explicit_map,
                    block_map, k_centroid, v_centroid, count, row_stats, workspace, workspace_bytes, false, stream);
}

int32_t sparse_attn_route_noalloc(const int8_t* q, const int8_t* k, const float* k_scale, const void* v,
                                  int32_t v_dtype, const float* v_scale, const int32_t* v_block_src,
                                  const int16_t* q_sums, const int16_t* k_sums, const sa_dims* dims,
                                  const sa_route_params* p, const uint8_t* explicit_map, uint8_t* block_map,
                                  float* k_centroid, float* v_centroid, float* count, double* row_stats,
                                  void* stream) {
  return route_impl(q, k, k_scale, v, v_dtype, v_scale, v_block_src, q_sums, k_sums, dims, p, explicit_map,
                    block_map, k_centroid, v_centroid, count, row_stats, nullptr, 0, true, stream);
}

int32_t sparse_attn_fwd(const int8_t* q, const float* q_scale, const int8_t* k, const float* k_scale, const void* v,
                        int32_t v_dtype, const float* v_scale, const int32_t* v_block_src, const sa_dims* dims,
                        const sa_route_params* p, const uint8_t* block_map, const float* k_centroid,
                        const float* v_centroid, const float* count, float sm_scale, void* out, int32_t out_dtype,
                        float* lse, void* stream) {
  if (const int32_t rc = check_dims(dims, p, v_block_src != nullptr)) return rc;
  sa::KvLayout lay;
  if (const int32_t rc = build_layout(dims, p, &lay)) return rc;
  if (!q || !q_scale || !k || !k_scale || !block_map || !out)
    return fail(SA_E_NULL, "sparse_attn_fwd: q, q_scale, k, k_scale, block_map and out are required");
  if (!aligned16(q) || !aligned16(k) || !aligned16(out)) return fail(SA_E_ALIGN, "sparse_attn_fwd: q, k and out must be 16-byte aligned");
  if (const int32_t rc = check_v(v_dtype, v, v_scale, dims, p)) return rc;
  if (out_dtype != SA_F32 && out_dtype != SA_BF16) return fail(SA_E_VALUE, "sparse_attn_fwd: out_dtype must be SA_F32 or SA_BF16");
  if (!(sm_scale > 0.0f) || isinf(sm_scale)) return fail(SA_E_VALUE, "sparse_attn_fwd: sm_scale must be positive and finite");
  if (p->centroids_per_block > 0) {
    if (!k_centroid || !v_centroid || !count) return fail(SA_E_NULL, "sparse_attn_fwd: centroids are required when G > 0");
    if (!aligned16(k_centroid) || !aligned16(v_centroid)) return fail(SA_E_ALIGN, "sparse_attn_fwd: centroids must be 16-byte aligned");
  }
  if (dims->Lkv % p->kblock) return fail(SA_E_SHAPE, "sparse_attn_fwd: Lkv must be a multiple of kblock");
  if (const int32_t rc = check_head_bytes(dims, 1, v_dtype == SA_INT8 ? 1 : 2, "sparse_attn_fwd")) return rc;
  if (const int32_t rc = check_current_device()) return rc;
  if (dims->Lq == 0) return ok();
  sa::FwdArgs a{};
  a.lay = lay;
  a.q = q; a.q_scale = q_scale; a.k = k; a.k_scale = k_scale; a.v = v; a.v_scale = v_scale; a.v_block_src = v_block_src;
  a.map = block_map; a.kc = k_centroid; a.vc = v_centroid; a.cnt = count; a.out = out; a.lse = lse;
  a.B = dims->B; a.H = dims->H; a.Lq = dims->Lq; a.Lkv = dims->Lkv; a.Lv = dims->Lv; a.d = dims->d;
  a.lq_valid = dims->lq_valid; a.lkv_valid = dims->lkv_valid;
  a.nQB = dims->Lq / 128; a.nKB = dims->Lkv / p->kblock; a.kblock = p->kblock; a.G = p->centroids_per_block;
  a.k_scale_rows = p->k_scale_rows; a.v_scale_rows = p->v_scale_rows;
  a.ks_shift = p->k_scale_rows == 128 ? 7 : 6;
  a.vs_shift = v_dtype == SA_INT8 && p->v_scale_rows == 128 ? 7 : 6;
  a.v_int8 = v_dtype == SA_INT8; a.out_bf16 = out_dtype == SA_BF16;
  a.sm_log2 = sm_scale * 1.4426950408889634f;
  if ((int64_t)a.B * a.H * a.nQB > 0x7FFFFFFF) return fail(SA_E_SHAPE, "sparse_attn_fwd: too many query blocks");
  return launched(sa::launch_fwd(a, static_cast<hipStream_t>(stream)), "fwd");
}

int32_t sparse_attn_fwd_float(const void* q_bf16, const void* k_bf16, const void* v_bf16, const int32_t* v_block_src,
                              const sa_dims* dims, const sa_route_params* p, const uint8_t* block_map,
                              const float* k_centroid, const float* v_centroid, const float* count, float sm_scale,
                              void* out, int32_t out_dtype, float* lse, void* stream) {
  if (const int32_t rc = check_dims(dims, p, v_block_src != nullptr)) return rc;
  sa::KvLayout lay;
  if (const int32_t rc = build_layout(dims, p, &lay)) return rc;
  if (!q_bf16 || !k_bf16 || !v_bf16 || !block_map || !out)
    return fail(SA_E_NULL, "sparse_attn_fwd_float: q, k, v, block_map and out are required");
  if (!aligned16(q_bf16) || !aligned16(k_bf16) || !aligned16(v_bf16) || !aligned16(out))
    return fail(SA_E_ALIGN, "sparse_attn_fwd_float: q, k, v and out must be 16-byte aligned");
  if (out_dtype != SA_F32 && out_dtype != SA_BF16) return fail(SA_E_VALUE, "sparse_attn_fwd_float: out_dtype must be SA_F32 or SA_BF16");
  if (!(sm_scale > 0.0f) || isinf(sm_scale)) return fail(SA_E_VALUE, "sparse_attn_fwd_float: sm_scale must be positive and finite");
  if (p->centroids_per_block > 0) {
    if (!k_centroid || !v_centroid || !count) return fail(SA_E_NULL, "sparse_attn_fwd_float: centroids are required when G > 0");
    if (!aligned16(k_centroid) || !aligned16(v_centroid)) return fail(SA_E_ALIGN, "sparse_attn_fwd_float: centroids must be 16-byte aligned");
  }
  if (dims->Lkv % p->kblock) return fail(SA_E_SHAPE, "sparse_attn_fwd_float: Lkv must be a multiple of kblock");
  if (const int32_t rc = check_head_bytes(dims, 2, 2, "sparse_attn_fwd_float")) return rc;
  if ((int64_t)dims->B * dims->H * (dims->Lq / 128) > 0x7FFFFFFF) return fail(SA_E_SHAPE, "sparse_attn_fwd_float: too many query blocks");
  if (const int32_t rc = check_current_device()) return rc;
  if (dims->Lq == 0) return ok();
  sa::FwdFloatArgs a{};
  a.q = static_cast<const uint16_t*>(q_bf16); a.k = static_cast<const uint16_t*>(k_bf16);
  a.v = static_cast<const uint16_t*>(v_bf16); a.v_block_src = v_block_src;
  a.map = block_map; a.kc = k_centroid; a.vc = v_centroid; a.cnt = count; a.out = out; a.lse = lse;
  a.B = dims->B; a.H = dims->H; a.Lq = dims->Lq; a.Lkv = dims->Lkv; a.Lv = dims->Lv; a.d = dims->d;
  a.lq_valid = dims->lq_valid; a.lkv_valid = dims->lkv_valid;
  a.nQB = dims->Lq / 128; a.nKB = dims->Lkv / p->kblock; a.kblock = p->kblock; a.G = p->centroids_per_block;
  a.lay = lay; a.out_bf16 = out_dtype == SA_BF16; a.sm_log2 = sm_scale * 1.4426950408889634f;
  return launched(sa::launch_fwd_float(a, static_cast<hipStream_t>(stream)), "fwd_float");
}

int32_t gather_virtual_kv(const void* k_phys_bf16, int32_t B, int32_t H, int32_t rows_per_slice, int32_t n_phys,
                          int32_t d, const int32_t* src_map_host, int32_t n_logical, const float* rope_cos,
                          const float* rope_sin, int32_t rot_offset, int32_t d_rot, int32_t k_rows_per_block,
                          int8_t* k_logical, float* k_scale, int32_t* v_block_src, void* stream) {
  if (!k_phys_bf16 || !src_map_host || !k_logical || !k_scale || !v_block_src)
    return fail(SA_E_NULL, "gather_virtual_kv: k_phys, src_map_host, k_logical, k_scale and v_block_src are required");
  if (B < 1 || H < 1 || n_phys < 1 || rows_per_slice < 1) return fail(SA_E_SHAPE, "gather_virtual_kv: bad sizes");
  if (d != 64 && d != 128) return fail(SA_E_SHAPE, "gather_virtual_kv: d must be 64 or 128 (got %d)", d);
  if (n_logical < 1 || n_logical > sa::kMaxLogical)
    return fail(SA_E_SHAPE, "gather_virtual_kv: n_logical must be in [1, %d] (got %d)", sa::kMaxLogical, n_logical);
  if (k_rows_per_block != 64 && k_rows_per_block != 128)
    return fail(SA_E_VALUE, "gather_virtual_kv: k_rows_per_block must be 64 or 128");
  if (rows_per_slice % k_rows_per_block || rows_per_slice % 64)
    return fail(SA_E_SHAPE, "gather_virtual_kv: rows_per_slice must be a multiple of 64 and of k_rows_per_block");
  if (d_rot < 0 || d_rot % 2 || rot_offset < 0 || rot_offset % 2 || rot_offset + d_rot > d)
    return fail(SA_E_VALUE, "gather_virtual_kv: need even rot_offset and d_rot with rot_offset + d_rot <= d");
  if (d_rot > 0 && (!rope_cos || !rope_sin)) return fail(SA_E_NULL, "gather_virtual_kv: rope tables are required");
  if (!aligned16(k_phys_bf16) || !aligned16(k_logical)) return fail(SA_E_ALIGN, "gather_virtual_kv: k tensors must be 16-byte aligned");
  sa::SrcMap sm{};
  for (int l = 0; l < n_logical; ++l) {
    if (src_map_host[l] < 0 || src_map_host[l] >= n_phys)
      return fail(SA_E_VALUE, "gather_virtual_kv: src_map[%d] = %d outside [0, %d)", l, src_map_host[l], n_phys);
    sm.v[l] = src_map_host[l];
  }
  if (const int32_t rc = check_current_device()) return rc;
  sa::GatherArgs a{static_cast<const uint16_t*>(k_phys_bf16), B, H, rows_per_slice, n_phys, d, n_logical, rot_offset,
                   d_rot, k_rows_per_block, sm, rope_cos, rope_sin, k_logical, k_scale, v_block_src};
  return launched(sa::launch_gather(a, static_cast<hipStream_t>(stream)), "gather_virtual_kv");
}

}  // extern "C"
