// Internal launch interface between the C ABI layer (abi.hip) and the kernels.
// Every struct carries already-validated arguments; launchers only enqueue.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sa {

constexpr int kQBlock = 128;     // query rows per routing block
constexpr int kTile = 64;        // key rows per exact tile in the forward kernel
constexpr int kMaxLogical = 16;  // virtual-KV logical slices passed by value
constexpr int kRuleThreshold = 0;  // routing rules, as in the C ABI
constexpr int kRuleTopK = 1;

struct SrcMap {
  int32_t v[kMaxLogical];
};

// Key layout: up to kMaxSegments segments in increasing start, each starting on
// a key-block boundary; valid key rows are [start, end) of a segment (end
// already capped at the valid length).  A key block lies in at most one
// segment, and its valid rows are a prefix of the block.  The plain layout
// (a dense prefix, then routed rows up to the valid length) is two segments.
constexpr int kMaxSegments = 16;

struct KvLayout {
  int n;
  int start[kMaxSegments];
  int end[kMaxSegments];
  uint32_t routed;   // bit s set: segment s is routed
  int kblock;

  // segment holding row r (the last starting at or before it), or -1
  __host__ __device__ int seg_of(int r) const {
    int s = -1;
    for (int x = 0; x < n; ++x) s = start[x] <= r ? x : s;
    return s;
  }
  // valid rows of key block j (a prefix of the block)
  __host__ __device__ int block_rows(int j) const {
    const int r0 = j * kblock, s = seg_of(r0);
    if (s < 0) return 0;
    const int v = end[s] - r0;
    return v < 0 ? 0 : (v > kblock ? kblock : v);
  }
  __host__ __device__ bool block_routed(int j) const {
    const int s = seg_of(j * kblock);
    return s >= 0 && ((routed >> s) & 1u);
  }
};

struct QuantizeArgs {
  const uint16_t* x;
  int64_t sB, sH, sL;
  int B, H, L, d, valid_len, R;
  int8_t* q;
  float* scale;
  int nslots, first;   // destination: block b goes to slot (first + b) % nslots of q / scale
  int16_t* sums;       // optional column sums of the codes per sum_rows chunk [B,H,L/sum_rows,d] (plain quantization)
  int sum_rows;        // 32 or R
};

struct GatherArgs {
  const uint16_t* kp;
  int B, H, S, n_phys, d, n_logical, rot_offset, d_rot, R;
  SrcMap src;
  const float* cosv;
  const float* sinv;
  int8_t* kq;
  float* kscale;
  int32_t* vbs;
};

struct RouteArgs {
  const int8_t* q;
  const int8_t* k;
  const float* k_scale;
  const void* v;
  bool v_int8;
  const float* v_scale;
  const int32_t* v_block_src;
  int B, H, Lq, Lkv, Lv, d, lq_valid, lkv_valid;
  int nQB, nKB, kblock, G, prefix, k_scale_rows, v_scale_rows, map_kblock;
  KvLayout lay;
  int rule;        // kRuleThreshold or kRuleTopK (routing rules without an explicit map)
  float tau;       // threshold rule
  float sparsity;  // fixed-sparsity rule: fraction of candidates pruned
  const uint8_t* explicit_map;
  uint8_t* map;
  float* kc;
  float* vc;
  float* cnt;
  double* stats;
  int8_t* qdig;    // workspace [B,H,nQB][2][d]: query-block column sums as two int8 digits (Sol rule only)
  int8_t* kdig;    // workspace [B,H,nKB][2][d]: key-block column sums, same form (Sol rule only)
  int num_cus;     // compute units of the device (sizes the decision grid)
  const int16_t* q_sums;   // optional: the quantizer's column sums of Q per 128-row block [B,H,Lq/128,d]
  const int16_t* k_sums;   // optional: the same for K per 32-row chunk [B,H,Lkv/32,d]
};

struct FwdArgs {
  const int8_t* q;
  const float* q_scale;
  const int8_t* k;
  const float* k_scale;
  const uint16_t* qb;   // floating path: bf16 Q [B,H,Lq,d] and K [B,H,Lkv,d] instead of q/k and their scales
  const uint16_t* kb;
  const void* v;
  const float* v_scale;
  const int32_t* v_block_src;
  const uint8_t* map;
  const float* kc;
  const float* vc;
  const float* cnt;
  void* out;
  float* lse;
  int B, H, Lq, Lkv, Lv, d, lq_valid, lkv_valid;
  int nQB, nKB, kblock, G, k_scale_rows, v_scale_rows;
  int ks_shift, vs_shift;   // log2 of k_scale_rows and v_scale_rows
  KvLayout lay;
  bool v_int8, out_bf16;
  float sm_log2;   // sm_scale * log2(e)
};

// Forward with a floating QK^T: bf16 Q [B,H,Lq,d], K [B,H,Lkv,d], V [B,H,Lv,d].
struct FwdFloatArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* v_block_src;
  const uint8_t* map;
  const float* kc;
  const float* vc;
  const float* cnt;
  void* out;
  float* lse;
  int B, H, Lq, Lkv, Lv, d, lq_valid, lkv_valid;
  int nQB, nKB, kblock, G;
  KvLayout lay;
  bool out_bf16;
  float sm_log2;   // sm_scale * log2(e)
};

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st);
hipError_t launch_fwd_float(const FwdFloatArgs& a, hipStream_t st);
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);
hipError_t launch_route(const RouteArgs& a, hipStream_t st);
hipError_t launch_fwd(const FwdArgs& a, hipStream_t st);

// Route workspace layout: qdig then kdig, each 256-byte aligned.
size_t route_workspace_bytes(int B, int H, int nQB, int nKB, int d);

// The library-owned route workspace of kRouteScratchBytes per device: its
// device address on device dev (which must be the current device).
constexpr size_t kRouteScratchBytes = size_t(16) << 20;
hipError_t route_scratch(int dev, void** ptr);

}  // namespace sa
