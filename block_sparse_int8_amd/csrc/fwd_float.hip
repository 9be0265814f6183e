// Block-sparse attention forward with a floating QK^T (gfx950).
//
// Configure Sol Sparse Attention, "How it works": with a floating dense backend
// the kept blocks are computed in floating point instead of on the W8A8
// integer path; the block map and the centroids are the same (routed on the
// INT8 codes).  Here the exact tiles take bf16 Q and K.
//
// Same shape as the INT8 kernel: one workgroup of 4 waves per 128-row query
// block, wave w owning query rows 32w..32w+31; 64-key tiles as two 32-key
// online-softmax steps; S^T = K.Q^T so each lane holds one query row's scores
// in the operand layout the PV product takes; O^T += V^T.P^T with V^T read by
// ds_read_b64_tr_b16; centroid columns 32 at a time in the same softmax.
// Differences: S^T on v_mfma_f32_32x32x16_bf16 (D/16 k-steps per half) from a
// bf16 K tile, scores straight in fp32 (the weights use the INT8 kernel's fast
// path against a lagging running max, with the same hand interleaving of one
// half's weights with the other half's matrix work), and tile copies straight
// into LDS: the next tile's copy goes into the other stage while the current
// tile is computed.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kFWin = 512;       // map entries scanned per list-building window
constexpr float kFLazy = 8.0f;   // rescale O only when the row max grows by more than 2^8

template <int D>
struct FltLds {
  static constexpr int KSTR = 2 * D + 16;   // bf16 K tile row stride (bytes); also centroid K rows
  static constexpr int VSTR = 2 * D + 64;   // bf16 V tile row stride (bytes)
  static constexpr int V_OFF = kTile * KSTR;
  static constexpr int STAGE = V_OFF + kTile * VSTR;
  static constexpr int KCL_OFF = 32 * KSTR;   // centroid K lo rows (hi rows at 0), in stage 0
  static constexpr int VCL_OFF = 32 * VSTR;   // centroid V lo rows (hi rows at 0), in stage 1
  static_assert(2 * 32 * KSTR <= STAGE && 2 * 32 * VSTR <= STAGE, "centroid staging must fit a stage");
  static_assert(V_OFF % 1024 == 0 && (kTile * KSTR) % 1024 == 0 && (kTile * VSTR) % 1024 == 0,
                "copy instructions write whole 1 KiB chunks");
};

__device__ __forceinline__ v4bf ftr16(const uint8_t* p) {
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS v4s*)(p));
  return __builtin_bit_cast(v4bf, r);
}

__device__ __forceinline__ v8bf fcat8(v4bf a, v4bf b) {
  return (v8bf){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

__device__ __forceinline__ float fpair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

template <int NS>
__device__ __forceinline__ void frescale(float m_tile, float& m_run, float& l_run, v16f (&O)[NS]) {
  const bool need = m_tile > m_run + kFLazy;
  if (__ballot(need)) {
    const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_tile) : 1.0f;
    if (need) m_run = m_tile;
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < NS; ++c) O[c] *= alpha;
  }
}

// Tile copies straight into LDS (buffer_load_dwordx4 ... lds): lane L of a
// wave instruction writes LDS bytes 16L..16L+15 of that instruction's 1 KiB
// chunk, so the padded row layout comes from each lane's source offset; lanes
// on padding read past the buffer (zeros, no memory access).  Instruction u
// of a tile belongs to wave u % 4.  The LDS address is handed over as a
// wave-uniform integer the compiler cannot trace to an LDS variable, so it
// adds no wait of its own before later LDS reads; the tile loop's barriers
// wait for the copies.  Kept out of templates (the host pass only accepts the
// builtin in a plain function).
constexpr uint32_t kFPad = 0xFFFFFFF0u;

__device__ __forceinline__ void flt_dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff,
                                          uint32_t lds_addr) {
  lds_addr = __builtin_amdgcn_readfirstlane(lds_addr);
  asm volatile("" : "+s"(lds_addr));
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (SA_LDS void*)(uintptr_t)lds_addr, 16, voff, soff, 0, 0);
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t flt_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes, 0x00020000);
}

template <int D>
struct FltPlan {
  static constexpr int KU = FltLds<D>::KSTR / 16, VU = FltLds<D>::VSTR / 16;   // 16-byte units per row
  static constexpr int KN = kTile * KU / 64, VN = kTile * VU / 64;               // wave instructions per tile
  static constexpr int KI = (KN + 3) / 4, VI = (VN + 3) / 4;                     // per wave (at most)
  uint32_t koff[KI], voff[VI];
};

template <int D>
__device__ __forceinline__ FltPlan<D> flt_plan(int wave, int lane) {
  using P = FltPlan<D>;
  P pl;
#pragma unroll
  for (int t = 0; t < P::KI; ++t) {
    const int u = (wave + 4 * t) * 64 + lane, row = u / P::KU, cc = u % P::KU;
    pl.koff[t] = cc < 2 * D / 16 ? (uint32_t)(row * 2 * D + cc * 16) : kFPad;
  }
#pragma unroll
  for (int t = 0; t < P::VI; ++t) {
    const int u = (wave + 4 * t) * 64 + lane, row = u / P::VU, cc = u % P::VU;
    pl.voff[t] = cc < 2 * D / 16 ? (uint32_t)(row * 2 * D + cc * 16) : kFPad;
  }
  return pl;
}

// Issue this wave's share of the copy of a tile (K rows from krow0, V rows
// from vrow0) into stage.
template <int D>
__device__ __forceinline__ void flt_copy(const FltPlan<D>& pl, __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                         int krow0, int vrow0, uint8_t* stage, int wave) {
  using P = FltPlan<D>;
  const uint32_t base = (uint32_t)(uintptr_t)(SA_LDS const void*)stage;
#pragma unroll
  for (int t = 0; t < P::KI; ++t)
    if (wave + 4 * t < P::KN) flt_dma16(krs, pl.koff[t], (uint32_t)krow0 * 2 * D, base + (wave + 4 * t) * 1024);
#pragma unroll
  for (int t = 0; t < P::VI; ++t)
    if (wave + 4 * t < P::VN)
      flt_dma16(vrs, pl.voff[t], (uint32_t)vrow0 * 2 * D, base + FltLds<D>::V_OFF + (wave + 4 * t) * 1024);
}

// Wait for this wave's copies into LDS, then the workgroup barrier: after it
// every copy issued before it has landed.
__device__ __forceinline__ void flt_copies_done_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// Physical first row of V for logical 64-row key tile kt.
__device__ __forceinline__ int flt_vrow(const FwdFloatArgs& a, int kt) {
  return a.v_block_src ? __builtin_amdgcn_readfirstlane(min(max(a.v_block_src[kt], 0), a.Lv / kTile - 1) * kTile)
                       : kt * kTile;
}

// O^T += V^T.P^T for one 32-key half (keys key0..key0+31 of the staged tile).
template <int D>
__device__ __forceinline__ void flt_half_pv(const uint8_t* vbuf, int key0, const uint32_t (&pw)[8], v16f (&O)[D / 32],
                                            int vlane) {
  using L = FltLds<D>;
  constexpr int NS = D / 32;
#pragma unroll
  for (int i = 0; i < 2 * NS; ++i) {
    const uint8_t* p0 = vbuf + vlane + (key0 + (i / NS) * 16) * L::VSTR + (i % NS) * 64;
    const int k2 = i / NS;
    const v4i pwv = (v4i){(int)pw[k2 * 4], (int)pw[k2 * 4 + 1], (int)pw[k2 * 4 + 2], (int)pw[k2 * 4 + 3]};
    O[i % NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fcat8(ftr16(p0), ftr16(p0 + 8 * L::VSTR)),
                                                         __builtin_bit_cast(v8bf, pwv), O[i % NS], 0, 0, 0);
  }
}

// One 32-key half: scores acc (fp32 dots) times c = sm_scale*log2(e); keys at
// or past nvalid (within the tile) are masked.  Moves m_run lazily, then the
// bf16 weights exp2(acc*c - m_run) go to pw; returns the lane's row-sum part
// (the bf16-rounded weights, as the PV product uses them).
template <int NS, bool MASKED>
__device__ __forceinline__ float flt_half_softmax(const v16f& acc, int key0, float c, int nvalid, int hh,
                                                  v16f (&O)[NS], float& m_run, float& l_run, uint32_t (&pw)[8]) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  float mx = -INFINITY;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    float v = acc[e];
    if (MASKED) v = key0 + (e / 4) * 8 + hh * 4 + (e % 4) < nvalid ? v : -INFINITY;
    mx = fmaxf(mx, v);
  }
  mx = fpair_max(mx);
  frescale<NS>(mx == -INFINITY ? -INFINITY : mx * c, m_run, l_run, O);
  const float m = m_run == -INFINITY ? 0.0f : m_run;
  float psum = 0.0f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2 * e], c, -m));
    float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2 * e + 1], c, -m));
    if (MASKED) {
      const int k0 = key0 + ((2 * e) / 4) * 8 + hh * 4 + (2 * e) % 4;
      p0 = k0 < nvalid ? p0 : 0.0f;
      p1 = k0 + 1 < nvalid ? p1 : 0.0f;
    }
    if (m_run == -INFINITY) p0 = p1 = 0.0f;   // nothing valid in this row yet
    const v2bf pk = (v2bf){(__bf16)p0, (__bf16)p1};
    psum = __builtin_amdgcn_fdot2_f32_bf16(pk, (v2bf){(__bf16)1.0f, (__bf16)1.0f}, psum, false);
    pw[e] = __builtin_bit_cast(uint32_t, pk);
  }
  return psum;
}

// Fast-path acceptance bound on a lane's partial row sum (weights taken against
// a running max that lags the scores stay far from fp32/bf16 overflow).
constexpr float kFFastSum = 4096.0f;

__device__ __forceinline__ bool flt_fast_ok(float psum) { return __ballot(!(psum <= kFFastSum)) == 0; }

// Weights 2e, 2e+1 of a half against the current m (b = -m): two FMAs, two
// exp2, one bf16 pack and the row-sum update.
__device__ __forceinline__ void flt_weight_pair(const v16f& acc, int e, float c, float b, float& psum,
                                                uint32_t (&pw)[8]) {
  typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
  const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2 * e], c, b));
  const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(acc[2 * e + 1], c, b));
  const v2bf pk = (v2bf){(__bf16)p0, (__bf16)p1};
  psum = __builtin_amdgcn_fdot2_f32_bf16(pk, (v2bf){(__bf16)1.0f, (__bf16)1.0f}, psum, false);
  pw[e] = __builtin_bit_cast(uint32_t, pk);
}

// One staged 64-key tile (keys >= nvalid masked when MASKED).
//   Full tiles: each half's weights are first taken against m_run as it
//   stands and kept when every lane's partial row sum is finite and at most
//   kFFastSum, else recomputed after moving m_run (the first tile, a jump in
//   the scores).  A wave issues in order, so the weights of half 0 are placed
//   between the QK MFMAs of half 1 and those of half 1 between the PV MFMAs
//   of half 0, in fixed scheduling segments.
//   Masked tiles: max, rescale and weights per half.
template <int D, bool MASKED>
__device__ __forceinline__ void flt_tile(const uint8_t* buf, const v8bf (&qf)[D / 16], v16f (&O)[D / 32],
                                         float& m_run, float& l_run, float c, int nvalid, int klane, int vlane,
                                         int hh) {
  using L = FltLds<D>;
  constexpr int NS = D / 32, KS = D / 16;
  const uint8_t* vbuf = buf + L::V_OFF;
  v16f acc0 = (v16f){}, acc1 = (v16f){};
#pragma unroll
  for (int s = 0; s < KS; ++s)
    acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const v8bf*>(buf + klane + s * 32), qf[s], acc0,
                                                   0, 0, 0);
  uint32_t pw0[8], pw1[8];
  if (MASKED) {
#pragma unroll
    for (int s = 0; s < KS; ++s)
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const v8bf*>(buf + klane + 32 * L::KSTR + s * 32), qf[s], acc1, 0, 0, 0);
    l_run += flt_half_softmax<NS, true>(acc0, 0, c, nvalid, hh, O, m_run, l_run, pw0);
    flt_half_pv<D>(vbuf, 0, pw0, O, vlane);
    l_run += flt_half_softmax<NS, true>(acc1, 32, c, nvalid, hh, O, m_run, l_run, pw1);
    flt_half_pv<D>(vbuf, 32, pw1, O, vlane);
    return;
  }
  // QK of half 1, interleaved with the weights of half 0
  float ps0 = 0.0f;
  {
    const float b = -m_run;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          *reinterpret_cast<const v8bf*>(buf + klane + 32 * L::KSTR + s * 32), qf[s], acc1, 0, 0, 0);
#pragma unroll
      for (int e = s * 8 / KS; e < (s + 1) * 8 / KS; ++e) flt_weight_pair(acc0, e, c, b, ps0, pw0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (!flt_fast_ok(ps0)) ps0 = flt_half_softmax<NS, false>(acc0, 0, c, kTile, hh, O, m_run, l_run, pw0);
  l_run += ps0;
  // PV of half 0, interleaved with the weights of half 1
  float ps1 = 0.0f;
  {
    const float b = -m_run;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * NS; ++i) {
      const uint8_t* p0 = vbuf + vlane + ((i / NS) * 16) * L::VSTR + (i % NS) * 64;
      const int k2 = i / NS;
      const v4i pwv = (v4i){(int)pw0[k2 * 4], (int)pw0[k2 * 4 + 1], (int)pw0[k2 * 4 + 2], (int)pw0[k2 * 4 + 3]};
      O[i % NS] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fcat8(ftr16(p0), ftr16(p0 + 8 * L::VSTR)),
                                                           __builtin_bit_cast(v8bf, pwv), O[i % NS], 0, 0, 0);
#pragma unroll
      for (int e = i * 8 / (2 * NS); e < (i + 1) * 8 / (2 * NS); ++e) flt_weight_pair(acc1, e, c, b, ps1, pw1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  if (!flt_fast_ok(ps1)) ps1 = flt_half_softmax<NS, false>(acc1, 32, c, kTile, hh, O, m_run, l_run, pw1);
  l_run += ps1;
  flt_half_pv<D>(vbuf, 32, pw1, O, vlane);
}

}  // namespace

template <int D, bool OBF16>
__global__ __launch_bounds__(256, 2) void fwd_float_kernel(FwdFloatArgs a) {
  using L = FltLds<D>;
  constexpr int NS = D / 32, KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint8_t stage0[L::STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t stage1[L::STAGE];
  __shared__ uint16_t elist[2 * kFWin];
  __shared__ uint16_t clist[kFWin];
  __shared__ int plist[kMaxSegments], pvalid[kMaxSegments];
  __shared__ float bias[32];
  __shared__ int cnts[3];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hh = lane >> 5;
  const int klane = n * L::KSTR + hh * 16;
  const int vlane = (hh * 4 + ((lane & 15) >> 2)) * L::VSTR + (((lane >> 4) & 1) * 16 + 4 * (lane & 3)) * 2;

  // XCD-aware block order, as in the INT8 kernel
  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  if ((nwg & 7) == 0) bid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int i = bid % a.nQB;
  const int64_t bh = bid / a.nQB;
  const int tpb = a.kblock / kTile;

  // Q fragment (B operand): lane holds query row n of this wave, channels
  // s*16 + hh*8 .. +7 for k-step s.
  const int qrow = i * kQBlock + wave * 32 + n;
  v8bf qf[KS];
  {
    const uint16_t* qp = a.q + (bh * a.Lq + qrow) * D + hh * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *reinterpret_cast<const v8bf*>(qp + s * 16);
  }
  const float c = a.sm_log2;
  v16f O[NS];
#pragma unroll
  for (int cc = 0; cc < NS; ++cc) O[cc] = (v16f){};
  float m_run = -INFINITY, l_run = 0.0f;
  const uint8_t* mrow = a.map + (bh * a.nQB + i) * a.nKB;
  // buffer resources over this head's K and V (per-head sizes fit 32 bits:
  // checked when the call is validated)
  const __amdgpu_buffer_rsrc_t krs = flt_rsrc(a.k + bh * a.Lkv * D, (uint32_t)((int64_t)a.Lkv * D * 2));
  const __amdgpu_buffer_rsrc_t vrs = flt_rsrc(a.v + bh * a.Lv * D, (uint32_t)((int64_t)a.Lv * D * 2));
  const FltPlan<D> plan = flt_plan<D>(wave, lane);
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);   // uniform copy of the wave index

  for (int w0 = 0; w0 < a.nKB; w0 += kFWin) {
    const int wend = min(a.nKB, w0 + kFWin);
    __syncthreads();
    if (wave == 0) {
      // full exact tiles -> elist; the tile holding a segment's last valid key
      // -> plist with its valid count; centroid blocks -> clist
      int nE = 0, nC = 0, nP = 0;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int c0 = w0; c0 < wend; c0 += 64) {
        const int j = c0 + lane;
        const int st = j < wend ? mrow[j] : 0;
        const bool isE = st == 1, isC = st == 2 && a.G > 0;
        const int nv = isE ? a.lay.block_rows(j) : 0;
        const int nf = nv / kTile, pv = nv % kTile;
        const uint64_t b0 = __ballot(nf & 1), b1 = __ballot(nf & 2), bC = __ballot(isC), bP = __ballot(pv > 0);
        if (nf) {
          const int pos = nE + __popcll(b0 & lt) + 2 * __popcll(b1 & lt);
          for (int sub = 0; sub < nf; ++sub) elist[pos + sub] = (uint16_t)((j - w0) * tpb + sub);
        }
        if (pv > 0) {
          const int pos = nP + __popcll(bP & lt);
          if (pos < kMaxSegments) {
            plist[pos] = j * tpb + nf;
            pvalid[pos] = pv;
          }
        }
        if (isC) clist[nC + __popcll(bC & lt)] = (uint16_t)(j - w0);
        nE += __popcll(b0) + 2 * __popcll(b1);
        nC += __popcll(bC);
        nP += __popcll(bP);
      }
      if (lane == 0) {
        cnts[0] = nE;
        cnts[1] = nC;
        cnts[2] = min(nP, kMaxSegments);
      }
    }
    __syncthreads();
    const int nE = cnts[0], nC = cnts[1], nP = cnts[2];

    // ---------------- full exact tiles, two stages ----------------
    if (nE > 0) {
      {
        const int kt = __builtin_amdgcn_readfirstlane(w0 * tpb + elist[0]);
        flt_copy<D>(plan, krs, vrs, kt * kTile, flt_vrow(a, kt), stage0, wave_u);
      }
      flt_copies_done_barrier();
      for (int e = 0; e < nE; ++e) {
        uint8_t* cur = (e & 1) ? stage1 : stage0;
        uint8_t* nxt = (e & 1) ? stage0 : stage1;
        if (e + 1 < nE) {   // next tile into the other stage, in flight during the compute
          const int kt = __builtin_amdgcn_readfirstlane(w0 * tpb + elist[e + 1]);
          flt_copy<D>(plan, krs, vrs, kt * kTile, flt_vrow(a, kt), nxt, wave_u);
        }
        flt_tile<D, false>(cur, qf, O, m_run, l_run, c, kTile, klane, vlane, hh);
        flt_copies_done_barrier();
      }
    }
    // ---------------- tiles with the end of a segment's valid keys ----------------
    for (int pi = 0; pi < nP; ++pi) {
      const int kt = __builtin_amdgcn_readfirstlane(plist[pi]), nvalid = pvalid[pi];
      flt_copy<D>(plan, krs, vrs, kt * kTile, flt_vrow(a, kt), stage0, wave_u);
      flt_copies_done_barrier();
      flt_tile<D, true>(stage0, qf, O, m_run, l_run, c, nvalid, klane, vlane, hh);
      __syncthreads();
    }

    // ---------------- centroid columns, 32 at a time ----------------
    const int ncols = nC * a.G;
    for (int c0 = 0; c0 < ncols; c0 += 32) {
      for (int idx = tid; idx < 32 * (D / 4); idx += 256) {
        const int col = idx / (D / 4), c4 = idx % (D / 4);
        const int ent = c0 + col, be = ent / a.G, g = ent % a.G;
        float4 kv = make_float4(0.f, 0.f, 0.f, 0.f), vv = kv;
        float cn = 0.0f;
        if (be < nC) {
          const int j = w0 + clist[be];
          const int64_t ci = (bh * a.nKB + j) * a.G + g;
          cn = a.cnt[ci];
          if (cn > 0.0f) {
            kv = *reinterpret_cast<const float4*>(a.kc + ci * D + c4 * 4);
            vv = *reinterpret_cast<const float4*>(a.vc + ci * D + c4 * 4);
          }
        }
        const float kfv[4] = {kv.x, kv.y, kv.z, kv.w}, vfv[4] = {vv.x, vv.y, vv.z, vv.w};
        v4bf khi, klo, vhi, vlo;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          khi[e2] = (__bf16)kfv[e2];
          klo[e2] = (__bf16)(kfv[e2] - (float)khi[e2]);
          vhi[e2] = (__bf16)vfv[e2];
          vlo[e2] = (__bf16)(vfv[e2] - (float)vhi[e2]);
        }
        *reinterpret_cast<v4bf*>(stage0 + col * L::KSTR + c4 * 8) = khi;
        *reinterpret_cast<v4bf*>(stage0 + L::KCL_OFF + col * L::KSTR + c4 * 8) = klo;
        *reinterpret_cast<v4bf*>(stage1 + col * L::VSTR + c4 * 8) = vhi;
        *reinterpret_cast<v4bf*>(stage1 + L::VCL_OFF + col * L::VSTR + c4 * 8) = vlo;
        if (c4 == 0) bias[col] = cn > 0.0f ? __log2f(cn) : -INFINITY;
      }
      __syncthreads();
      v16f acc = (v16f){};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const int off = klane + s * 32;
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const v8bf*>(stage0 + off), qf[s], acc, 0,
                                                      0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const v8bf*>(stage0 + L::KCL_OFF + off),
                                                      qf[s], acc, 0, 0, 0);
      }
      float x[16];
      float mx = -INFINITY;
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) {
        const int col = (e2 / 4) * 8 + hh * 4 + (e2 % 4);
        x[e2] = __builtin_fmaf(acc[e2], c, bias[col]);
        mx = fmaxf(mx, x[e2]);
      }
      mx = fpair_max(mx);
      frescale<NS>(mx, m_run, l_run, O);
      const float msub = m_run == -INFINITY ? 0.0f : m_run;
      float psum = 0.0f;
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) {
        x[e2] = __builtin_amdgcn_exp2f(x[e2] - msub);
        psum += x[e2];
      }
      l_run += psum;
      const int g16 = lane >> 4, j16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        v8bf pf;
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) pf[e2] = (__bf16)x[ks * 8 + e2];
        const int krow = ks * 16 + hh * 4 + (j16 >> 2);
#pragma unroll
        for (int cb = 0; cb < NS; ++cb) {
          const int col = cb * 32 + (g16 & 1) * 16 + 4 * (j16 & 3);
          const uint8_t* ph = stage1 + krow * L::VSTR + col * 2;
          const uint8_t* pl = stage1 + L::VCL_OFF + krow * L::VSTR + col * 2;
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fcat8(ftr16(ph), ftr16(ph + 8 * L::VSTR)), pf, O[cb], 0, 0,
                                                          0);
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fcat8(ftr16(pl), ftr16(pl + 8 * L::VSTR)), pf, O[cb], 0, 0,
                                                          0);
        }
      }
      __syncthreads();
    }
  }

  // ---------------- finalize ----------------
  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const bool row_ok = qrow < a.lq_valid && l_tot > 0.0f;
  const float inv = row_ok ? 1.0f / l_tot : 0.0f;
#pragma unroll
  for (int cb = 0; cb < NS; ++cb) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch = cb * 32 + gq * 8 + hh * 4;
      const int64_t o = (bh * a.Lq + qrow) * D + ch;
      if (OBF16) {
        v4bf r;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) r[e2] = (__bf16)(O[cb][gq * 4 + e2] * inv);
        *reinterpret_cast<v4bf*>(static_cast<uint16_t*>(a.out) + o) = r;
      } else {
        float4 r = make_float4(O[cb][gq * 4] * inv, O[cb][gq * 4 + 1] * inv, O[cb][gq * 4 + 2] * inv,
                               O[cb][gq * 4 + 3] * inv);
        *reinterpret_cast<float4*>(static_cast<float*>(a.out) + o) = r;
      }
    }
  }
  if (a.lse && hh == 0)
    a.lse[bh * a.Lq + qrow] = row_ok ? (m_run + __log2f(l_tot)) * 0.69314718055994530942f : -INFINITY;
}

template <int D>
static hipError_t launch_fwd_float_d(const FwdFloatArgs& a, hipStream_t st) {
  dim3 grid(a.B * a.H * a.nQB);
  if (a.out_bf16) fwd_float_kernel<D, true><<<grid, 256, 0, st>>>(a);
  else fwd_float_kernel<D, false><<<grid, 256, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd_float(const FwdFloatArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_fwd_float_d<64>(a, st) : launch_fwd_float_d<128>(a, st);
}

}  // namespace sa
