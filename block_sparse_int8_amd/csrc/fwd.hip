// Block-sparse INT8 attention forward (gfx950).
//
// Configure Sol Sparse Attention, "How it works": kept key blocks are computed
// exactly on the INT8 Q/K (the W8A8 integer path), skipped blocks contribute
// their centroids to the same online softmax (Configure H3 Static Virtual KV,
// mode list, "residual").  FlashVSR Sparge Attention, "How it works": one sparse
// call over the whole compact block map.
//
// Mapping onto CDNA4:
//  * One workgroup (4 waves, 256 threads) per 128-row query block; wave w owns
//    query rows 32w..32w+31.  Its INT8 Q fragment stays in registers for the
//    whole kernel.
//  * Exact 64-key tiles: K (int8) and V (bf16) are staged in LDS; S^T = K.Q^T
//    with v_mfma_i32_32x32x32_i8 (two 32-key halves), so each lane ends up
//    holding one query row's scores — the layout the PV product needs as its B
//    operand, with no LDS round trip.  O^T = V^T.P^T with
//    v_mfma_f32_32x32x16_bf16; the V^T operand comes straight from the
//    row-major V tile through ds_read_b64_tr_b16.
//  * Softmax in base 2 with sm_scale*log2(e) folded into the per-tile scale
//    a_i*b_j; the running max is shared by the two lanes (l, l^32) that hold
//    the same query row; row sums stay per lane until the end.
//  * Centroid columns are batched 32 at a time into the same tile shapes, as
//    bf16 hi+lo pairs (about 16 mantissa bits), with log2(count) added to the
//    logit so a centroid weighs as much as the keys it stands for.
//  * The grid walks query blocks XCD by XCD (block id b lands on XCD b % 8), so
//    the query blocks of one head share that XCD's L2 while they stream the same
//    K/V tiles.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

namespace {

constexpr int kWin = 512;   // map entries scanned per list-building window

template <int D>
struct FwdLds {
  static constexpr int KSTR = D + 16;         // int8 K tile row stride (bytes)
  static constexpr int VSTR = 2 * D + 64;     // bf16 V tile row stride (bytes)
  static constexpr int KCSTR = 2 * D + 16;    // bf16 centroid-K row stride (bytes)
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = K_OFF + kTile * KSTR;
  static constexpr int TILE_END = V_OFF + kTile * VSTR;
  static constexpr int KCH_OFF = 0;
  static constexpr int KCL_OFF = KCH_OFF + 32 * KCSTR;
  static constexpr int VCH_OFF = KCL_OFF + 32 * KCSTR;
  static constexpr int VCL_OFF = VCH_OFF + 32 * VSTR;
  static constexpr int CENT_END = VCL_OFF + 32 * VSTR;
  static constexpr int DATA = (TILE_END > CENT_END ? TILE_END : CENT_END);
  static constexpr int BIAS_OFF = DATA;                   // float[32]
  static constexpr int ELIST_OFF = BIAS_OFF + 32 * 4;     // uint16[2*kWin]
  static constexpr int CLIST_OFF = ELIST_OFF + 2 * kWin * 2;  // uint16[kWin]
  static constexpr int CNT_OFF = CLIST_OFF + kWin * 2;    // int[2]
  static constexpr int TOTAL = CNT_OFF + 16;
};

__device__ __forceinline__ v4bf tr16(const uint8_t* lds_byte_ptr) {
  v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((SA_LDS v4s*)(lds_byte_ptr));
  return __builtin_bit_cast(v4bf, r);
}

__device__ __forceinline__ v8bf cat8(v4bf a, v4bf b) {
  return (v8bf){a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// 8 int8 codes (two dwords) -> 8 bf16 (exact: |code| <= 127).
__device__ __forceinline__ v8bf i8x8_to_bf16(int lo, int hi) {
  v8bf r;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    r[e] = (__bf16)(float)(int8_t)((lo >> (8 * e)) & 0xFF);
    r[4 + e] = (__bf16)(float)(int8_t)((hi >> (8 * e)) & 0xFF);
  }
  return r;
}


// Online-softmax update for CNT scores per lane (log2 units).  The two lanes
// l and l^32 hold the same query row, so the tile max is exchanged between
// them; each lane keeps its own partial row sum.  On return x holds the
// unnormalized probabilities exp2(x - m).
template <int CNT, int NS>
__device__ __forceinline__ void softmax_update(float (&x)[CNT], float& m_run, float& l_run, v16f (&O)[NS]) {
  float mloc = -INFINITY;
#pragma unroll
  for (int e = 0; e < CNT; ++e) mloc = fmaxf(mloc, x[e]);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32, 64));
  const float m_new = fmaxf(m_run, mloc);
  const float msub = m_new == -INFINITY ? 0.0f : m_new;
  if (m_new > m_run) {
    const float alpha = __builtin_amdgcn_exp2f(m_run - msub);
    l_run *= alpha;
#pragma unroll
    for (int c = 0; c < NS; ++c) O[c] *= alpha;
    m_run = m_new;
  }
  float lsum = 0.0f;
#pragma unroll
  for (int e = 0; e < CNT; ++e) {
    x[e] = __builtin_amdgcn_exp2f(x[e] - msub);
    lsum += x[e];
  }
  l_run += lsum;
}

}  // namespace

template <int D, bool VI8, bool OBF16>
__global__ __launch_bounds__(256, 2) void fwd_kernel(FwdArgs a) {
  using L = FwdLds<D>;
  constexpr int NS = D / 32;   // int8 k-steps of 32 channels; also 32-channel output blocks
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31, hh = lane >> 5;

  // XCD-aware block order: hardware id b runs on XCD b % 8; give each XCD a
  // contiguous range of (head, query block) work items.
  const int nwg = gridDim.x;
  int bid = blockIdx.x;
  if ((nwg & 7) == 0) bid = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
  const int i = bid % a.nQB;
  const int64_t bh = bid / a.nQB;
  const int nKS = a.Lkv / a.k_scale_rows;
  const int nVS = VI8 ? a.Lv / a.v_scale_rows : 1;
  const int tpb = a.kblock / kTile;   // 64-key tiles per key block

  // Q fragment (B operand of S^T = K.Q^T): lane holds query row n of this
  // wave, channels s*32 + hh*16 .. +15 for each k-step s.
  const int qrow = i * kQBlock + wave * 32 + n;
  v4i qreg[NS];
  {
    const int8_t* qp = a.q + (bh * a.Lq + qrow) * D + hh * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) qreg[s] = *reinterpret_cast<const v4i*>(qp + s * 32);
  }
  const float qc = a.q_scale[bh * a.nQB + i] * a.sm_log2;

  v16f O[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) O[c] = (v16f){};
  float m_run = -INFINITY, l_run = 0.0f;

  uint16_t* elist = reinterpret_cast<uint16_t*>(lds + L::ELIST_OFF);
  uint16_t* clist = reinterpret_cast<uint16_t*>(lds + L::CLIST_OFF);
  int* cnts = reinterpret_cast<int*>(lds + L::CNT_OFF);
  float* bias = reinterpret_cast<float*>(lds + L::BIAS_OFF);
  const uint8_t* mrow = a.map + (bh * a.nQB + i) * a.nKB;

  for (int w0 = 0; w0 < a.nKB; w0 += kWin) {
    const int wend = min(a.nKB, w0 + kWin);
    __syncthreads();
    if (wave == 0) {
      int nE = 0, nC = 0;
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      for (int c0 = w0; c0 < wend; c0 += 64) {
        const int j = c0 + lane;
        const int st = j < wend ? mrow[j] : 0;
        const bool isE = st == 1, isC = st == 2 && a.G > 0;
        const uint64_t bE = __ballot(isE), bC = __ballot(isC);
        if (isE) {
          const int pos = nE + __popcll(bE & lt);
          for (int sub = 0; sub < tpb; ++sub) elist[pos * tpb + sub] = (uint16_t)((j - w0) * tpb + sub);
        }
        if (isC) clist[nC + __popcll(bC & lt)] = (uint16_t)(j - w0);
        nE += __popcll(bE);
        nC += __popcll(bC);
      }
      if (lane == 0) {
        cnts[0] = nE * tpb;
        cnts[1] = nC;
      }
    }
    __syncthreads();
    const int nE = cnts[0], nC = cnts[1];

    // ---------------- exact 64-key tiles ----------------
    for (int e = 0; e < nE; ++e) {
      const int kt = w0 * tpb + elist[e];     // global 64-key tile index
      const int krow0 = kt * kTile;
      int vrow0 = krow0;
      if (a.v_block_src) {
        int pb = a.v_block_src[kt];
        pb = min(max(pb, 0), a.Lv / kTile - 1);
        vrow0 = pb * kTile;
      }
      // stage K (int8) and V (bf16; INT8 V is widened exactly) into LDS
      {
        const int8_t* ks = a.k + (bh * a.Lkv + krow0) * D;
        for (int v = tid; v < kTile * D / 16; v += 256) {
          const int r = v / (D / 16), cc = v % (D / 16);
          *reinterpret_cast<uint4*>(lds + L::K_OFF + r * L::KSTR + cc * 16) =
              *reinterpret_cast<const uint4*>(ks + r * D + cc * 16);
        }
        if (VI8) {
          const int8_t* vs = static_cast<const int8_t*>(a.v) + (bh * a.Lv + vrow0) * D;
          for (int v = tid; v < kTile * D / 16; v += 256) {
            const int r = v / (D / 16), cc = v % (D / 16);
            const v4i raw = *reinterpret_cast<const v4i*>(vs + r * D + cc * 16);
            *reinterpret_cast<v8bf*>(lds + L::V_OFF + r * L::VSTR + cc * 32) = i8x8_to_bf16(raw[0], raw[1]);
            *reinterpret_cast<v8bf*>(lds + L::V_OFF + r * L::VSTR + cc * 32 + 16) = i8x8_to_bf16(raw[2], raw[3]);
          }
        } else {
          const uint16_t* vs = static_cast<const uint16_t*>(a.v) + (bh * a.Lv + vrow0) * D;
          for (int v = tid; v < kTile * D / 8; v += 256) {
            const int r = v / (D / 8), cc = v % (D / 8);
            *reinterpret_cast<uint4*>(lds + L::V_OFF + r * L::VSTR + cc * 16) =
                *reinterpret_cast<const uint4*>(vs + r * D + cc * 8);
          }
        }
      }
      __syncthreads();

      // S^T = K . Q^T  (two 32-key halves)
      v16i acc0 = (v16i){}, acc1 = (v16i){};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const v4i k0 = *reinterpret_cast<const v4i*>(lds + L::K_OFF + n * L::KSTR + s * 32 + hh * 16);
        const v4i k1 = *reinterpret_cast<const v4i*>(lds + L::K_OFF + (32 + n) * L::KSTR + s * 32 + hh * 16);
        acc0 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k0, qreg[s], acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(k1, qreg[s], acc1, 0, 0, 0);
      }
      const float c = qc * a.k_scale[bh * nKS + krow0 / a.k_scale_rows];
      float x[32];
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) {
        x[e2] = (float)acc0[e2] * c;
        x[16 + e2] = (float)acc1[e2] * c;
      }
      if (krow0 + kTile > a.lkv_valid) {
#pragma unroll
        for (int e2 = 0; e2 < 32; ++e2) {
          const int key = krow0 + (e2 / 16) * 32 + ((e2 % 16) / 4) * 8 + hh * 4 + (e2 % 4);
          if (key >= a.lkv_valid) x[e2] = -INFINITY;
        }
      }
      softmax_update<32, NS>(x, m_run, l_run, O);
      float pscale = 1.0f;
      if (VI8) pscale = a.v_scale[bh * nVS + vrow0 / a.v_scale_rows];

      // O^T += V^T . P^T  (four 16-key steps)
      const int g16 = lane >> 4, j16 = lane & 15;
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        v8bf pf;
#pragma unroll
        for (int e2 = 0; e2 < 8; ++e2) pf[e2] = (__bf16)(x[ks * 8 + e2] * pscale);
        const int krow = ks * 16 + hh * 4 + (j16 >> 2);
#pragma unroll
        for (int cb = 0; cb < NS; ++cb) {
          const int col = cb * 32 + (g16 & 1) * 16 + 4 * (j16 & 3);
          const uint8_t* p0 = lds + L::V_OFF + krow * L::VSTR + col * 2;
          const v8bf vf = cat8(tr16(p0), tr16(p0 + 8 * L::VSTR));
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, O[cb], 0, 0, 0);
        }
      }
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
        const float kf[4] = {kv.x, kv.y, kv.z, kv.w}, vf[4] = {vv.x, vv.y, vv.z, vv.w};
        v4bf khi, klo, vhi, vlo;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
          khi[e2] = (__bf16)kf[e2];
          klo[e2] = (__bf16)(kf[e2] - (float)khi[e2]);
          vhi[e2] = (__bf16)vf[e2];
          vlo[e2] = (__bf16)(vf[e2] - (float)vhi[e2]);
        }
        *reinterpret_cast<v4bf*>(lds + L::KCH_OFF + col * L::KCSTR + c4 * 8) = khi;
        *reinterpret_cast<v4bf*>(lds + L::KCL_OFF + col * L::KCSTR + c4 * 8) = klo;
        *reinterpret_cast<v4bf*>(lds + L::VCH_OFF + col * L::VSTR + c4 * 8) = vhi;
        *reinterpret_cast<v4bf*>(lds + L::VCL_OFF + col * L::VSTR + c4 * 8) = vlo;
        if (c4 == 0) bias[col] = cn > 0.0f ? __log2f(cn) : -INFINITY;
      }
      __syncthreads();
      v16f acc = (v16f){};
#pragma unroll
      for (int s = 0; s < NS; ++s) {
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const v8bf qb = i8x8_to_bf16(qreg[s][2 * pp], qreg[s][2 * pp + 1]);
          const int off = n * L::KCSTR + (s * 32 + hh * 16 + pp * 8) * 2;
          const v8bf khi = *reinterpret_cast<const v8bf*>(lds + L::KCH_OFF + off);
          const v8bf klo = *reinterpret_cast<const v8bf*>(lds + L::KCL_OFF + off);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(khi, qb, acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(klo, qb, acc, 0, 0, 0);
        }
      }
      float x[16];
#pragma unroll
      for (int e2 = 0; e2 < 16; ++e2) {
        const int col = (e2 / 4) * 8 + hh * 4 + (e2 % 4);
        x[e2] = acc[e2] * qc + bias[col];
      }
      softmax_update<16, NS>(x, m_run, l_run, O);
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
          const uint8_t* ph = lds + L::VCH_OFF + krow * L::VSTR + col * 2;
          const uint8_t* pl = lds + L::VCL_OFF + krow * L::VSTR + col * 2;
          const v8bf vh = cat8(tr16(ph), tr16(ph + 8 * L::VSTR));
          const v8bf vl = cat8(tr16(pl), tr16(pl + 8 * L::VSTR));
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vh, pf, O[cb], 0, 0, 0);
          O[cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vl, pf, O[cb], 0, 0, 0);
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

template <int D, bool VI8>
static hipError_t launch_fwd_dv(const FwdArgs& a, hipStream_t st) {
  const size_t lds = FwdLds<D>::TOTAL;
  dim3 grid(a.B * a.H * a.nQB);
  if (a.out_bf16) fwd_kernel<D, VI8, true><<<grid, 256, lds, st>>>(a);
  else fwd_kernel<D, VI8, false><<<grid, 256, lds, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_fwd(const FwdArgs& a, hipStream_t st) {
  if (a.d == 64) return a.v_int8 ? launch_fwd_dv<64, true>(a, st) : launch_fwd_dv<64, false>(a, st);
  return a.v_int8 ? launch_fwd_dv<128, true>(a, st) : launch_fwd_dv<128, false>(a, st);
}

}  // namespace sa
