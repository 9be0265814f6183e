// Routing pass (gfx950): block sums, centroids and the block map.
//
// Configure Sol Sparse Attention, "How it works": every 128-token query block
// scores each 64-token key block with a cheap proxy on the same INT8 Q/K the
// exact path uses, and skips a block (replacing it by one 64-token centroid, or
// two 32-token ones) when its score exceeds mean + routing_threshold * std over
// the query block's candidates.  "The inputs that matter": a manually protected
// token prefix stays exact.  FlashVSR Sparge Attention, "How it works": an
// explicit map on logical blocks is converted to the physical block size.
//
// Two launches, reading their inputs once from HBM:
//   pool     — int32 column sums of the INT8 codes of each 128-row query block
//              and of each key block (into the workspace, for the proxy; taken
//              from the quantizer's 32-row chunk sums when the caller passes
//              them, so the codes are not read again) and per-group centroids:
//              kbar = mean of the dequantized keys, vbar = mean of V, count =
//              valid rows
//   decide   — proxy s_ij = (Qsum_i . Ksum_j) * b_j / n_j (exact integer dot on
//              the int8 matrix cores, combined in float64), then the threshold
//              rule (mean and population std over the candidates in float64),
//              the fixed-sparsity rule (top-k by exact radix select), or the
//              explicit-map expansion.
#include "sa_device.h"
#include "sa_launch.h"

#include <mutex>

namespace sa {

// Column sums straight from HBM: a lane owns one dword column (4 int8 codes, or
// 2 bf16 values) of a block and every RG-th row of it; its loads are issued
// before any is used, so each workgroup keeps the whole block in flight, and
// the per-lane partial sums meet in LDS.  All rows of a block lie inside the
// tensor (L is a multiple of the block size); rows past the valid length are
// loaded and multiplied by zero.

// Per-column sums of the 4 int8 codes in a dword, over the rows a lane owns.
// u = w ^ 0x80808080 holds code + 128 (0..255) in each byte; bytes 0 and 2
// accumulate in the 16-bit halves of lo, bytes 1 and 3 in those of hi, with
// plain 32-bit adds (no carry crosses a half: at most 128 rows x 255 < 2^16),
// and 128 per counted row is taken off at the end.  Five vector operations
// per four codes.
struct I8Cols {
  uint32_t lo = 0, hi = 0;
  int n = 0;
  __device__ __forceinline__ void add(uint32_t w, bool valid) {
    const uint32_t u = valid ? (w ^ 0x80808080u) : 0u;
    lo += u & 0x00FF00FFu;
    hi += (u >> 8) & 0x00FF00FFu;
    n += valid ? 1 : 0;
  }
  __device__ __forceinline__ int4 sums() const {
    const int o = 128 * n;
    return make_int4((int)(lo & 0xFFFFu) - o, (int)(hi & 0xFFFFu) - o, (int)(lo >> 16) - o, (int)(hi >> 16) - o);
  }
};

// A column sum x (|x| <= 127 * 128) as two int8 digits, x = 128 * hi + lo with
// lo in [-64, 63] and |hi| <= 127, so the proxy products run on the int8
// matrix cores.
__device__ __forceinline__ void store_digits(int8_t* dst, int d, int col, int32_t x) {
  const int32_t hi = (x + 64) >> 7;
  dst[col] = (int8_t)hi;
  dst[d + col] = (int8_t)(x - 128 * hi);
}

// Query block i: the column sums of its codes over the valid rows, stored as
// two int8 digits.  From the quantizer's 128-row block sums when the caller
// passes them (padding rows are coded 0, so they add nothing), else from the
// codes: a lane owns one dword column (4 codes) and every RG-th row.
template <int D>
__device__ __forceinline__ void pool_q_block(const RouteArgs& a, int i, int h, int b) {
  constexpr int DW = D / 4;              // dwords per row
  constexpr int RG = 256 / DW;           // row groups
  constexpr int NR = kQBlock / RG;       // rows per lane
  __shared__ int32_t part[RG][D];
  const int t = threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  int8_t* dst = a.qdig + (bh * a.nQB + i) * 2 * D;
  if (a.q_sums) {
    for (int col = t; col < D; col += 256) store_digits(dst, D, col, a.q_sums[(bh * a.nQB + i) * D + col]);
    return;
  }
  const int dw = t % DW, rg = t / DW;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(a.q + (bh * a.Lq + (int64_t)i * kQBlock) * D) + dw;
  const int nvalid = min(kQBlock, max(0, a.lq_valid - i * kQBlock));
  uint32_t w[NR];
#pragma unroll
  for (int k = 0; k < NR; ++k) w[k] = src[(rg + RG * k) * DW];
  I8Cols acc;
#pragma unroll
  for (int k = 0; k < NR; ++k) acc.add(w[k], rg + RG * k < nvalid);
  *reinterpret_cast<int4*>(&part[rg][dw * 4]) = acc.sums();
  __syncthreads();
  for (int col = t; col < D; col += 256) {
    int32_t s = 0;
#pragma unroll
    for (int r = 0; r < RG; ++r) s += part[r][col];
    store_digits(dst, D, col, s);
  }
}

// The pooling pass, one launch.  Workgroup x < nKB: key block x of (head y,
// batch z) — its column sums (into the workspace, for the proxy; per 32-row
// chunk so that 2x32 groups, and groups spanning two K scale blocks, combine
// their chunks with the right scale) and its centroids: kbar = mean of the
// dequantized keys, vbar = mean of V, count = valid rows.  Workgroup x >= nKB
// (routing rules only): query block x - nKB (pool_q_block).  With SUMS the key
// sums come from the quantizer's chunk sums and the K codes are not read.
template <int D, bool VI8, int MAXCH, bool SUMS>
__global__ __launch_bounds__(256) void pool_kernel(RouteArgs a) {
  // MAXCH: 32-row chunks per key block (kblock / 32)
  constexpr int KDW = D / 4, KRG = 256 / KDW;   // K: dwords per row, row groups
  constexpr int VDW = VI8 ? D / 4 : D / 2, VRG = 256 / VDW;
  static_assert(32 % KRG == 0 && 32 % VRG == 0, "row groups must divide a chunk");
  if ((int)blockIdx.x >= a.nKB) {                 // uniform over the workgroup
    pool_q_block<D>(a, blockIdx.x - a.nKB, blockIdx.y, blockIdx.z);
    return;
  }
  __shared__ int32_t kpart[SUMS ? 1 : KRG][MAXCH][D];
  __shared__ float vpart[VRG][MAXCH][D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  const int kb = MAXCH * 32, row0 = j * kb, nch = MAXCH;
  const int nKS = a.Lkv / a.k_scale_rows;
  const int nvalid = a.lay.block_rows(j);   // valid rows: a prefix of the block
  if (SUMS) {
    // the chunk sums, 8 columns per lane
    for (int u = t; u < MAXCH * D / 8; u += 256) {
      const int c = u / (D / 8), col0 = (u % (D / 8)) * 8;
      const v8s sv =
          *reinterpret_cast<const v8s*>(a.k_sums + (bh * (a.Lkv / 32) + (int64_t)j * MAXCH + c) * D + col0);
#pragma unroll
      for (int e = 0; e < 8; ++e) kpart[0][c][col0 + e] = sv[e];
    }
  } else {
    // K: lane (dw, rg) sums rows rg, rg + KRG, ... of each chunk
    constexpr int NR = 32 / KRG;
    const int dw = t % KDW, rg = t / KDW;
    const uint32_t* src = reinterpret_cast<const uint32_t*>(a.k + (bh * a.Lkv + row0) * D) + dw;
    uint32_t w[MAXCH][NR];
#pragma unroll
    for (int c = 0; c < MAXCH; ++c)
#pragma unroll
      for (int k = 0; k < NR; ++k) w[c][k] = src[(c * 32 + rg + KRG * k) * KDW];
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      I8Cols acc;
#pragma unroll
      for (int k = 0; k < NR; ++k) acc.add(w[c][k], c * 32 + rg + KRG * k < nvalid);
      *reinterpret_cast<int4*>(&kpart[SUMS ? 0 : rg][c][dw * 4]) = acc.sums();
    }
  }
  // V (centroids only): physical rows through v_block_src, one 64-row block at a time
  if (a.G > 0) {
    constexpr int NR = 32 / VRG;
    const int dw = t % VDW, rg = t / VDW;
    uint32_t w[MAXCH][NR];
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      int prow = row0 + c * 32;   // physical first row of the chunk
      if (a.v_block_src) {
        const int pb = min(max(a.v_block_src[(row0 + c * 32) / 64], 0), a.Lv / 64 - 1);
        prow = pb * 64 + (row0 + c * 32) % 64;
      }
      const uint32_t* src =
          VI8 ? reinterpret_cast<const uint32_t*>(static_cast<const int8_t*>(a.v) + (bh * a.Lv + prow) * D) + dw
              : reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(a.v) + (bh * a.Lv + prow) * D) + dw;
#pragma unroll
      for (int k = 0; k < NR; ++k) w[c][k] = src[(rg + VRG * k) * VDW];
    }
#pragma unroll
    for (int c = 0; c < MAXCH; ++c) {
      if (VI8) {
        I8Cols acc;   // |sum| <= 127*32: exact in float
#pragma unroll
        for (int k = 0; k < NR; ++k) acc.add(w[c][k], c * 32 + rg + VRG * k < nvalid);
        const int4 sm = acc.sums();
        *reinterpret_cast<float4*>(&vpart[rg][c][dw * 4]) = make_float4((float)sm.x, (float)sm.y, (float)sm.z, (float)sm.w);
      } else {
        float acc0 = 0.0f, acc1 = 0.0f;
#pragma unroll
        for (int k = 0; k < NR; ++k) {
          const bool valid = c * 32 + rg + VRG * k < nvalid;
          acc0 += valid ? __uint_as_float(w[c][k] << 16) : 0.0f;
          acc1 += valid ? __uint_as_float(w[c][k] & 0xFFFF0000u) : 0.0f;
        }
        *reinterpret_cast<float2*>(&vpart[rg][c][dw * 2]) = make_float2(acc0, acc1);
      }
    }
  }
  __syncthreads();
  // chunk sums into row 0 of the partial arrays (each element is read and
  // written by the same thread only)
  for (int w = t; w < nch * D; w += 256) {
    const int c = w / D, col = w % D;
    if (!SUMS) {
      int32_t s = 0;
#pragma unroll
      for (int r = 0; r < KRG; ++r) s += kpart[SUMS ? 0 : r][c][col];
      kpart[0][c][col] = s;
    }
    float vsum = 0.0f;
    if (a.G > 0) {
#pragma unroll
      for (int r = 0; r < VRG; ++r) vsum += vpart[r][c][col];
    }
    vpart[0][c][col] = vsum;
  }
  __syncthreads();
  if (a.kdig) {
    for (int col = t; col < D; col += 256) {
      int32_t s = 0;
      for (int c = 0; c < nch; ++c) s += kpart[0][c][col];
      store_digits(a.kdig + ((int64_t)bh * a.nKB + j) * 2 * D, D, col, s);
    }
  }
  if (a.G > 0) {
    const int gr = kb / a.G, cpg = gr / 32 > 0 ? gr / 32 : 1;
    for (int w = t; w < a.G * D; w += 256) {
      const int g = w / D, col = w % D;
      const int n = min(gr, max(0, nvalid - g * gr));
      float ksum = 0.0f, vsum = 0.0f;
      for (int c = g * cpg; c < (g + 1) * cpg && c < nch; ++c) {
        const int crow = row0 + c * 32;
        ksum += a.k_scale[bh * nKS + crow / a.k_scale_rows] * (float)kpart[0][c][col];
        if (VI8) {
          int pr = crow;
          if (a.v_block_src) {
            int pb = min(max(a.v_block_src[crow / 64], 0), a.Lv / 64 - 1);
            pr = pb * 64 + crow % 64;
          }
          vsum += a.v_scale[bh * (a.Lv / a.v_scale_rows) + pr / a.v_scale_rows] * vpart[0][c][col];
        } else {
          vsum += vpart[0][c][col];
        }
      }
      const int64_t o = ((bh * a.nKB + j) * a.G + g);
      a.kc[o * D + col] = n > 0 ? ksum / (float)n : 0.0f;
      a.vc[o * D + col] = n > 0 ? vsum / (float)n : 0.0f;
      if (col == 0) a.cnt[o] = (float)n;
    }
  }
}

// Proxies for 32 query blocks of one (head, batch) against 32-block column
// tiles of key blocks, on the int8 matrix cores.  The proxy numerator
// D_ij = Qsum_i . Ksum_j is exact: with x = 128*hi + lo for both sums,
//   D = 2^14 * sum(hq*hk) + 2^7 * sum(hq*lk + lq*hk) + sum(lq*lk),
// three v_mfma_i32_32x32x32_i8 products (the middle one over 2d), each partial
// sum below 2^22 in int32, combined exactly in float64.  s_ij = (D * b_j) / n_j
// in float64, rounded after the product and after the quotient, so it is the
// same float64 value whatever evaluates it in that order.  A 32x32 tile costs
// 16 MFMAs, so the decision kernels recompute
// s on every pass over the key blocks instead of storing it.
//
// Lane (n, hf) of a tile holds s[r][j] for rows r = (e/4)*8 + hf*4 + e%4
// (e < 16) and column j = n.
template <int D>
struct ProxyTiles {
  static constexpr int NS = D / 32;   // 32-channel MFMA k-steps
  struct KOps {
    v4i h[NS], l[NS];
  };
  v4i qh[NS], ql[NS];   // A operands: digit rows of query block i0 + n (zero past the last block)
  int64_t bh;
  int n, hf, kb, nKS;

  __device__ __forceinline__ ProxyTiles(const RouteArgs& a, int64_t bh_, int i0, int lane)
      : bh(bh_), n(lane & 31), hf(lane >> 5), kb(a.kblock), nKS(a.Lkv / a.k_scale_rows) {
    const bool ok = i0 + n < a.nQB;
    const int8_t* qr = a.qdig + (bh * a.nQB + (ok ? i0 + n : 0)) * 2 * D + hf * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      qh[s] = ok ? *reinterpret_cast<const v4i*>(qr + s * 32) : (v4i){0, 0, 0, 0};
      ql[s] = ok ? *reinterpret_cast<const v4i*>(qr + D + s * 32) : (v4i){0, 0, 0, 0};
    }
  }
  // key digits of column tile tt (lane: key block tt*32 + n, channels hf*16..)
  __device__ __forceinline__ void load_k(const RouteArgs& a, int tt, KOps& k) const {
    const int j = tt * 32 + n;
    const int8_t* kr = a.kdig + (bh * a.nKB + (j < a.nKB ? j : 0)) * 2 * D + hf * 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      k.h[s] = *reinterpret_cast<const v4i*>(kr + s * 32);
      k.l[s] = *reinterpret_cast<const v4i*>(kr + D + s * 32);
    }
  }
  // s for column tile tt (column n of this lane)
  __device__ __forceinline__ void tile(const RouteArgs& a, int tt, const KOps& k, double (&sv)[16]) const {
    const int j = tt * 32 + n;
    v16i p1 = (v16i){}, p2 = (v16i){}, p3 = (v16i){};
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      p1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qh[s], k.h[s], p1, 0, 0, 0);
      p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(qh[s], k.l[s], p2, 0, 0, 0);
      p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ql[s], k.h[s], p2, 0, 0, 0);
      p3 = __builtin_amdgcn_mfma_i32_32x32x32_i8(ql[s], k.l[s], p3, 0, 0, 0);
    }
    const int nj = j < a.nKB ? a.lay.block_rows(j) : 0;
    const double bj = nj > 0 ? (double)a.k_scale[bh * nKS + j] : 0.0, nd = nj > 0 ? (double)nj : 1.0;
    // D is an exact integer in float64; then one rounding for the product
    // and one for the quotient, in that order.  A full block has a power of
    // two rows, and dividing by a power of two only shifts the exponent, so
    // there round(D*b)/n = D*(b/n) exactly: one multiply.  Other blocks (the
    // last one of a segment) divide.
#pragma unroll
    for (int e = 0; e < 16; ++e) sv[e] = 16384.0 * (double)p1[e] + 128.0 * (double)p2[e] + (double)p3[e];
    if ((nj & (nj - 1)) == 0) {
      const double cj = bj / nd;   // exact
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[e] *= cj;
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) sv[e] = (sv[e] * bj) / nd;
    }
  }
  __device__ __forceinline__ int row_of(int e) const { return (e / 4) * 8 + hf * 4 + (e % 4); }
};

// Work item of a decision workgroup: (chunk of R query blocks, head, batch)
// from a 1-D grid of chunks * H * B.  Hardware workgroup id w runs on XCD
// w % 8; each XCD is given a contiguous range of work items, so the chunks of
// one head, which all read that head's key-block sums, share one L2.
struct DecideItem {
  int i0, h, b;
  __device__ __forceinline__ DecideItem(const RouteArgs& a, int R = 32) {
    const int nwg = gridDim.x, nch = (a.nQB + R - 1) / R;
    int w = blockIdx.x;
    if ((nwg & 7) == 0) w = (blockIdx.x & 7) * (nwg >> 3) + (blockIdx.x >> 3);
    i0 = (w % nch) * R;
    h = (w / nch) % a.H;
    b = w / (nch * a.H);
  }
};

// Class of key block j in the key layout: 0 without valid rows (dropped),
// 1 dense (always exact), 2 a routing candidate.
__host__ __device__ __forceinline__ int block_class(const KvLayout& lay, int j) {
  if (lay.block_rows(j) == 0) return 0;
  return lay.block_routed(j) ? 2 : 1;
}

// Routing candidates: the key blocks with a valid row in routed segments.  They
// lie in [jc0, jc1) (N of them; the range may hold other blocks between
// routed segments).
struct CandRange {
  int jc0, jc1, N;
  const KvLayout* lay;
  __host__ __device__ __forceinline__ explicit CandRange(const RouteArgs& a) : jc0(0), jc1(0), N(0), lay(&a.lay) {
    const int kb = a.lay.kblock;
    bool any = false;
    for (int x = 0; x < a.lay.n; ++x) {
      if (!((a.lay.routed >> x) & 1u) || a.lay.end[x] <= a.lay.start[x]) continue;
      const int b0 = a.lay.start[x] / kb, b1 = min(a.nKB, (a.lay.end[x] + kb - 1) / kb);
      if (b1 <= b0) continue;
      jc0 = any ? min(jc0, b0) : b0;
      jc1 = any ? max(jc1, b1) : b1;
      N += b1 - b0;
      any = true;
    }
  }
  __device__ __forceinline__ bool has(int j) const { return j >= jc0 && j < jc1 && block_class(*lay, j) == 2; }
};

// Sol decisions (threshold rule) for 32 query blocks of one (head, batch): three
// passes over the key blocks, the mean, the population variance about it, then
// the decisions.
// Each wave takes every NW-th 32-block column tile.
constexpr int kDecideWaves = 4;

template <int D>
__global__ __launch_bounds__(64 * kDecideWaves) void decide_sol_kernel(RouteArgs a) {
  constexpr int NW = kDecideWaves;
  using PT = ProxyTiles<D>;
  __shared__ double red[NW][32];
  __shared__ double colsum[NW][32][33];   // per wave: [row][column lane], padded
  __shared__ double mu_s[32], thr_s[32];
  __shared__ int keep_s[32];
  const DecideItem wi(a);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t bh = (int64_t)wi.b * a.H + wi.h;
  const int i0 = wi.i0;
  const PT pt(a, bh, i0, lane);
  const int n = pt.n;
  const CandRange cr(a);
  const int N = cr.N;
  const int t0 = cr.jc0 / 32, t1 = (cr.jc1 + 31) / 32;   // column tiles touching the candidates
  // per-row sum over the candidate columns of f(s, row), reduced over the workgroup into red[0][row]
  auto row_sum = [&](auto f) __attribute__((always_inline)) {
    double acc[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] = 0.0;
    typename PT::KOps kn;
    if (t0 + wave < t1) pt.load_k(a, t0 + wave, kn);
    for (int tt = t0 + wave; tt < t1; tt += NW) {
      const typename PT::KOps kc = kn;
      if (tt + NW < t1) pt.load_k(a, tt + NW, kn);   // next tile's operands in flight
      double sv[16];
      pt.tile(a, tt, kc, sv);
      const bool cand = cr.has(tt * 32 + n);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] += cand ? f(sv[e], pt.row_of(e)) : 0.0;
    }
    // over the 32 columns held by lanes with the same hf: through LDS
#pragma unroll
    for (int e = 0; e < 16; ++e) colsum[wave][pt.row_of(e)][n] = acc[e];
    __syncthreads();
    if (lane < 32) {
      double sum = 0.0;
#pragma unroll
      for (int c = 0; c < 32; ++c) sum += colsum[wave][lane][c];
      red[wave][lane] = sum;
    }
    __syncthreads();
    if (t < 32) {
      double sum = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) sum += red[w][t];
      red[0][t] = sum;
    }
    __syncthreads();
  };
  row_sum([](double s, int) { return s; });
  if (t < 32) mu_s[t] = N > 0 ? red[0][t] / N : __builtin_nan("");
  __syncthreads();
  row_sum([&](double s, int r) { const double dl = s - mu_s[r]; return dl * dl; });
  const double tau = (double)a.tau;
  if (t < 32) {
    const double mu = mu_s[t];
    const double sigma = N > 0 ? sqrt(red[0][t] / N) : __builtin_nan("");
    const bool keep_all = N == 0 || (tau > 0 && __builtin_isinf(tau)) || sigma == 0.0;
    keep_s[t] = keep_all ? 1 : 0;
    thr_s[t] = keep_all ? 0.0 : mu + tau * sigma;
    if (a.stats && i0 + t < a.nQB) {
      a.stats[(bh * a.nQB + i0 + t) * 2] = mu;
      a.stats[(bh * a.nQB + i0 + t) * 2 + 1] = sigma;
    }
  }
  __syncthreads();
  // decisions for every key block: DROP past the valid keys, EXACT in the
  // prefix, CENTROID for candidates above the threshold
  const int nt = (a.nKB + 31) / 32;
  for (int tt = wave; tt < nt; tt += NW) {
    const int j = tt * 32 + n;
    double sv[16];
    const bool any_cand = tt * 32 + 31 >= cr.jc0 && tt * 32 < cr.jc1;
    if (any_cand) {
      typename PT::KOps kc;
      pt.load_k(a, tt, kc);
      pt.tile(a, tt, kc, sv);
    }
    const int cls = j < a.nKB ? block_class(a.lay, j) : 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = pt.row_of(e), i = i0 + r;
      if (i >= a.nQB || j >= a.nKB) continue;
      const uint8_t st = cls < 2 ? (uint8_t)cls : ((!keep_s[r] && sv[e] > thr_s[r]) ? 2 : 1);
      a.map[(bh * a.nQB + i) * a.nKB + j] = st;
    }
  }
}

// Fixed-sparsity decisions (Ref2VA VSA, two-stage attention patch: top-k
// pruning of the video key tiles at a set sparsity) for 32 query blocks of one
// (head, batch).  With N candidates, each query block keeps the
// keep = N - floor(sparsity * N) candidates of largest proxy; the rest become
// centroids (G > 0) or are dropped (G = 0).
//
// Selection is an exact radix select on a 96-bit key per candidate: the
// float64 proxy mapped to an order-preserving uint64 (with -0 taken as +0),
// then the complement of the block index, so equal proxies rank the lower
// index first and no two keys are equal.  Pass p histograms digit p (8 bits,
// most significant first) of the keys that match the boundary prefix found so
// far, 256 bins per query block in LDS; the bin holding the keep-th largest key
// extends the prefix.  A query block is settled once that bin is kept whole
// (at pass 12 at the latest, when the bin holds a single key); its kept
// candidates are then exactly those whose key prefix is >= the boundary
// prefix.  Proxies are recomputed on every pass.
__device__ __forceinline__ uint64_t order_key(double s) {
  const uint64_t u = (uint64_t)__double_as_longlong(s + 0.0);   // -0 + 0 = +0
  return (u >> 63) ? ~u : (u | 0x8000000000000000ull);
}

// First p digits (8 bits each) of the key (hi, lo) as integers: the top
// min(p, 8) digits of hi, the top p - 8 digits of lo.
__device__ __forceinline__ uint64_t key_hi_prefix(uint64_t hi, int p) {
  return p == 0 ? 0ull : (p >= 8 ? hi : hi >> (64 - 8 * p));
}
__device__ __forceinline__ uint32_t key_lo_prefix(uint32_t lo, int p) {
  return p <= 8 ? 0u : (p >= 12 ? lo : lo >> (32 - 8 * (p - 8)));
}
__device__ __forceinline__ uint32_t key_digit(uint64_t hi, uint32_t lo, int p) {
  return p < 8 ? (uint32_t)(hi >> (56 - 8 * p)) & 255u : (lo >> (24 - 8 * (p - 8))) & 255u;
}

template <int D>
__global__ __launch_bounds__(64 * kDecideWaves) void decide_topk_kernel(RouteArgs a) {
  constexpr int NW = kDecideWaves;
  constexpr int kDigits = 12;
  using PT = ProxyTiles<D>;
  __shared__ uint32_t hist[32][256];
  __shared__ uint64_t phi_s[32];   // boundary prefix: digits from the proxy
  __shared__ uint32_t plo_s[32];   // boundary prefix: digits from the block index
  __shared__ int dig_s[32];        // digits in the prefix
  __shared__ int krem_s[32];       // kept keys still to place inside the prefix's bin
  __shared__ int done_s[32];
  const DecideItem wi(a);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t bh = (int64_t)wi.b * a.H + wi.h;
  const int i0 = wi.i0;
  const PT pt(a, bh, i0, lane);
  const int n = pt.n;
  const CandRange cr(a);
  const int N = cr.N;
  const int keep = N - (int)floor((double)a.sparsity * (double)N);
  const uint8_t pruned = a.G > 0 ? 2 : 0;
  const bool select = keep > 0 && keep < N;
  if (t < 32) {
    phi_s[t] = 0;
    plo_s[t] = 0;
    dig_s[t] = 0;
    krem_s[t] = keep;
    done_s[t] = (!select || i0 + t >= a.nQB) ? 1 : 0;
    if (a.stats && i0 + t < a.nQB) {
      a.stats[(bh * a.nQB + i0 + t) * 2] = __builtin_nan("");
      a.stats[(bh * a.nQB + i0 + t) * 2 + 1] = __builtin_nan("");
    }
  }
  const int t0 = cr.jc0 / 32, t1 = (cr.jc1 + 31) / 32;
  if (select) {
    for (int p = 0; p < kDigits; ++p) {
      for (int x = t; x < 32 * 256; x += 256) (&hist[0][0])[x] = 0u;
      __syncthreads();   // cleared bins and the previous pass's prefixes are visible
      int active = 0;
#pragma unroll
      for (int r = 0; r < 32; ++r) active += done_s[r] ? 0 : 1;
      if (active == 0) break;   // same value in every thread
      typename PT::KOps kn;
      if (t0 + wave < t1) pt.load_k(a, t0 + wave, kn);
      for (int tt = t0 + wave; tt < t1; tt += NW) {
        const typename PT::KOps kc = kn;
        if (tt + NW < t1) pt.load_k(a, tt + NW, kn);
        double sv[16];
        pt.tile(a, tt, kc, sv);
        const int j = tt * 32 + n;
        if (!cr.has(j)) continue;
        const uint32_t lo = ~(uint32_t)j;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int r = pt.row_of(e);
          if (done_s[r]) continue;
          const uint64_t hi = order_key(sv[e]);
          if (key_hi_prefix(hi, p) != phi_s[r] || key_lo_prefix(lo, p) != plo_s[r]) continue;
          atomicAdd(&hist[r][key_digit(hi, lo, p)], 1u);
        }
      }
      __syncthreads();
      // boundary bin per unsettled query block: wave w scans rows 8w..8w+7,
      // lane l holding bins 255-4l .. 252-4l (largest digits first)
      for (int r = wave * 8; r < wave * 8 + 8; ++r) {
        if (done_s[r]) continue;
        uint32_t c4[4];
        uint32_t own = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c4[q] = hist[r][255 - 4 * lane - q];
          own += c4[q];
        }
        uint32_t incl = own;   // inclusive prefix over lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_up(incl, off);
          incl += lane >= off ? o : 0u;
        }
        const uint32_t k = (uint32_t)krem_s[r];
        uint32_t above = incl - own;
        if (above < k && k <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (above + c4[q] >= k) {
              const uint32_t dgt = 255u - 4u * lane - q, kr = k - above;
              if (p < 8) phi_s[r] = (phi_s[r] << 8) | dgt;
              else plo_s[r] = (plo_s[r] << 8) | dgt;
              dig_s[r] = p + 1;
              krem_s[r] = (int)kr;
              done_s[r] = c4[q] == kr ? 1 : 0;
              break;
            }
            above += c4[q];
          }
        }
      }
      __syncthreads();
    }
  }
  __syncthreads();
  // decisions for every key block
  const int nt = (a.nKB + 31) / 32;
  for (int tt = wave; tt < nt; tt += NW) {
    const int j = tt * 32 + n;
    double sv[16];
    const bool any_cand = select && tt * 32 + 31 >= cr.jc0 && tt * 32 < cr.jc1;
    if (any_cand) {
      typename PT::KOps kc;
      pt.load_k(a, tt, kc);
      pt.tile(a, tt, kc, sv);
    }
    const uint32_t lo = ~(uint32_t)j;
    const int cls = j < a.nKB ? block_class(a.lay, j) : 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int r = pt.row_of(e), i = i0 + r;
      if (i >= a.nQB || j >= a.nKB) continue;
      uint8_t st;
      if (cls < 2) st = (uint8_t)cls;
      else if (!select) st = keep > 0 ? 1 : pruned;
      else {
        const int pd = dig_s[r];
        const uint64_t hi = order_key(sv[e]), hp = key_hi_prefix(hi, pd);
        const bool ge = pd <= 8 ? hp >= phi_s[r]
                                : (hp > phi_s[r] || (hp == phi_s[r] && key_lo_prefix(lo, pd) >= plo_s[r]));
        st = ge ? 1 : pruned;
      }
      a.map[(bh * a.nQB + i) * a.nKB + j] = st;
    }
  }
}

// ---------------------------------------------------------------------------
// Decisions with the proxies held in LDS.  When a query block has at most
// kLdsCand candidates, one pass of matrix-core tiles writes s_ij for the R
// query blocks of a workgroup into an R x kLdsCand float64 array, and every
// later pass reads it from there (slot j - jc0; NaN for slots that hold no
// candidate).  The rules and their arithmetic are those of the kernels above;
// only where s lives changes (and the summation order of the mean and
// variance).  R = 32 (128 KiB, one workgroup per CU) or R = 16 (64 KiB, two
// per CU; the 32-row proxy tiles then keep only their first 16 rows), picked
// at launch (see launch_route_d).
// ---------------------------------------------------------------------------
constexpr int kLdsCand = 512;
constexpr int kLdsWaves = 8;

template <int D, int NW, int R>
__device__ __forceinline__ void proxies_to_lds(const RouteArgs& a, const ProxyTiles<D>& pt, const CandRange& cr,
                                               int wave, double (*sv_s)[kLdsCand]) {
  // at most kLdsCand / 32 + 1 column tiles, so at most MT per wave: all of a
  // wave's key operands are loaded before the first product
  constexpr int MT = (kLdsCand / 32 + 1 + NW - 1) / NW;
  const int t0 = cr.jc0 / 32, t1 = (cr.jc1 + 31) / 32;
  typename ProxyTiles<D>::KOps ko[MT];
#pragma unroll
  for (int u = 0; u < MT; ++u)
    if (t0 + wave + u * NW < t1) pt.load_k(a, t0 + wave + u * NW, ko[u]);
#pragma unroll
  for (int u = 0; u < MT; ++u) {
    const int tt = t0 + wave + u * NW;
    if (tt >= t1) break;
    double sv[16];
    pt.tile(a, tt, ko[u], sv);
    const int j = tt * 32 + pt.n;
    if (j < cr.jc0 || j >= cr.jc1) continue;
    const bool cand = cr.has(j);
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (R == 32 || pt.row_of(e) < R) sv_s[pt.row_of(e)][j - cr.jc0] = cand ? sv[e] : __builtin_nan("");
  }
  // slots past the candidate range hold NaN too, so later passes read every slot
  const int span = cr.jc1 - cr.jc0;
  for (int x = threadIdx.x; x < R * kLdsCand; x += 64 * NW) {
    const int r = x / kLdsCand, c = x % kLdsCand;
    if (c >= span) sv_s[r][c] = __builtin_nan("");
  }
}

// Classes of all key blocks (block_class) in LDS, filled once per workgroup.
constexpr int kMaxRouteKB = 6144;   // key blocks per row accepted by the routing rules

__device__ __forceinline__ void fill_classes(const RouteArgs& a, int nt, uint8_t* cls_s) {
  for (int j = threadIdx.x; j < a.nKB; j += nt) cls_s[j] = (uint8_t)block_class(a.lay, j);
}

// Block states of the workgroup's query blocks: DROP for key blocks without
// valid rows, EXACT for dense ones, cand_state(r, j - jc0) for candidates.  A
// thread owns groups of four consecutive key blocks of one row and writes the
// four states with one store when the row allows it.
template <int R, typename F>
__device__ __forceinline__ void write_map_rows(const RouteArgs& a, int64_t bh, int i0, const CandRange& cr, int nt,
                                               const uint8_t* cls_s, F cand_state) {
  const int ng = (a.nKB + 3) / 4, rows = min(R, a.nQB - i0);
  const bool wide = (a.nKB & 3) == 0 && (reinterpret_cast<uintptr_t>(a.map) & 3) == 0;   // 4-byte aligned rows
  for (int x = threadIdx.x; x < ng * rows; x += nt) {
    const int r = x / ng, j0 = (x % ng) * 4;
    uint8_t* mrow = a.map + (bh * a.nQB + i0 + r) * a.nKB;
    // four classes at once (cls_s has room past nKB; entries there are unused)
    const uint32_t cl4 = *reinterpret_cast<const uint32_t*>(cls_s + j0);
    uint32_t packed = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t cls = (cl4 >> (8 * q)) & 255u;
      const int c = min(max(j0 + q - cr.jc0, 0), kLdsCand - 1);   // any slot when not a candidate
      const uint32_t cs = cand_state(r, c);
      packed |= (cls < 2 ? cls : cs) << (8 * q);
    }
    if (wide) {
      *reinterpret_cast<uint32_t*>(mrow + j0) = packed;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        if (j0 + q < a.nKB) mrow[j0 + q] = (uint8_t)(packed >> (8 * q));
    }
  }
}

template <int D, int NW, int R>
__global__ __launch_bounds__(64 * NW) void decide_sol_lds_kernel(RouteArgs a) {
  constexpr int NT = 64 * NW, TPR = NT / R;   // threads per query-block row
  static_assert(TPR <= 64 && (kLdsCand / TPR) % 8 == 0, "row groups inside a wave, slots in batches of 8");
  __shared__ double sv_s[R][kLdsCand];
  __shared__ double thr_s[R];
  __shared__ int keep_s[R];
  __shared__ __attribute__((aligned(4))) uint8_t cls_s[kMaxRouteKB + 4];
  const DecideItem wi(a, R);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t bh = (int64_t)wi.b * a.H + wi.h;
  const int i0 = wi.i0;
  const ProxyTiles<D> pt(a, bh, i0, lane);
  const CandRange cr(a);
  const int N = cr.N;
  proxies_to_lds<D, NW, R>(a, pt, cr, wave, sv_s);
  fill_classes(a, NT, cls_s);
  __syncthreads();
  // row r's mean and population variance: TPR adjacent lanes per row
  const int r = t / TPR, part = t % TPR;
  // kLdsCand / TPR slots per thread, read in batches of 8 into independent sums
  constexpr int PER = kLdsCand / TPR;
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int c0 = 0; c0 < PER; c0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double v = sv_s[r][part + (c0 + u) * TPR];
      acc[u] += __builtin_isnan(v) ? 0.0 : v;
    }
  }
  double sum = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) sum += __shfl_xor(sum, o, 64);
  const double mu = N > 0 ? sum / N : __builtin_nan("");
#pragma unroll
  for (int u = 0; u < 8; ++u) acc[u] = 0.0;
#pragma unroll
  for (int c0 = 0; c0 < PER; c0 += 8) {
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const double v = sv_s[r][part + (c0 + u) * TPR];
      const double dl = v - mu;
      acc[u] += __builtin_isnan(v) ? 0.0 : dl * dl;
    }
  }
  double acc2 = ((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]));
#pragma unroll
  for (int o = TPR / 2; o >= 1; o >>= 1) acc2 += __shfl_xor(acc2, o, 64);
  if (part == 0) {
    const double tau = (double)a.tau;
    const double sigma = N > 0 ? sqrt(acc2 / N) : __builtin_nan("");
    const bool keep_all = N == 0 || (tau > 0 && __builtin_isinf(tau)) || sigma == 0.0;
    keep_s[r] = keep_all ? 1 : 0;
    thr_s[r] = keep_all ? 0.0 : mu + tau * sigma;
    if (a.stats && i0 + r < a.nQB) {
      a.stats[(bh * a.nQB + i0 + r) * 2] = mu;
      a.stats[(bh * a.nQB + i0 + r) * 2 + 1] = sigma;
    }
  }
  __syncthreads();
  write_map_rows<R>(a, bh, i0, cr, NT, cls_s, [&](int rr, int c) -> uint32_t {
    return 1u + ((uint32_t)(keep_s[rr] == 0) & (uint32_t)(sv_s[rr][c] > thr_s[rr]));
  });
}

// Fixed-sparsity decisions with LDS-resident proxies.  The keep-th largest
// 96-bit key of a query block (the same keys as decide_topk_kernel) is found
// bit by bit inside one wave: lane l holds candidates l, l+64, ... of the row
// in registers, and each step counts the keys that match the prefix so far
// and have a 1 in the next bit.  If at least `remaining` do, the bit is 1;
// otherwise it is 0 and those keys are all kept.  The row is settled when
// every key matching the prefix is kept (at bit 96 at the latest, where one
// key matches).  Which of its candidates still match the prefix is one byte
// per lane in a vector register, and a step's count is the lane's popcount
// summed over the wave with one ballot per bit of it: the scalar unit, shared
// by the CU's waves, issues a few instructions per step.  No atomics and no
// barriers.
template <int D, int NW, int R>
__global__ __launch_bounds__(64 * NW) void decide_topk_lds_kernel(RouteArgs a) {
  constexpr int NT = 64 * NW;
  constexpr int NV = kLdsCand / 64;   // candidates per lane
  __shared__ double sv_s[R][kLdsCand];
  __shared__ uint64_t phi_s[R];
  __shared__ uint32_t plo_s[R];
  __shared__ int nb_s[R];
  __shared__ __attribute__((aligned(4))) uint8_t cls_s[kMaxRouteKB + 4];
  const DecideItem wi(a, R);
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t bh = (int64_t)wi.b * a.H + wi.h;
  const int i0 = wi.i0;
  const CandRange cr(a);
  const int N = cr.N, span = cr.jc1 - cr.jc0;
  const int keep = N - (int)floor((double)a.sparsity * (double)N);
  const uint8_t pruned = a.G > 0 ? 2 : 0;
  const bool select = keep > 0 && keep < N;
  if (t < R && a.stats && i0 + t < a.nQB) {
    a.stats[(bh * a.nQB + i0 + t) * 2] = __builtin_nan("");
    a.stats[(bh * a.nQB + i0 + t) * 2 + 1] = __builtin_nan("");
  }
  fill_classes(a, NT, cls_s);
  if (select) {
    const ProxyTiles<D> pt(a, bh, i0, lane);
    proxies_to_lds<D, NW, R>(a, pt, cr, wave, sv_s);
    __syncthreads();
    for (int r = wave; r < R; r += NW) {
      if (i0 + r >= a.nQB) break;
      // the key of each register in three 32-bit words, most significant first;
      // bit k of live: candidate k of this lane still matches the prefix
      static_assert(NV <= 8, "the per-lane count must fit four bits");
      uint32_t w0[NV], w1[NV], w2[NV];
      uint32_t live = 0;
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int c = lane + 64 * k;
        const double v = c < span ? sv_s[r][c] : __builtin_nan("");
        const bool cand = !__builtin_isnan(v);
        const uint64_t hk = cand ? order_key(v) : 0ull;
        w0[k] = (uint32_t)(hk >> 32);
        w1[k] = (uint32_t)hk;
        w2[k] = ~(uint32_t)(cr.jc0 + c);
        live |= cand ? 1u << k : 0u;
      }
      int m = N, rem = keep, nb = 0;
      uint64_t ph = 0;
      uint32_t pl = 0;
      // one bit per step, bit 31 - step of the word
      auto phase = [&](const uint32_t (&w)[NV]) __attribute__((always_inline)) {
        for (int step = 0; step < 32 && m != rem; ++step, ++nb) {
          uint32_t plane = 0;   // bit k: the step's bit of candidate k
#pragma unroll
          for (int k = 0; k < NV; ++k) plane |= ((w[k] >> (31 - step)) & 1u) << k;
          const uint32_t ones = live & plane;
          const uint32_t cnt = __builtin_popcount(ones);   // 0 .. NV
          int c1 = 0;
#pragma unroll
          for (int bit = 0; bit < 4; ++bit) c1 += __popcll(__ballot((cnt >> bit) & 1u)) << bit;
          const bool one = c1 >= rem;
          if (one) {
            m = c1;
          } else {
            rem -= c1;
            m -= c1;
          }
          live = one ? ones : live & ~plane;
          if (nb < 64) ph = (ph << 1) | (one ? 1ull : 0ull);
          else pl = (pl << 1) | (one ? 1u : 0u);
        }
      };
      phase(w0);
      phase(w1);
      phase(w2);
      if (lane == 0) {
        phi_s[r] = ph;
        plo_s[r] = pl;
        nb_s[r] = nb;
      }
    }
  }
  __syncthreads();
  // kept iff the key's first nb bits are >= the boundary prefix
  write_map_rows<R>(a, bh, i0, cr, NT, cls_s, [&](int r, int c) -> uint32_t {
    if (!select) return keep > 0 ? 1u : (uint32_t)pruned;   // uniform
    const int nb = nb_s[r];
    const uint64_t hi = order_key(sv_s[r][c]), ph = phi_s[r];
    const uint32_t lo = ~(uint32_t)(cr.jc0 + c);
    const uint64_t hp = nb == 0 ? 0ull : hi >> (64 - min(nb, 64));
    const uint32_t lp = nb <= 64 ? 0u : (nb == 96 ? lo : lo >> (96 - nb));
    const bool ge = nb <= 64 ? hp >= ph : ((hi > ph) | ((hi == ph) & (lp >= plo_s[r])));
    return ge ? 1u : (uint32_t)pruned;
  });
}

__global__ __launch_bounds__(256) void decide_explicit_kernel(RouteArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  const int nMB = a.Lkv / a.map_kblock;
  const uint8_t* erow = a.explicit_map + (bh * a.nQB + i) * nMB;
  uint8_t* mrow = a.map + (bh * a.nQB + i) * a.nKB;
  for (int j = t; j < a.nKB; j += 256) {
    int st = erow[(int64_t)j * a.kblock / a.map_kblock];
    if (st > 2 || (st == 2 && a.G == 0)) st = 1;
    const int cls = block_class(a.lay, j);
    if (cls == 1) st = 1;
    if (cls == 0) st = 0;
    mrow[j] = (uint8_t)st;
  }
  if (a.stats && t == 0) {
    a.stats[(bh * a.nQB + i) * 2] = __builtin_nan("");
    a.stats[(bh * a.nQB + i) * 2 + 1] = __builtin_nan("");
  }
}

// ---------------------------------------------------------------------------
// Library-owned route workspace (sparse_attn_route_noalloc), for callers that
// cannot allocate device memory.  Every device the library runs on holds its
// own copy until the process ends.  In host code the array's name is not a
// device address: the address comes from hipGetSymbolAddress, once per device
// with that device current, and only that address is handed to the kernels.
// ---------------------------------------------------------------------------
__device__ __align__(256) uint8_t scratch[kRouteScratchBytes];

namespace {
constexpr int kScratchDevices = 64;
void* g_scratch[kScratchDevices] = {};
std::mutex g_scratch_mu;
}  // namespace

hipError_t route_scratch(int dev, void** ptr) {
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

size_t route_workspace_bytes(int B, int H, int nQB, int nKB, int d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)B * H * nQB * 2 * d) + al((size_t)B * H * nKB * 2 * d);
}

template <int D>
static hipError_t launch_route_d(const RouteArgs& a, hipStream_t st) {
  const bool sol = a.explicit_map == nullptr;
  if (sol || a.G > 0) {
    // key blocks, then (routing rules) query blocks
    const dim3 grid(a.nKB + (sol ? a.nQB : 0), a.H, a.B);
    const bool sums = a.k_sums != nullptr;
    if (a.kblock == 64) {
      if (a.v_int8) sums ? pool_kernel<D, true, 2, true><<<grid, 256, 0, st>>>(a)
                         : pool_kernel<D, true, 2, false><<<grid, 256, 0, st>>>(a);
      else sums ? pool_kernel<D, false, 2, true><<<grid, 256, 0, st>>>(a)
                : pool_kernel<D, false, 2, false><<<grid, 256, 0, st>>>(a);
    } else {
      if (a.v_int8) sums ? pool_kernel<D, true, 4, true><<<grid, 256, 0, st>>>(a)
                         : pool_kernel<D, true, 4, false><<<grid, 256, 0, st>>>(a);
      else sums ? pool_kernel<D, false, 4, true><<<grid, 256, 0, st>>>(a)
                : pool_kernel<D, false, 4, false><<<grid, 256, 0, st>>>(a);
    }
  }
  if (sol) {
    const dim3 grid((a.nQB + 31) / 32 * a.H * a.B);
    const CandRange cr(a);
    const bool lds = cr.jc1 - cr.jc0 <= kLdsCand;   // candidates' proxies fit in LDS
    // 32-row workgroups take one CU each.  When there are more of them than
    // CUs, the fixed-sparsity rule runs 16-row ones, two per CU: its per-row
    // selection, which dominates, then spreads over twice the workgroups
    // (measured 4 % faster route on the 32K workload).  The threshold rule
    // stays at 32 rows: its per-row work is light, and 16-row workgroups would
    // repeat the whole proxy pass (the 32-row tiles) for half the rows
    // (measured 5 % slower).
    const bool half = a.rule == kRuleTopK && (int64_t)grid.x > a.num_cus;
    const dim3 grid16((a.nQB + 15) / 16 * a.H * a.B);
    if (a.rule == kRuleTopK) {
      if (lds && half) decide_topk_lds_kernel<D, kLdsWaves, 16><<<grid16, 64 * kLdsWaves, 0, st>>>(a);
      else if (lds) decide_topk_lds_kernel<D, kLdsWaves, 32><<<grid, 64 * kLdsWaves, 0, st>>>(a);
      else decide_topk_kernel<D><<<grid, 64 * kDecideWaves, 0, st>>>(a);
    } else {
      if (lds && half) decide_sol_lds_kernel<D, kLdsWaves, 16><<<grid16, 64 * kLdsWaves, 0, st>>>(a);
      else if (lds) decide_sol_lds_kernel<D, kLdsWaves, 32><<<grid, 64 * kLdsWaves, 0, st>>>(a);
      else decide_sol_kernel<D><<<grid, 64 * kDecideWaves, 0, st>>>(a);
    }
  } else {
    decide_explicit_kernel<<<dim3(a.nQB, a.H, a.B), 256, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_route_d<64>(a, st) : launch_route_d<128>(a, st);
}

}  // namespace sa
