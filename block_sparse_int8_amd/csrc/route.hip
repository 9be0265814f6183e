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
// Three kernels, all reading their inputs once from HBM:
//   pool_q   — int32 column sums of the INT8 codes of each 128-row query block
//   pool_kv  — int32 column sums of each key block (into the workspace, for the
//              proxy) and per-group centroids: kbar = mean of the dequantized
//              keys, vbar = mean of V, count = valid rows
//   decide   — proxy s_ij = (Qsum_i . Ksum_j) * b_j / n_j (exact integer dot in
//              int32 pieces of 8 products, accumulated in float64), mean and
//              population std over the candidates in float64, decisions; or the
//              explicit-map expansion.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

// One workgroup per (query block, head, batch): stage the 128 x D codes in LDS,
// then each thread sums one column over a half of the rows.
template <int D>
__global__ __launch_bounds__(256) void pool_q_kernel(const int8_t* __restrict__ q, int H, int Lq,
                                                     int lq_valid, int nQB, int32_t* __restrict__ qsum) {
  __shared__ __attribute__((aligned(16))) int8_t tile[kQBlock * D];
  __shared__ int32_t part[2][D];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * H + h;
  const int8_t* src = q + (bh * Lq + (int64_t)i * kQBlock) * D;
  constexpr int NV = kQBlock * D / 16 / 256;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int v = t + 256 * e;
    reinterpret_cast<uint4*>(tile)[v] = reinterpret_cast<const uint4*>(src)[v];
  }
  __syncthreads();
  const int nvalid = min(kQBlock, max(0, lq_valid - i * kQBlock));
  for (int w = t; w < 2 * D; w += 256) {
    const int col = w % D, half = w / D;
    int32_t s = 0;
    for (int r = half * 64; r < half * 64 + 64 && r < nvalid; ++r) s += tile[r * D + col];
    part[half][col] = s;
  }
  __syncthreads();
  for (int col = t; col < D; col += 256) qsum[(bh * nQB + i) * D + col] = part[0][col] + part[1][col];
}

// One workgroup per (key block, head, batch).  Rows are summed per 32-row
// chunk so that 2x32 groups, and groups that span two K scale blocks, combine
// their chunks with the right scale.
template <int D, bool VI8>
__global__ __launch_bounds__(256) void pool_kv_kernel(RouteArgs a) {
  constexpr int MAXR = 128;
  __shared__ __attribute__((aligned(16))) int8_t ktile[MAXR * D];
  __shared__ __attribute__((aligned(16))) uint16_t vtile[MAXR * D];   // bf16 bits, or int8 codes (low byte)
  __shared__ int32_t ks[MAXR / 32][D];
  __shared__ float vs[MAXR / 32][D];
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int64_t bh = (int64_t)b * a.H + h;
  const int kb = a.kblock, row0 = j * kb, nch = kb / 32;
  const int nKS = a.Lkv / a.k_scale_rows;
  // stage K rows
  const int8_t* ksrc = a.k + (bh * a.Lkv + row0) * D;
  for (int v = t; v < kb * D / 16; v += 256)
    reinterpret_cast<uint4*>(ktile)[v] = reinterpret_cast<const uint4*>(ksrc)[v];
  // stage V rows (64-row blocks remapped through v_block_src)
  if (a.G > 0) {
    constexpr int EPV = VI8 ? 16 : 8;  // elements per 16-byte load
    for (int v = t; v < kb * D / EPV; v += 256) {
      const int r = v / (D / EPV), cc = v % (D / EPV);
      const int lr = row0 + r;
      int pr = lr;
      if (a.v_block_src) {
        int pb = a.v_block_src[lr / 64];
        pb = min(max(pb, 0), a.Lv / 64 - 1);
        pr = pb * 64 + lr % 64;
      }
      if (VI8) {
        const uint4 raw = *reinterpret_cast<const uint4*>(static_cast<const int8_t*>(a.v) + (bh * a.Lv + pr) * D + cc * 16);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) vtile[r * D + cc * 16 + e] = (uint16_t)((w[e / 4] >> (8 * (e % 4))) & 0xFF);
      } else {
        reinterpret_cast<uint4*>(vtile)[(r * D + cc * 8) / 8] =
            *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(a.v) + (bh * a.Lv + pr) * D + cc * 8);
      }
    }
  }
  __syncthreads();
  const int nvalid = min(kb, max(0, a.lkv_valid - row0));
  for (int w = t; w < nch * D; w += 256) {
    const int c = w / D, col = w % D;
    int32_t s = 0;
    float fv = 0.0f;
    int32_t iv = 0;
    for (int r = c * 32; r < c * 32 + 32 && r < nvalid; ++r) {
      s += ktile[r * D + col];
      if (a.G > 0) {
        if (VI8) iv += (int32_t)(int8_t)(vtile[r * D + col] & 0xFF);
        else fv += bf16_to_f32(vtile[r * D + col]);
      }
    }
    ks[c][col] = s;
    vs[c][col] = VI8 ? (float)iv : fv;   // |int sum| <= 127*32: exact in float
  }
  __syncthreads();
  if (a.ksum) {
    for (int col = t; col < D; col += 256) {
      int32_t s = 0;
      for (int c = 0; c < nch; ++c) s += ks[c][col];
      a.ksum[((int64_t)bh * a.nKB + j) * D + col] = s;
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
        ksum += a.k_scale[bh * nKS + crow / a.k_scale_rows] * (float)ks[c][col];
        if (VI8) {
          int pr = crow;
          if (a.v_block_src) {
            int pb = min(max(a.v_block_src[crow / 64], 0), a.Lv / 64 - 1);
            pr = pb * 64 + crow % 64;
          }
          vsum += a.v_scale[bh * (a.Lv / a.v_scale_rows) + pr / a.v_scale_rows] * vs[c][col];
        } else {
          vsum += vs[c][col];
        }
      }
      const int64_t o = ((bh * a.nKB + j) * a.G + g);
      a.kc[o * D + col] = n > 0 ? ksum / (float)n : 0.0f;
      a.vc[o * D + col] = n > 0 ? vsum / (float)n : 0.0f;
      if (col == 0) a.cnt[o] = (float)n;
    }
  }
}

// Sol decisions for QB query blocks of one (head, batch).  Dynamic LDS holds the
// proxies s[QB][nKB] in float64.
template <int D, int QB>
__global__ __launch_bounds__(256) void decide_sol_kernel(RouteArgs a) {
  extern __shared__ double sprox[];   // [QB][nKB]
  __shared__ int32_t qs[QB][D];
  __shared__ double red[4];
  const int h = blockIdx.y, b = blockIdx.z, t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int64_t bh = (int64_t)b * a.H + h;
  const int i0 = blockIdx.x * QB, nq = min(QB, a.nQB - i0);
  const int nKS = a.Lkv / a.k_scale_rows;
  for (int w = t; w < QB * D; w += 256) {
    const int qi = w / D, col = w % D;
    qs[qi][col] = qi < nq ? a.qsum[(bh * a.nQB + i0 + qi) * D + col] : 0;
  }
  __syncthreads();
  const int kb = a.kblock;
  auto is_cand = [&](int j) { return j * kb >= a.prefix && j * kb < a.lkv_valid; };
  for (int j = t; j < a.nKB; j += 256) {
    if (!is_cand(j)) continue;
    double acc[QB];
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) acc[qi] = 0.0;
    const int32_t* kr = a.ksum + (bh * a.nKB + j) * D;
#pragma unroll 2
    for (int c8 = 0; c8 < D / 8; ++c8) {
      const int4 k0 = reinterpret_cast<const int4*>(kr)[2 * c8];
      const int4 k1 = reinterpret_cast<const int4*>(kr)[2 * c8 + 1];
      const int kk[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
      for (int qi = 0; qi < QB; ++qi) {
        // |sum of 8 products| <= 8 * 16256^2 < 2^31: exact in int32
        int32_t part = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e) part += __mul24(qs[qi][c8 * 8 + e], kk[e]);
        acc[qi] += (double)part;
      }
    }
    const double bj = (double)a.k_scale[bh * nKS + j];
    const double nj = (double)min(kb, a.lkv_valid - j * kb);
#pragma unroll
    for (int qi = 0; qi < QB; ++qi) sprox[qi * a.nKB + j] = acc[qi] * bj / nj;
  }
  __syncthreads();
  // candidates form the contiguous range [jc0, jc1)
  const int jc0 = (a.prefix + kb - 1) / kb;
  const int jc1 = min(a.nKB, (a.lkv_valid + kb - 1) / kb);
  const int N = max(0, jc1 - jc0);
  const double tau = (double)a.tau;
  for (int qi = 0; qi < nq; ++qi) {
    const int i = i0 + qi;
    double s = 0.0;
    for (int j = jc0 + t; j < jc1; j += 256) s += sprox[qi * a.nKB + j];
    s = wave_sum_f64(s);
    if (lane == 0) red[wave] = s;
    __syncthreads();
    const double mu = N > 0 ? (red[0] + red[1] + red[2] + red[3]) / N : __builtin_nan("");
    __syncthreads();
    double ss = 0.0;
    for (int j = jc0 + t; j < jc1; j += 256) {
      const double dlt = sprox[qi * a.nKB + j] - mu;
      ss += dlt * dlt;
    }
    ss = wave_sum_f64(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    const double sigma = N > 0 ? sqrt((red[0] + red[1] + red[2] + red[3]) / N) : __builtin_nan("");
    __syncthreads();
    const bool keep_all = N == 0 || (tau > 0 && __builtin_isinf(tau)) || sigma == 0.0;
    const double thr = keep_all ? 0.0 : mu + tau * sigma;
    uint8_t* mrow = a.map + (bh * a.nQB + i) * a.nKB;
    for (int j = t; j < a.nKB; j += 256) {
      uint8_t st;
      if (j * kb >= a.lkv_valid) st = 0;
      else if (j * kb < a.prefix) st = 1;
      else st = (!keep_all && sprox[qi * a.nKB + j] > thr) ? 2 : 1;
      mrow[j] = st;
    }
    if (a.stats && t == 0) {
      a.stats[(bh * a.nQB + i) * 2] = mu;
      a.stats[(bh * a.nQB + i) * 2 + 1] = sigma;
    }
  }
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
    if (j * a.kblock < a.prefix) st = 1;
    if (j * a.kblock >= a.lkv_valid) st = 0;
    mrow[j] = (uint8_t)st;
  }
  if (a.stats && t == 0) {
    a.stats[(bh * a.nQB + i) * 2] = __builtin_nan("");
    a.stats[(bh * a.nQB + i) * 2 + 1] = __builtin_nan("");
  }
}

size_t route_workspace_bytes(int B, int H, int nQB, int nKB, int d) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return al((size_t)B * H * nQB * d * 4) + al((size_t)B * H * nKB * d * 4);
}

static int sol_qb(int nKB) {
  // proxies of QB query blocks stay in LDS: QB * nKB * 8 bytes <= 64 KiB
  int qb = 8;
  while (qb > 1 && (size_t)qb * nKB * 8 > 65536) qb /= 2;
  return qb;
}

template <int D>
static hipError_t launch_route_d(const RouteArgs& a, hipStream_t st) {
  const bool sol = a.explicit_map == nullptr;
  if (sol) {
    pool_q_kernel<D><<<dim3(a.nQB, a.H, a.B), 256, 0, st>>>(a.q, a.H, a.Lq, a.lq_valid, a.nQB, a.qsum);
  }
  if (sol || a.G > 0) {
    if (a.v_int8) pool_kv_kernel<D, true><<<dim3(a.nKB, a.H, a.B), 256, 0, st>>>(a);
    else pool_kv_kernel<D, false><<<dim3(a.nKB, a.H, a.B), 256, 0, st>>>(a);
  }
  if (sol) {
    const int qb = sol_qb(a.nKB);
    const size_t lds = (size_t)qb * a.nKB * 8;
    dim3 grid((a.nQB + qb - 1) / qb, a.H, a.B);
    switch (qb) {
      case 8: decide_sol_kernel<D, 8><<<grid, 256, lds, st>>>(a); break;
      case 4: decide_sol_kernel<D, 4><<<grid, 256, lds, st>>>(a); break;
      case 2: decide_sol_kernel<D, 2><<<grid, 256, lds, st>>>(a); break;
      default: decide_sol_kernel<D, 1><<<grid, 256, lds, st>>>(a); break;
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
