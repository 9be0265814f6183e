// Per-block symmetric INT8 quantization and the virtual-KV gather (gfx950).
//
// Both kernels are HBM-bound streams: one workgroup owns one quantization block
// (64 or 128 rows x d channels), keeps the whole block in registers (16-byte
// loads, 8 bf16 per load), reduces amax across the workgroup, and writes the
// INT8 codes with 8-byte stores — one read and one write of every element.
//
// Quantization rule (Configure Sol Sparse Attention, "How it works": Q and K are
// prequantized to INT8 and those codes serve routing and the exact path;
// FlashVSR Kitchen Sparse Attention, opening section: INT8 cache in 128-row
// slabs): scale = amax/127; code = clamp(rint(x * (127/amax)), -127, 127) with
// IEEE float32 division, one multiply and round-half-even; an all-zero block has
// scale 0; rows at or past the valid length get code 0 and are left out of amax.
// The streaming cache (same opening section: a sliding INT8 cache of past K/V
// per block) writes each block into a ring slot of a slab tensor instead.
#include "sa_device.h"
#include "sa_launch.h"

namespace sa {

// Source block blk is written to destination block (first + blk) mod nslots of
// a tensor of nslots blocks: the identity for a plain quantization (first = 0,
// nslots = L / R), a ring position for the streaming cache.
//
// With `sums` (plain quantization only) the kernel also writes the column sums
// of the codes it has just produced over each chunk of SR rows (32 or R), int16
// [B,H,L/SR,d] (|sum| <= 127 * 128): the routing pass then needs neither the
// codes nor a second read of them.  Thread t holds 8 channels (one 16-byte
// vector) of rows t / VPR + (256 / VPR) * i; the threads holding the same
// channels meet through lane swaps inside a wave and LDS across the four
// waves.
template <int D, int R, int SR>
__global__ __launch_bounds__(256) void quantize_kernel(const uint16_t* __restrict__ x, int64_t sB,
                                                       int64_t sH, int64_t sL, int H, int valid_len,
                                                       int nslots, int first, int8_t* __restrict__ q,
                                                       float* __restrict__ scale, int16_t* __restrict__ sums) {
  constexpr int VPR = D / 8;            // 16-byte vectors per row
  constexpr int NV = R * VPR / 256;     // vectors per thread
  constexpr int RPI = 256 / VPR;        // rows between a thread's vectors
  constexpr int NCH = R / SR;           // sum chunks per block
  // A thread's rows are t / VPR + RPI * i with t / VPR < RPI; with RPI
  // dividing SR, vector i lies in chunk i * RPI / SR for every thread.
  static_assert(SR % RPI == 0 && R % SR == 0, "a thread's vectors must fall into fixed chunks");
  static_assert(VPR == 8 || VPR == 16, "lane groups of 8 or 16 channel vectors");
  constexpr int RPC = SR / RPI;         // a thread's rows per chunk
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const uint16_t* xb = x + b * sB + h * sH;
  float vals[NV][8];
  bool valid[NV];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = t + 256 * i, row = blk * R + v / VPR, cc = v % VPR;
    valid[i] = row < valid_len;
    const uint4 raw = *reinterpret_cast<const uint4*>(xb + row * sL + cc * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      vals[i][2 * e] = __uint_as_float(w[e] << 16);
      vals[i][2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
    if (valid[i]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(vals[i][e]));
    }
  }
  __shared__ float red[4];
  __shared__ int part[4][NCH][D];   // per-wave chunk column sums
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  const int slot = (first + blk) % nslots;
  if (t == 0) scale[((int64_t)b * H + h) * nslots + slot] = amax / 127.0f;
  int8_t* qb = q + (((int64_t)b * H + h) * nslots + slot) * R * D;
  uint64_t codes[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = t + 256 * i, r = v / VPR, cc = v % VPR;
    codes[i] = quant8(vals[i], inv, valid[i]);
    *reinterpret_cast<uint64_t*>(qb + (int64_t)r * D + cc * 8) = codes[i];
  }
  if (sums == nullptr) return;   // uniform over the grid
  // Per chunk, two channels per 32-bit word as 16-bit halves holding
  // code + 128 (1..255) per row: flipping the sign bit of each byte turns a
  // code into code + 128, and masking bytes 0, 2 (or 1, 3) of a dword gives
  // channels (0, 2) (or (1, 3)) as 16-bit halves.  A wave adds SR / 4 <= 32
  // rows into a half (<= 8160), so no carry crosses into the other half.
  // pk[2w + s]: dword w of the vector, channels 4w + s and 4w + s + 2.
  const int lane = t & 63, wave = t >> 6, cc = t % VPR;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    uint32_t pk[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int i = c * RPC; i < (c + 1) * RPC; ++i) {
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const uint32_t u = (uint32_t)(codes[i] >> (32 * w)) ^ 0x80808080u;
        pk[2 * w] += u & 0x00FF00FFu;
        pk[2 * w + 1] += (u >> 8) & 0x00FF00FFu;
      }
    }
    // threads with the same channels inside the wave: lanes cc + VPR * k.
    // Lane pairs (l, l ^ 16) and (l, l ^ 32) meet through the permlane swaps
    // (VALU, no LDS traffic).
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      if (VPR <= 8) pk[e] += (uint32_t)__shfl_xor((int)pk[e], 8, 64);
      const auto r16 = __builtin_amdgcn_permlane16_swap(pk[e], pk[e], false, false);
      pk[e] = r16[0] + r16[1];
      const auto r32 = __builtin_amdgcn_permlane32_swap(pk[e], pk[e], false, false);
      pk[e] = r32[0] + r32[1];
    }
    // rows of this chunk summed into pk by the wave: (64 / VPR) lanes x RPC each
    constexpr int bias = 128 * (64 / VPR) * RPC;
    if (lane < VPR) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = cc * 8 + 4 * (e / 2) + (e % 2);
        part[wave][c][ch] = (int)(pk[e] & 0xFFFFu) - bias;
        part[wave][c][ch + 2] = (int)(pk[e] >> 16) - bias;
      }
    }
  }
  __syncthreads();
  int16_t* sb = sums + (((int64_t)b * H + h) * (nslots * R / SR) + (int64_t)blk * NCH) * D;
  for (int u = t; u < NCH * D; u += 256) {
    const int c = u / D, ch = u % D;
    sb[c * D + ch] = (int16_t)(part[0][c][ch] + part[1][c][ch] + part[2][c][ch] + part[3][c][ch]);
  }
}

// Virtual-KV gather (Configure H3 Static Virtual KV, mode list, "fast"): logical
// row r of slice l reads physical slice src[l]; channel pairs inside the rotary
// span are rotated by slice l's phase with y0 = fma(x0, c, -(x1*s)),
// y1 = fma(x0, s, x1*c) in float32, rounded to bf16, then quantized per R
// logical rows exactly as quantize_kernel does.  Nothing else is materialized.
template <int D, int R>
__global__ __launch_bounds__(256) void gather_kernel(const uint16_t* __restrict__ kp, int H, int S,
                                                     int n_phys, SrcMap src, const float* __restrict__ cosv,
                                                     const float* __restrict__ sinv, int rot_offset,
                                                     int d_rot, int n_logical, int8_t* __restrict__ kq,
                                                     float* __restrict__ kscale, int32_t* __restrict__ vbs) {
  constexpr int VPR = D / 8;
  constexpr int NV = R * VPR / 256;
  const int blk = blockIdx.x, h = blockIdx.y, b = blockIdx.z, t = threadIdx.x;
  const int row0 = blk * R, l = row0 / S, npairs = d_rot / 2;
  const int Lp = S * n_phys, Ll = S * n_logical;
  const uint16_t* base = kp + (((int64_t)b * H + h) * Lp + (int64_t)src.v[l] * S + (row0 - l * S)) * D;
  float vals[NV][8];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = t + 256 * i, r = v / VPR, cc = v % VPR;
    const uint4 raw = *reinterpret_cast<const uint4*>(base + (int64_t)r * D + cc * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float x0 = __uint_as_float(w[e] << 16), x1 = __uint_as_float(w[e] & 0xFFFF0000u);
      const int c0 = cc * 8 + 2 * e;   // rot_offset is even, so pairs never straddle
      if (c0 >= rot_offset && c0 < rot_offset + d_rot) {
        const int pidx = l * npairs + (c0 - rot_offset) / 2;
        const float cs = cosv[pidx], sn = sinv[pidx];
        const float t1 = x1 * sn, t2 = x1 * cs;
        const float y0 = __builtin_fmaf(x0, cs, -t1);
        const float y1 = __builtin_fmaf(x0, sn, t2);
        x0 = bf16_to_f32(f32_to_bf16_rne(y0));
        x1 = bf16_to_f32(f32_to_bf16_rne(y1));
      }
      vals[i][2 * e] = x0;
      vals[i][2 * e + 1] = x1;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(vals[i][e]));
  }
  __shared__ float red[4];
  amax = wave_max(amax);
  if ((t & 63) == 0) red[t >> 6] = amax;
  __syncthreads();
  amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
  if (t == 0) kscale[((int64_t)b * H + h) * (Ll / R) + blk] = amax / 127.0f;
  int8_t* qb = kq + (((int64_t)b * H + h) * Ll + row0) * D;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int v = t + 256 * i, r = v / VPR, cc = v % VPR;
    *reinterpret_cast<uint64_t*>(qb + (int64_t)r * D + cc * 8) = quant8(vals[i], inv, true);
  }
  if (b == 0 && h == 0 && t < R / 64) {
    const int bps = S / 64, j = row0 / 64 + t;
    vbs[j] = src.v[l] * bps + j % bps;
  }
}

template <int D>
static hipError_t launch_quantize_d(const QuantizeArgs& a, hipStream_t st) {
  dim3 grid(a.L / a.R, a.H, a.B);
  // sum_rows is 32 or R (only read when sums are written)
  if (a.R == 64) {
    if (a.sum_rows == 64)
      quantize_kernel<D, 64, 64><<<grid, 256, 0, st>>>(a.x, a.sB, a.sH, a.sL, a.H, a.valid_len, a.nslots, a.first,
                                                       a.q, a.scale, a.sums);
    else
      quantize_kernel<D, 64, 32><<<grid, 256, 0, st>>>(a.x, a.sB, a.sH, a.sL, a.H, a.valid_len, a.nslots, a.first,
                                                       a.q, a.scale, a.sums);
  } else {
    if (a.sum_rows == 128)
      quantize_kernel<D, 128, 128><<<grid, 256, 0, st>>>(a.x, a.sB, a.sH, a.sL, a.H, a.valid_len, a.nslots, a.first,
                                                         a.q, a.scale, a.sums);
    else
      quantize_kernel<D, 128, 32><<<grid, 256, 0, st>>>(a.x, a.sB, a.sH, a.sL, a.H, a.valid_len, a.nslots, a.first,
                                                        a.q, a.scale, a.sums);
  }
  return hipGetLastError();
}

hipError_t launch_quantize(const QuantizeArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_quantize_d<64>(a, st) : launch_quantize_d<128>(a, st);
}

template <int D>
static hipError_t launch_gather_d(const GatherArgs& a, hipStream_t st) {
  dim3 grid(a.n_logical * a.S / a.R, a.H, a.B);
  if (a.R == 64)
    gather_kernel<D, 64><<<grid, 256, 0, st>>>(a.kp, a.H, a.S, a.n_phys, a.src, a.cosv, a.sinv, a.rot_offset,
                                               a.d_rot, a.n_logical, a.kq, a.kscale, a.vbs);
  else
    gather_kernel<D, 128><<<grid, 256, 0, st>>>(a.kp, a.H, a.S, a.n_phys, a.src, a.cosv, a.sinv, a.rot_offset,
                                                a.d_rot, a.n_logical, a.kq, a.kscale, a.vbs);
  return hipGetLastError();
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t st) {
  return a.d == 64 ? launch_gather_d<64>(a, st) : launch_gather_d<128>(a, st);
}

}  // namespace sa
