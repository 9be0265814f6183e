// Measurement probes for the roofline ceilings (not part of the attention
// path): matrix-core throughput of the two MFMA shapes the forward issues, alone
// and in the forward's mix, and HBM read / write / copy bandwidth.
//
// The clock of this part follows its power draw, which follows the operands'
// switching activity, so the matrix-core loops cycle through several random
// operand registers per lane (loaded once) instead of reusing one.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

namespace {

constexpr int kOps = 4;    // operand registers cycled per lane
constexpr int kAcc = 4;    // independent accumulators per wave

// mode 0: v_mfma_i32_32x32x32_i8 only; 1: v_mfma_f32_32x32x16_bf16 only;
// 2: one int8 MFMA per two bf16 ones (equal int8 ops and bf16 flops, the
// forward's exact-tile mix).  Each iteration issues kAcc MFMAs per wave
// (mode 2: kAcc / 2 int8 and kAcc bf16 ones).
__global__ __launch_bounds__(256) void probe_mfma_kernel(const int* __restrict__ src, int iters, int mode,
                                                         int* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v4i a[kOps], b[kOps];
#pragma unroll
  for (int u = 0; u < kOps; ++u) {
    a[u] = *reinterpret_cast<const v4i*>(src + ((blockIdx.x * 7 + u) % 64) * 256 + lane * 4);
    b[u] = *reinterpret_cast<const v4i*>(src + ((blockIdx.x * 5 + u + 3) % 64) * 256 + lane * 4);
  }
  v16i ai[kAcc];
  v16f af[kAcc];
#pragma unroll
  for (int c = 0; c < kAcc; ++c) {
    ai[c] = (v16i){};
    af[c] = (v16f){};
  }
  // the loop is unrolled by kOps so every operand index is a compile-time
  // constant (a run-time index into a register array would go through memory)
  if (mode == 0) {
    for (int it = 0; it < iters; it += kOps) {
#pragma unroll
      for (int u = 0; u < kOps; ++u)
#pragma unroll
        for (int c = 0; c < kAcc; ++c)
          ai[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(u + c) % kOps], b[(u + 2 * c) % kOps], ai[c], 0, 0, 0);
    }
  } else if (mode == 1) {
    for (int it = 0; it < iters; it += kOps) {
#pragma unroll
      for (int u = 0; u < kOps; ++u)
#pragma unroll
        for (int c = 0; c < kAcc; ++c)
          af[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[(u + c) % kOps]),
                                                          __builtin_bit_cast(v8bf, b[(u + 2 * c) % kOps]), af[c],
                                                          0, 0, 0);
    }
  } else {
    // per iteration: kAcc/2 int8 MFMAs and kAcc bf16 MFMAs
    for (int it = 0; it < iters; it += kOps) {
#pragma unroll
      for (int u = 0; u < kOps; ++u)
#pragma unroll
        for (int c = 0; c < kAcc; ++c) {
          if (c % 2 == 0)
            ai[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[(u + c) % kOps], b[(u + 2 * c) % kOps], ai[c], 0, 0, 0);
          af[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, b[(u + c) % kOps]),
                                                          __builtin_bit_cast(v8bf, a[(u + 3 * c) % kOps]), af[c],
                                                          0, 0, 0);
        }
    }
  }
  int r = 0;
#pragma unroll
  for (int c = 0; c < kAcc; ++c)
#pragma unroll
    for (int e = 0; e < 16; ++e) r ^= ai[c][e] ^ __float_as_int(af[c][e]);
  if (r == 0x7F123456) sink[blockIdx.x * 256 + threadIdx.x] = r;   // keeps the work; practically never taken
}

// Grid-stride bandwidth kernels over n16 16-byte units; each thread keeps four
// independent 16-byte accesses in flight per iteration (n16 must be a
// multiple of 4 * 256 * gridDim.x for full coverage by the unrolled part;
// the tail loop covers the rest).
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4* __restrict__ x, int64_t n16,
                                                         int* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256, base = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t i = base;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = x[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  if (acc == 0x7F123456u) sink[0] = (int)acc;
}

__global__ __launch_bounds__(256) void probe_write_kernel(uint4* __restrict__ y, int64_t n16) {
  const uint4 v = make_uint4(1u, 2u, 3u, 4u);
  const int64_t stride = (int64_t)gridDim.x * 256, base = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t i = base;
  for (; i + 3 * stride < n16; i += 4 * stride) {
#pragma unroll
    for (int u = 0; u < 4; ++u) y[i + u * stride] = v;
  }
  for (; i < n16; i += stride) y[i] = v;
}

__global__ __launch_bounds__(256) void probe_copy_kernel(const uint4* __restrict__ x, uint4* __restrict__ y,
                                                         int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * 256, base = (int64_t)blockIdx.x * 256 + threadIdx.x;
  int64_t i = base;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = x[i + u * stride];
#pragma unroll
    for (int u = 0; u < 4; ++u) y[i + u * stride] = v[u];
  }
  for (; i < n16; i += stride) y[i] = x[i];
}

}  // namespace

extern "C" {

// src: 64 * 256 int32 of random bits; sink: blocks * 256 int32.  iters is
// rounded up to a multiple of 4.  MFMAs per wave: iters * kAcc (modes 0, 1) or
// iters * kAcc * 3 / 2 (mode 2).
int32_t sa_probe_mfma(const int* src, int* sink, int32_t mode, int32_t iters, int32_t blocks, void* stream) {
  if (!src || !sink || mode < 0 || mode > 2 || iters < 1 || blocks < 1) return 1;
  probe_mfma_kernel<<<blocks, 256, 0, static_cast<hipStream_t>(stream)>>>(src, iters, mode, sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

// kind 0: read x; 1: write y; 2: copy x -> y.  bytes: a multiple of 16.
int32_t sa_probe_bandwidth(const void* x, void* y, int64_t bytes, int32_t kind, int32_t blocks, int* sink,
                           void* stream) {
  if (bytes % 16 || blocks < 1 || kind < 0 || kind > 2) return 1;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n = bytes / 16;
  if (kind == 0) probe_read_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint4*>(x), n, sink);
  else if (kind == 1) probe_write_kernel<<<blocks, 256, 0, st>>>(static_cast<uint4*>(y), n);
  else probe_copy_kernel<<<blocks, 256, 0, st>>>(static_cast<const uint4*>(x), static_cast<uint4*>(y), n);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
