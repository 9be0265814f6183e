// Device-side helpers shared by the gfx950 kernels of libsparse_attn.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef short v4s __attribute__((ext_vector_type(4)));
typedef unsigned short v8us __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

#define SA_LDS __attribute__((address_space(3)))

namespace sa {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// Quantize 8 floats with a block's reciprocal; rows past the valid length give 0.
__device__ __forceinline__ uint64_t quant8(const float* x, float inv, bool valid) {
  uint64_t packed = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float y = __builtin_rintf(x[e] * inv);
    y = fminf(fmaxf(y, -127.0f), 127.0f);
    int code = valid ? (int)y : 0;
    packed |= (uint64_t)(uint8_t)(int8_t)code << (8 * e);
  }
  return packed;
}

}  // namespace sa
