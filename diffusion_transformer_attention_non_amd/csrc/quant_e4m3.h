// Per-tensor absmax quantisation of bfloat16 to OCP e4m3 on gfx950.
//
// Three launches on one stream: clear the caller's amax word, reduce max|x|
// into it with one atomic per workgroup, then quantise every element with
// s = 448 / amax (fp32, correctly rounded), y = x * s (fp32), clamp to
// [-448, 448] and round to e4m3 with the hardware converter (nearest-even).
// This is an HBM-bound pass (2 bytes read + 1 byte written per element,
// plus a second 2-byte read), kept as plain coalesced 16-byte accesses.
#pragma once
#include "attn_common.h"

namespace ditattn {

constexpr int kQuantThreads = 256;

__global__ void amax_clear_kernel(uint32_t* ws) {
  if (threadIdx.x == 0) *ws = 0u;
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

__global__ __launch_bounds__(kQuantThreads)
void amax_kernel(const uint16_t* __restrict__ x, int64_t n8, uint32_t* __restrict__ ws) {
  float m = 0.f;
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n8; i += stride) {
    const i32x4_t w = *(const i32x4_t*)(x + i * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)w[e];
      m = fmaxf(m, fabsf(bf16_bits_to_float(u & 0xffffu)));
      m = fmaxf(m, fabsf(bf16_bits_to_float(u >> 16)));
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
  __shared__ float red[kQuantThreads / 64];
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float b = red[0];
#pragma unroll
    for (int w = 1; w < kQuantThreads / 64; ++w) b = fmaxf(b, red[w]);
    // non-negative floats order like their bit patterns
    atomicMax(ws, __float_as_uint(b));
  }
}

__device__ __forceinline__ float quant_scale(float amax) {
  const float s = __fdiv_rn(448.0f, amax);
  return (amax > 0.f && __builtin_isfinite(s)) ? s : 1.0f;
}

__global__ __launch_bounds__(kQuantThreads)
void quant_e4m3_kernel(const uint16_t* __restrict__ x, int64_t n8, uint8_t* __restrict__ x8,
                       float* __restrict__ descale, const uint32_t* __restrict__ ws) {
  const float s = quant_scale(__uint_as_float(*ws));
  if (blockIdx.x == 0 && threadIdx.x == 0) *descale = __fdiv_rn(1.0f, s);
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n8; i += stride) {
    const i32x4_t w = *(const i32x4_t*)(x + i * 8);
    float y[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const uint32_t u = (uint32_t)w[e];
      y[2 * e] = fminf(fmaxf(__fmul_rn(bf16_bits_to_float(u & 0xffffu), s), -448.f), 448.f);
      y[2 * e + 1] = fminf(fmaxf(__fmul_rn(bf16_bits_to_float(u >> 16), s), -448.f), 448.f);
    }
    uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0u, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], lo, true);
    uint32_t hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0u, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], hi, true);
    *(uint2*)(x8 + i * 8) = make_uint2(lo, hi);
  }
}

}  // namespace ditattn
