// Sustained matrix-core rate on attention-like operands.
//
// The dense MFMA peaks of the MI355X assume the 2.4 GHz peak engine clock.
// Under a stream of products whose operands change from one product to the
// next, the part reaches its power limit well below that clock, and how far
// below depends on the operands' bits (zeros or repeated operands draw far
// less). This kernel measures the rate such a stream sustains, so that an
// attention kernel can be set against what the matrix cores deliver on the
// same kind of data on the same card: one workgroup of four waves per CU
// (one wave per SIMD, as the attention kernels run), every wave issuing
// independent products back to back on operands drawn once from a counter
// hash and cycled through, bf16 values of roughly unit variance (the
// attention workloads' Q, K, V) or e4m3 codes of magnitude 2^-4 .. 2^3.
// Each wave records its shader-clock cycles (s_memtime) and wall-clock
// ticks (s_memrealtime) over the loop; their ratio is the shader clock.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "attn_common.h"

namespace ditattn {

constexpr int kCeilingLds = 96 * 1024;   // more than half the CU's LDS: one workgroup per CU

__device__ __forceinline__ uint32_t ceiling_hash(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

// rec[2 w], rec[2 w + 1]: cycles and wall ticks of wave w = 4 blockIdx + wave
template <bool FP8>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_ceiling_kernel(long long* __restrict__ rec, int rounds) {
  extern __shared__ char ceiling_lds[];
  (void)ceiling_lds;
  typedef int i32x8_t __attribute__((ext_vector_type(8)));
  const int tid = threadIdx.x, wave = tid >> 6;
  const uint32_t base = (blockIdx.x * 256u + tid) * 64u;
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.f;
  long long t0, w0;
  if constexpr (FP8) {
    // bytes with exponent field 4..11 and a random sign: normal e4m3 values
    auto code4 = [](uint32_t h) {
      uint32_t r = 0;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const uint32_t x = (h >> (8 * k)) & 0xffu;
        r |= (((x & 0x3fu) + 0x20u) | (x & 0x80u)) << (8 * k);
      }
      return (int)r;
    };
    i32x8_t a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t h1 = ceiling_hash(base + j * 8 + i), h2 = ceiling_hash(h1 + 0x9e3779b9u);
        a[j][i] = code4(h1);
        b[j][i] = code4(h2);
      }
    // the operands and the zeroed accumulators exist before the first clock
    // reading (the compiler would otherwise build them inside the timed span)
#pragma unroll
    for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(a[j]), "+v"(b[j]), "+v"(acc[j]));
    __builtin_amdgcn_sched_barrier(0);
    t0 = clock64();
    w0 = wall_clock64();
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j)   // scale exponents 127: 2^0
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[j], b[(j + 3) & 7], acc[j], 0, 0, 0, 127, 0, 127);
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[(j + 5) & 7], b[j], acc[j], 0, 0, 0, 127, 0, 127);
    }
  } else {
    bf16x8_t a[8], b[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t h1 = ceiling_hash(base + j * 8 + i), h2 = ceiling_hash(h1 + 0x9e3779b9u);
        // a sum of four 16-bit uniforms, centred and scaled: about N(0, 1)
        const float u = ((h1 & 0xffffu) + (h1 >> 16) + (h2 & 0xffffu) + (h2 >> 16)) * (1.f / 65536.f) - 2.f;
        const float w = ((h2 & 0xffu) * (1.f / 256.f) - 0.5f) * 3.4f;
        a[j][i] = (__bf16)(u * 1.7f);
        b[j][i] = (__bf16)w;
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      i32x4_t x = __builtin_bit_cast(i32x4_t, a[j]), y = __builtin_bit_cast(i32x4_t, b[j]);
      asm volatile("" : "+v"(x), "+v"(y), "+v"(acc[j]));
      a[j] = __builtin_bit_cast(bf16x8_t, x);
      b[j] = __builtin_bit_cast(bf16x8_t, y);
    }
    __builtin_amdgcn_sched_barrier(0);
    t0 = clock64();
    w0 = wall_clock64();
    for (int it = 0; it < rounds; ++it) {
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[(j + 3) & 7], acc[j], 0, 0, 0);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(j + 5) & 7], b[j], acc[j], 0, 0, 0);
    }
  }
  const long long dt = clock64() - t0, dw = wall_clock64() - w0;
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  const int w = blockIdx.x * 4 + wave;
  if ((tid & 63) == 0) {
    rec[2 * w] = dt;
    rec[2 * w + 1] = dw;
  }
  // the products must not be dropped: a sum that is never this bit pattern
  // (the largest finite float) stores nothing
  if (__float_as_uint(s) == 0x7F7FFFFFu) rec[2 * w] = -1;
}

}  // namespace ditattn
