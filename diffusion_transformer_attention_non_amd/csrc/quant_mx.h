// Block-scaled (MX-style) quantisation of bfloat16 to e4m3 on gfx950: every
// 32 consecutive values along one axis share a power-of-two scale 2^e,
// stored as the E8M0 byte e + 127. e is the smallest integer with
// amax / 2^e <= 448 (at least -127; an all-zero block takes -127), so no
// element saturates; each element is x / 2^e (exact) rounded to e4m3 by the
// hardware converter (nearest-even). HBM-bound passes with one thread per
// block: along d (Q, K rows) a thread reads its 64 contiguous bytes; along
// the tokens (V columns) neighbouring threads take neighbouring columns, so
// each token row is read and written coalesced.
#pragma once
#include "attn_common.h"
#include "quant_e4m3.h"   // bf16_bits_to_float, kQuantThreads

namespace ditattn {

// smallest e >= -127 with amax / 2^e <= 448: with amax = 1.f 2^E, amax / 2^(E-8)
// = 256 * 1.f, which exceeds 448 exactly when the significand passes 1.75
__device__ __forceinline__ int mx_exponent(float amax) {
  const uint32_t b = __float_as_uint(amax);
  const int E = (int)((b >> 23) & 255u);
  if (E == 0) return -127;                       // zero, or below 2^-126 (e would be under -127)
  const int e = E - 127 - 8 + ((b & 0x7FFFFFu) > 0x600000u ? 1 : 0);
  return e < -127 ? -127 : e;
}

// 2^-e as a float (e in [-127, 120]: the exponent field 127 - e is in [7, 254])
__device__ __forceinline__ float mx_inv_scale(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// along d: block i = 32 consecutive values (row-major), scale byte i
__global__ __launch_bounds__(kQuantThreads)
void quant_mx_rows_kernel(const uint16_t* __restrict__ x, int64_t n_blocks, uint8_t* __restrict__ x8,
                          uint8_t* __restrict__ scales) {
  const int64_t stride = (int64_t)gridDim.x * kQuantThreads;
  for (int64_t i = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; i < n_blocks; i += stride) {
    float v[32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const i32x4_t w = *(const i32x4_t*)(x + i * 32 + q * 8);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        v[q * 8 + 2 * e] = bf16_bits_to_float((uint32_t)w[e] & 0xffffu);
        v[q * 8 + 2 * e + 1] = bf16_bits_to_float((uint32_t)w[e] >> 16);
      }
    }
    float amax = 0.f;
#pragma unroll
    for (int t = 0; t < 32; ++t) amax = fmaxf(amax, fabsf(v[t]));
    const int e = mx_exponent(amax);
    const float inv = mx_inv_scale(e);
    i32x4_t out[2];
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const float* p = v + h * 16 + wd * 4;
        uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0] * inv, p[1] * inv, 0u, false);
        out[h][wd] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(p[2] * inv, p[3] * inv, lo, true);
      }
    *(i32x4_t*)(x8 + i * 32) = out[0];
    *(i32x4_t*)(x8 + i * 32 + 16) = out[1];
    scales[i] = (uint8_t)(e + 127);
  }
}

// along the tokens: workgroup (t, bh) with d threads; thread c takes column c
// over tokens 32 t .. min(32 t + 32, N) - 1 and writes its scale to
// [bh][t][c % 32][c / 32]
__global__ void quant_mx_tokens_kernel(const uint16_t* __restrict__ x, int N, int d, uint8_t* __restrict__ x8,
                                       uint8_t* __restrict__ scales) {
  const int t = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const int n0 = t * 32, rows = min(32, N - n0);
  const size_t base = ((size_t)bh * N + n0) * d + c;
  float amax = 0.f;
  for (int r = 0; r < rows; ++r) amax = fmaxf(amax, fabsf(bf16_bits_to_float(x[base + (size_t)r * d])));
  const int e = mx_exponent(amax);
  const float inv = mx_inv_scale(e);
  for (int r = 0; r < rows; ++r) {
    const float y = bf16_bits_to_float(x[base + (size_t)r * d]) * inv;
    x8[base + (size_t)r * d] = (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(y, 0.f, 0u, false) & 0xffu);
  }
  const int n_vb = (N + 31) / 32;
  scales[((size_t)bh * n_vb + t) * d + (c % 32) * (d / 32) + c / 32] = (uint8_t)(e + 127);
}

}  // namespace ditattn
