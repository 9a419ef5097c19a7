// Shared device helpers for the gfx950 attention kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ditattn {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));

#define DIT_LDS(T, p) ((__attribute__((address_space(3))) T*)(p))

// Where the rows of one (b, h) live: element strides of batch, head and token
// for q, k, v (shared) and for o. The d values of a row are contiguous.
// Contiguous [B][H][N][d]: qb = H N d, qh = N d, qn = d (and the same for o).
struct Layout {
  long long qb, qh, qn;
  long long ob, oh, on;
  int H;
  __device__ __forceinline__ long long in_off(int bh) const {
    const int b = bh / H;
    return (long long)b * qb + (long long)(bh - b * H) * qh;
  }
  __device__ __forceinline__ long long out_off(int bh) const {
    const int b = bh / H;
    return (long long)b * ob + (long long)(bh - b * H) * oh;
  }
};

// Workgroups are dispatched round-robin over the 8 XCDs (blockIdx % 8), and
// each XCD has its own L2. Remap so that each XCD receives one contiguous
// range of logical tiles: consecutive q-tiles of one head then share their
// K/V stream through that XCD's L2.
__device__ __forceinline__ int xcd_remap(int w, int total) {
  const int q = total >> 3, r = total & 7;
  const int xcd = w & 7, loc = w >> 3;
  return xcd < r ? xcd * (q + 1) + loc : r * (q + 1) + (xcd - r) * q + loc;
}

// Value of the same register in lane (l + 32) % 64: swaps the two half-waves.
// Both results of v_permlane32_swap together hold the low and the high half;
// reducing them gives the pairwise reduction in every lane.
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

}  // namespace ditattn
