// bf16 flash-style attention forward for gfx950 (CDNA4).
//
// One workgroup owns BR = NW * QB * 32 query rows of one (b, h); each of its
// NW waves owns QB blocks of 32 query rows. The workgroup streams the K and V
// rows of its head through LDS in tiles of KB keys (double-buffered) and keeps
// a running row maximum m and row sum l (online softmax), so the N x N score
// matrix never exists in memory.
//
// Transposed formulation. A 32x32x16 MFMA leaves each lane with one column and
// 16 rows of its 32x32 result. Computing S^T = K Q^T puts one query per lane
// and 16 of its keys in registers, so a row maximum / row sum is 15 in-lane
// operations plus one exchange between the two half-waves, and the
// probabilities P^T are already in the B-operand layout of O^T = V^T P^T.
// V^T comes out of LDS with ds_read_b64_tr_b16, which hands each lane one
// d-column of a 4-key x 16-column block.
//
// Lazy rescaling: the running maximum used for the exponentials is only
// raised when some row's new maximum exceeds it by more than TAU (log2 units).
// The result is the same real number (O and l carry the same stale maximum);
// the probabilities stay below 2^TAU, far inside bf16/fp32 range.
#pragma once
#include "attn_common.h"

namespace ditattn {

template <int D, int QB, int NW, int KB, int VSWZ = 2>
struct Bf16Cfg {
  static constexpr int kD = D, kQB = QB, kNW = NW, kKB = KB, kVSwz = VSWZ;
  static constexpr int kThreads = NW * 64;
  static constexpr int kBR = NW * QB * 32;          // query rows per workgroup
  static constexpr int kKS = D / 16;                // MFMA k-steps over d
  static constexpr int kDB = D / 32;                // 32-wide d blocks of O
  static constexpr int kKBLK = KB / 32;             // 32-key blocks per tile
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;    // 16-byte chunks per row
  static constexpr int kTileBytes = KB * kRowBytes;
  static constexpr int kLdsBytes = 2 * 2 * kTileBytes;   // {K,V} x double buffer
  static constexpr int kLoadsPerThread = KB * kChunks / kThreads;
  static_assert(KB * kChunks % kThreads == 0, "tile chunks must split evenly over the workgroup");
};

// Byte offset of 16-byte chunk c of row r inside a [rows][kChunks] tile. The
// XOR swizzle spreads the rows read together by one LDS instruction over
// distinct banks.
template <int CHUNKS>
__device__ __forceinline__ int swz(int r, int c) {
  return r * (CHUNKS * 16) + ((c ^ (r & (CHUNKS - 1))) << 4);
}

// V tiles are read with ds_read_b64_tr_b16: each 16-lane group reads 4
// consecutive rows x 32 contiguous bytes (one 32-byte pair of chunks), and the
// two groups of a half-wave read neighbouring pairs of the same rows.
// Swizzling 16-byte chunks by row (MODE 0) leaves rows r and r^1 on the same
// 32-byte bank slots. MODE 1 XORs the pair index with (row mod 8): the 4 rows
// of one group land on 4 distinct 32-byte slots of 128 bytes. MODE 2 XORs it
// with f(row mod 4), f = {0, 3, 5, 6}: distinct in the low two bits (4 rows
// of one group over 128 bytes) and, together with their neighbour pair
// (f ^ 1), 8 distinct slots over 256 bytes (both groups of a half-wave).
// Stores of whole rows stay conflict-free since a row's pairs are permuted.
template <int CHUNKS, int MODE = 2>
__device__ __forceinline__ int swz_v(int r, int c) {
  if constexpr (MODE == 0) {
    return r * (CHUNKS * 16) + ((c ^ (r & (CHUNKS - 1))) << 4);
  } else if constexpr (MODE == 1) {
    constexpr int kPairMask = (CHUNKS / 2 < 8 ? CHUNKS / 2 : 8) - 1;
    return r * (CHUNKS * 16) + ((((c >> 1) ^ (r & kPairMask)) << 5) | ((c & 1) << 4));
  } else {
    constexpr int kPairMask = CHUNKS / 2 - 1;
    const int f = (0x6530 >> ((r & 3) * 4)) & 7;      // f(0..3) = 0, 3, 5, 6
    return r * (CHUNKS * 16) + (((((c >> 1) ^ f) & kPairMask) << 5) | ((c & 1) << 4));
  }
}

constexpr float kTauBf16 = 8.0f;

template <class C>
__global__ __launch_bounds__(C::kThreads)
void attn_fwd_bf16_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                          const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                          float* __restrict__ LSEg, int N, int n_qtiles,
                          float scale_log2, float scale, Layout L) {
  constexpr int QB = C::kQB, KB = C::kKB, KS = C::kKS, DB = C::kDB, KBLK = C::kKBLK;
  constexpr int CH = C::kChunks, TB = C::kTileBytes;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const long long ibase = L.in_off(bh);
  const uint16_t* Q = Qg + ibase;
  const uint16_t* K = Kg + ibase;
  const uint16_t* V = Vg + ibase;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * C::kBR + wave * QB * 32;

  // ---- Q^T fragments (B operand): lane holds query q0+qb*32+l32, d = ks*16 + hh*8 .. +7
  bf16x8_t qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4_t raw = {0, 0, 0, 0};
      if (row < N) raw = *(const i32x4_t*)(Q + (long long)row * L.qn + ks * 16 + hh * 8);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  f32x16_t acc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) { m_run[qb] = -INFINITY; l_run[qb] = 0.f; }

  const int n_kt = (N + KB - 1) / KB;

  // ---- global -> register staging of one K/V tile
  i32x4_t stK[C::kLoadsPerThread], stV[C::kLoadsPerThread];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::kLoadsPerThread; ++i) {
      const int ci = tid + i * C::kThreads;
      const int r = ci / CH, c = ci % CH;
      const int key = kt * KB + r;
      if (key < N) {
        stK[i] = *(const i32x4_t*)(K + (long long)key * L.qn + c * 8);
        stV[i] = *(const i32x4_t*)(V + (long long)key * L.qn + c * 8);
      } else {
        stK[i] = i32x4_t{0, 0, 0, 0};
        stV[i] = i32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto store_tile = [&](int buf) {
    char* kb = smem + buf * 2 * TB;
    char* vb = kb + TB;
#pragma unroll
    for (int i = 0; i < C::kLoadsPerThread; ++i) {
      const int ci = tid + i * C::kThreads;
      const int r = ci / CH, c = ci % CH;
      *(i32x4_t*)(kb + swz<CH>(r, c)) = stK[i];
      *(i32x4_t*)(vb + swz_v<CH, C::kVSwz>(r, c)) = stV[i];
    }
  };

  load_tile(0);
  store_tile(0);
  __syncthreads();

  // per-lane constant parts of the V^T transpose-read address
  const int g = lane >> 4, gi = lane & 15;
  const int tr_row = (g >> 1) * 4 + (gi >> 2);            // key row within an 8-key slab
  const int tr_chunk = (g & 1) * 2 + ((gi & 3) >> 1);     // chunk within a 32-wide d block
  const int tr_off = (gi & 1) * 8;                         // byte within chunk

  for (int kt = 0; kt < n_kt; ++kt) {
    const int buf = kt & 1;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) load_tile(kt + 1);
    const char* kbuf = smem + buf * 2 * TB;
    const char* vbuf = kbuf + TB;

    // ---- S^T = K Q^T for KB keys x QB*32 queries
    f32x16_t s[KBLK][QB];
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb) {
        const int r = kb * 32 + l32;
        const bf16x8_t a = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(kbuf + swz<CH>(r, ks * 2 + hh)));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }

    // ---- keys past N (last tile only) do not exist
    if (kt == n_kt - 1 && (N % KB) != 0) {
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = kt * KB + kb * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
          if (key >= N)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][r] = -INFINITY;
        }
    }

    // ---- online softmax: row max, lazy rescale
    float m_new[QB];
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = s[0][qb][0];
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][qb][r]);
      mx = pair_max(mx);
      m_new[qb] = fmaxf(m_run[qb], mx);
      grow |= (m_new[qb] - m_run[qb]) * scale_log2 > kTauBf16;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float alpha = fast_exp2((m_run[qb] - m_new[qb]) * scale_log2);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
        m_run[qb] = m_new[qb];
      }
    }

    // ---- P = exp2(S*c - m*c), row sums, bf16 B operands of O^T += V^T P^T
    bf16x8_t pb[KBLK][2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = m_run[qb] * scale_log2;
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          bf16x8_t v;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float p = fast_exp2(fmaf(s[kb][qb][half * 8 + e], scale_log2, -mc));
            ls += p;
            v[e] = (__bf16)p;
          }
          pb[kb][half][qb] = v;
        }
      l_run[qb] += ls;
    }

    // ---- O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < KBLK; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int rbase = kb * 32 + half * 16 + tr_row;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const int c = db * 4 + tr_chunk;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              DIT_LDS(i16x4_t, (vbuf + swz_v<CH, C::kVSwz>(rbase, c) + tr_off)));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              DIT_LDS(i16x4_t, (vbuf + swz_v<CH, C::kVSwz>(rbase + 8, c) + tr_off)));
          const i32x2_t lo2 = __builtin_bit_cast(i32x2_t, lo), hi2 = __builtin_bit_cast(i32x2_t, hi);
          const i32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
          const bf16x8_t a = __builtin_bit_cast(bf16x8_t, a4);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][half][qb], acc[qb][db], 0, 0, 0);
        }
      }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, bf16 round-to-nearest-even, [B][H][N][d]
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    const float inv = 1.0f / l_tot;
    const int row = q0 + qb * 32 + l32;
    if (row < N) {
      uint16_t* orow = Og + L.out_off(bh) + (long long)row * L.on;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + i * 8 + hh * 4;
          uint2 w;
          w.x = pack_bf16x2(acc[qb][db][i * 4 + 0] * inv, acc[qb][db][i * 4 + 1] * inv);
          w.y = pack_bf16x2(acc[qb][db][i * 4 + 2] * inv, acc[qb][db][i * 4 + 3] * inv);
          *(uint2*)(orow + d0) = w;
        }
      if (LSEg != nullptr && hh == 0)
        LSEg[(size_t)bh * N + row] = m_run[qb] * scale + logf(l_tot);
    }
  }
}

}  // namespace ditattn
