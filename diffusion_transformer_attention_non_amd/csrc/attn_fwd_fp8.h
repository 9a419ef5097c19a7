// fp8-e4m3 flash-style attention forward for gfx950 (CDNA4), d = 128, bf16 out.
//
// Same structure as the bf16 kernel (transposed S^T = K Q^T, online softmax,
// O^T += V^T P^T), with both contractions on the 32x32x64 f8f6f4 MFMA in its
// e4m3 x e4m3 form. Per-tensor descales dq, dk fold into the logit
// multiplier and dv into the epilogue. The probabilities, below 2^TAU
// relative to the running maximum, are multiplied by 2^(8-TAU) (so at most
// 256 < 448; the factor is added to the exponent argument, not multiplied)
// and rounded to e4m3 (round-to-nearest-even) before the second
// contraction; the row sum uses the unrounded fp32 values. The last, partly
// filled round of workgroups is split along the keys like the bf16 kernel's
// (PipeSplit, attn_split_combine_kernel).
//
// The two MFMA operands of one product must place the same k index in the
// same (half-wave, byte) slot; any such placement gives the same sum. For
// S^T both sides hold 32 consecutive d values per lane. For O^T the P^T
// slots are the S^T accumulator order, and V^T is gathered to match with
// ds_read_b64_tr_b8: each lane pair addresses one key row, and each lane
// receives one d-column of an 8-key x 16-column block.
#pragma once
#include "attn_common.h"
#include "attn_fwd_bf16_pipe.h"     // PipeSplit

namespace ditattn {

template <int QB, int NW, int KB>
struct Fp8Cfg {
  static constexpr int kD = 128, kQB = QB, kNW = NW, kKB = KB;
  static constexpr int kThreads = NW * 64;
  static constexpr int kBR = NW * QB * 32;
  static constexpr int kKS = 128 / 64;              // MFMA k-steps over d (k = 64)
  static constexpr int kDB = 128 / 32;
  static constexpr int kKBLK = KB / 32;
  static constexpr int kRowBytes = 128;
  static constexpr int kChunks = 8;
  static constexpr int kTileBytes = KB * kRowBytes;
  static constexpr int kLdsBytes = 2 * 2 * kTileBytes;
  static constexpr int kLoadsPerThread = KB * kChunks / kThreads;
  static_assert(KB % 64 == 0, "the PV contraction consumes 64 keys per MFMA");
  static_assert(KB * kChunks % kThreads == 0, "tile chunks must split evenly over the workgroup");
};

constexpr float kTauFp8 = 4.0f;
constexpr float kPScaleLog2Fp8 = 4.0f;   // P is scaled by 2^(8 - TAU) = 16

// LDS serves 256 bytes (64 four-byte banks) per pass; with 128-byte rows two
// rows share a pass, one in each half (row parity). Both swizzles below
// permute the 16-byte chunks inside a row, so row-wise stores stay
// conflict-free.
// K tiles: a ds_read_b128 pass covers rows 0..15 of one chunk column. The
// rows of each parity need 8 distinct chunks: XOR with (row >> 1) mod 8.
__device__ __forceinline__ int swz8_k(int r, int c) {
  return r * 128 + ((c ^ ((r >> 1) & 7)) << 4);
}
// V tiles: a ds_read_b64_tr_b8 pass covers 8 rows {0-3, 8-11} (+4) and two
// neighbouring chunk columns c, c+1 (c even). The 4 rows of each parity need
// {c ^ f, c ^ f ^ 1} disjoint: f = 2 * ((r >> 1) & 1) + 4 * ((r >> 3) & 1).
__device__ __forceinline__ int swz8_v(int r, int c) {
  return r * 128 + ((c ^ ((((r >> 1) & 1) << 1) | (((r >> 3) & 1) << 2))) << 4);
}

__device__ __forceinline__ uint32_t pack_e4m3x4(float a, float b, float c, float d) {
  uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0u, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

template <class C>
__global__ __launch_bounds__(C::kThreads)
void attn_fwd_fp8_kernel(const uint8_t* __restrict__ Qg, const uint8_t* __restrict__ Kg,
                         const uint8_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                         float* __restrict__ LSEg, const float* __restrict__ descale,
                         int N, int n_qtiles, float scale_log2, float scale, PipeSplit split) {
  constexpr int D = 128, QB = C::kQB, KB = C::kKB, KS = C::kKS, DB = C::kDB, KBLK = C::kKBLK;
  constexpr int CH = C::kChunks, TB = C::kTileBytes;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  float dq = 1.f, dk = 1.f, dv = 1.f;
  if (descale != nullptr) { dq = descale[0]; dk = descale[1]; dv = descale[2]; }
  const float c_log2 = scale_log2 * dq * dk;       // raw fp8 dot -> log2 units

  const int n_kt = (N + KB - 1) / KB;
  // query tile and key-tile range [kt0, kt1) of this workgroup
  int tile, kt0 = 0, kt1 = n_kt, ws_index = -1;
  if ((int)blockIdx.x < split.n_full) {
    tile = xcd_remap(blockIdx.x, split.n_full);
  } else {
    const int sidx = xcd_remap(blockIdx.x - split.n_full, gridDim.x - split.n_full);
    const int part = sidx / split.n_split;
    const int ti = sidx - part * split.n_split;
    tile = split.n_full + ti;
    kt0 = part * n_kt / split.parts;
    kt1 = (part + 1) * n_kt / split.parts;
    ws_index = part * split.n_split + ti;
  }
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint8_t* Q = Qg + base;
  const uint8_t* K = Kg + base;
  const uint8_t* V = Vg + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * C::kBR + wave * QB * 32;

  // ---- Q^T fragments: lane holds query q0+qb*32+l32, d = ks*64 + hh*32 .. +31
  i32x8_t qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4_t a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      if (row < N) {
        const uint8_t* p = Q + (size_t)row * D + ks * 64 + hh * 32;
        a = *(const i32x4_t*)p;
        b = *(const i32x4_t*)(p + 16);
      }
      qf[qb][ks] = i32x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
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

  i32x4_t stK[C::kLoadsPerThread], stV[C::kLoadsPerThread];
  auto load_tile = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::kLoadsPerThread; ++i) {
      const int ci = tid + i * C::kThreads;
      const int r = ci / CH, c = ci % CH;
      const int key = kt * KB + r;
      if (key < N) {
        stK[i] = *(const i32x4_t*)(K + (size_t)key * D + c * 16);
        stV[i] = *(const i32x4_t*)(V + (size_t)key * D + c * 16);
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
      *(i32x4_t*)(kb + swz8_k(r, c)) = stK[i];
      *(i32x4_t*)(vb + swz8_v(r, c)) = stV[i];
    }
  };

  load_tile(kt0);
  store_tile(0);
  __syncthreads();

  // V^T gather: lane pair (gi>>1) addresses key slot e = gi>>1 of an 8-key read
  const int g = lane >> 4, gi = lane & 15;
  const int tr_e = gi >> 1;
  const int tr_key = (tr_e >> 2) * 8 + (g >> 1) * 4 + (tr_e & 3);   // key offset within a 16-key step
  const int tr_chunk = g & 1;                                          // chunk within a 32-wide d block
  const int tr_off = (gi & 1) * 8;

  for (int kt = kt0; kt < kt1; ++kt) {
    const int buf = (kt - kt0) & 1;
    const bool has_next = kt + 1 < kt1;
    if (has_next) load_tile(kt + 1);
    const char* kbuf = smem + buf * 2 * TB;
    const char* vbuf = kbuf + TB;

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
        const i32x4_t a0 = *(const i32x4_t*)(kbuf + swz8_k(r, ks * 4 + hh * 2));
        const i32x4_t a1 = *(const i32x4_t*)(kbuf + swz8_k(r, ks * 4 + hh * 2 + 1));
        const i32x8_t a = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[qb][ks], s[kb][qb],
                                                                      0, 0, 0, 0, 0, 0);
      }
    }

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
      grow |= (m_new[qb] - m_run[qb]) * c_log2 > kTauFp8;
    }
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float alpha = fast_exp2((m_run[qb] - m_new[qb]) * c_log2);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
        m_run[qb] = m_new[qb];
      }
    }

    // P^T as e4m3: 64 keys per MFMA step, slot = kb*16 + r of the S^T accumulators
    i32x8_t pb[KBLK / 2][QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float mc = m_run[qb] * c_log2 - kPScaleLog2Fp8;   // p scaled by 16
      float ls = 0.f;
#pragma unroll
      for (int kp = 0; kp < KBLK / 2; ++kp) {
        i32x8_t w;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const int kb = kp * 2 + (t >> 2);
          float p[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            p[e] = fast_exp2(fmaf(s[kb][qb][(t & 3) * 4 + e], c_log2, -mc));
            ls += p[e];
          }
          w[t] = (int)pack_e4m3x4(p[0], p[1], p[2], p[3]);
        }
        pb[kp][qb] = w;
      }
      l_run[qb] += ls;
    }

#pragma unroll
    for (int kp = 0; kp < KBLK / 2; ++kp)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        i32x8_t a;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int key = kp * 64 + (u >> 1) * 32 + (u & 1) * 16 + tr_key;
          const int c = db * 2 + tr_chunk;
          const i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
              DIT_LDS(i32x2_t, vbuf + swz8_v(key, c) + tr_off));
          a[2 * u] = t[0];
          a[2 * u + 1] = t[1];
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb[kp][qb], acc[qb][db],
                                                                        0, 0, 0, 0, 0, 0);
      }

    if (has_next) store_tile(buf ^ 1);
    __syncthreads();
  }

  // l_run sums 16 p, and so does acc: their ratio needs no further scaling
  if (ws_index >= 0) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float l_tot = pair_sum(l_run[qb]);
      const float mul = dv / l_tot;
      const int r = wave * QB * 32 + qb * 32 + l32;
      float* orow = split.ws_o + ((size_t)ws_index * C::kBR + r) * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + i * 8 + hh * 4;
          f32x4_t w = {acc[qb][db][i * 4 + 0] * mul, acc[qb][db][i * 4 + 1] * mul, acc[qb][db][i * 4 + 2] * mul,
                       acc[qb][db][i * 4 + 3] * mul};
          *(f32x4_t*)(orow + d0) = w;
        }
      if (hh == 0)
        split.ws_lse[(size_t)ws_index * C::kBR + r] = m_run[qb] * c_log2 + __log2f(l_tot) - kPScaleLog2Fp8;
    }
    return;
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    const float mul = dv / l_tot;
    const int row = q0 + qb * 32 + l32;
    if (row < N) {
      uint16_t* orow = Og + base + (size_t)row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + i * 8 + hh * 4;
          uint2 w;
          w.x = pack_bf16x2(acc[qb][db][i * 4 + 0] * mul, acc[qb][db][i * 4 + 1] * mul);
          w.y = pack_bf16x2(acc[qb][db][i * 4 + 2] * mul, acc[qb][db][i * 4 + 3] * mul);
          *(uint2*)(orow + d0) = w;
        }
      if (LSEg != nullptr && hh == 0)
        LSEg[(size_t)bh * N + row] = (m_run[qb] * c_log2 + __log2f(l_tot) - kPScaleLog2Fp8) * 0.6931471805599453f;
    }
  }
}

}  // namespace ditattn
