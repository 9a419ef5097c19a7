// bf16 attention forward for gfx950, software-pipelined, 64 query rows per wave.
//
// Why this shape. An MFMA operand read from LDS is reused once per 32-row
// query block that the wave owns, so the LDS bytes read per flop fall as the
// rows per wave grow. With 64 rows per wave (two 32-row blocks) the O
// accumulator alone is 128 registers per lane, so one wave runs per SIMD and
// the wave itself must keep the matrix cores busy. The loop is therefore
// software-pipelined and explicitly interleaved:
//
// Iteration j (one tile of 32 keys) starts with S_j and its row maxima in
// registers, K_{j+1} and V_j in LDS:
//   [rare] raise the running maximum and rescale O, l
//   read all K_{j+1} and V_j MFMA fragments from LDS (latency hidden by the
//   first steps below); issue global loads of K_{j+2} and V_{j+1}
//   phase A, one step per 16-wide d slice:  2 MFMAs of S_{j+1} = K_{j+1} Q^T
//                                           + softmax of keys 0-15 of S_j
//   phase B1, one step per 32-wide d block: 2 MFMAs of O^T += V_j^T P_j^T
//                                           (keys 0-15) + softmax of keys 16-31
//   phase B2, one step per 32-wide d block: 2 MFMAs (keys 16-31)
//                                           + row maxima of S_{j+1}
//   store K_{j+2}, V_{j+1} to LDS; barrier
// Each step is fenced with a scheduling barrier, so the compiler keeps the
// matrix-core and vector-ALU work of a step next to each other instead of
// grouping all MFMAs and all VALU work. K_{j+2} overwrites K_j (last read in
// iteration j-1) and V_{j+1} overwrites V_{j-1} (also read in iteration
// j-1), so one barrier per tile suffices. The last two iterations are peeled
// so the steady-state body has no branch other than the rare rescale.
//
// Layout conventions (S^T = K Q^T, O^T = V^T P^T, V^T via LDS transpose
// reads, lazy rescaling) are those of the 32-row kernel in attn_fwd_bf16.h.
// Built with -mllvm -amdgpu-mfma-vgpr-form so that the accumulators stay in
// VGPRs and the rescale does not copy them between register files.
#pragma once
#include <type_traits>

#include "attn_common.h"
#include "attn_fwd_bf16.h"

namespace ditattn {

template <int D, int NW, int VSWZ = 2>
struct PipeCfg {
  static constexpr int kD = D, kNW = NW, kKB = 32, kQB = 2, kVSwz = VSWZ;
  static constexpr int kThreads = NW * 64;
  static constexpr int kBR = NW * 64;
  static constexpr int kKS = D / 16;
  static constexpr int kDB = D / 32;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunks = kRowBytes / 16;
  static constexpr int kTileBytes = kKB * kRowBytes;
  static constexpr int kLdsBytes = 2 * 2 * kTileBytes;
  static constexpr int kLoadsPerThread = kKB * kChunks / kThreads;
  static_assert(kKB * kChunks % kThreads == 0, "tile chunks must split evenly over the workgroup");
  static_assert(8 % kKS == 0 && 8 % kDB == 0, "softmax slices must split evenly over the steps");
};

template <bool B>
using flag_t = std::integral_constant<bool, B>;

// Keep the instructions of one pipeline step together.
#define DIT_STEP_FENCE() __builtin_amdgcn_sched_barrier(0)

template <class C>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_bf16_pipe_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                               const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                               float* __restrict__ LSEg, int N, int n_qtiles, float scale_log2, float scale) {
  constexpr int D = C::kD, QB = 2, KB = C::kKB, KS = C::kKS, DB = C::kDB;
  constexpr int CH = C::kChunks, TB = C::kTileBytes, LPT = C::kLoadsPerThread;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  char* const kbuf0 = smem;               // K tiles: [2][TB]
  char* const vbuf0 = smem + 2 * TB;      // V tiles: [2][TB]

  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const size_t base = (size_t)bh * (size_t)N * D;
  const uint16_t* Q = Qg + base;
  const uint16_t* K = Kg + base;
  const uint16_t* V = Vg + base;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * C::kBR + wave * 64;

  bf16x8_t qf[QB][KS];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4_t raw = {0, 0, 0, 0};
      if (row < N) raw = *(const i32x4_t*)(Q + (size_t)row * D + ks * 16 + hh * 8);
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
  float m_run[QB] = {-INFINITY, -INFINITY}, l_run[QB] = {0.f, 0.f};
  float m_cur[QB];          // row maxima of the tile in s_cur

  const int n_kt = (N + KB - 1) / KB;

  // ---- global -> register staging (rows past N read row N-1: they are masked or weighted 0)
  auto gload = [&](const uint16_t* src, int kt, i32x4_t (&st)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ci = tid + i * C::kThreads;
      const int r = ci / CH, c = ci % CH;
      const int key = min(kt * KB + r, N - 1);
      st[i] = *(const i32x4_t*)(src + (size_t)key * D + c * 8);
    }
  };
  auto lstore_k = [&](char* dst, const i32x4_t (&st)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ci = tid + i * C::kThreads;
      *(i32x4_t*)(dst + swz<CH>(ci / CH, ci % CH)) = st[i];
    }
  };
  auto lstore_v = [&](char* dst, const i32x4_t (&st)[LPT]) {
#pragma unroll
    for (int i = 0; i < LPT; ++i) {
      const int ci = tid + i * C::kThreads;
      *(i32x4_t*)(dst + swz_v<CH, C::kVSwz>(ci / CH, ci % CH)) = st[i];
    }
  };
  auto read_kfrags = [&](const char* kb_lds, bf16x8_t (&kf)[KS]) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      kf[ks] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(kb_lds + swz<CH>(l32, ks * 2 + hh)));
  };

  const int g = lane >> 4, gi = lane & 15;
  const int tr_row = (g >> 1) * 4 + (gi >> 2);
  const int tr_chunk = (g & 1) * 2 + ((gi & 3) >> 1);
  const int tr_off = (gi & 1) * 8;
  auto read_vfrags = [&](const char* vb, bf16x8_t (&vf)[2][DB]) {
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int rbase = half * 16 + tr_row;
        const int c = db * 4 + tr_chunk;
        const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            DIT_LDS(i16x4_t, (vb + swz_v<CH, C::kVSwz>(rbase, c) + tr_off)));
        const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            DIT_LDS(i16x4_t, (vb + swz_v<CH, C::kVSwz>(rbase + 8, c) + tr_off)));
        const i32x2_t lo2 = __builtin_bit_cast(i32x2_t, lo), hi2 = __builtin_bit_cast(i32x2_t, hi);
        const i32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
        vf[half][db] = __builtin_bit_cast(bf16x8_t, a4);
      }
  };
  auto mask_tail = [&](int kt, f32x16_t (&s)[QB]) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * KB + (r >> 2) * 8 + hh * 4 + (r & 3);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb][r] = key < N ? s[qb][r] : -INFINITY;
    }
  };

  i32x4_t stK[LPT], stV[LPT];
  // ---- prologue: K_0, V_0 -> buffer 0, K_1 -> buffer 1; S_0 and its row maxima
  gload(K, 0, stK);
  gload(V, 0, stV);
  lstore_k(kbuf0, stK);
  lstore_v(vbuf0, stV);
  if (n_kt > 1) {
    gload(K, 1, stK);
    lstore_k(kbuf0 + TB, stK);
  }
  __syncthreads();
  f32x16_t s_cur[QB];
  {
    bf16x8_t kf[KS];
    read_kfrags(kbuf0, kf);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s_cur[qb][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s_cur[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[qb][ks], s_cur[qb], 0, 0, 0);
    }
  }
  if (n_kt == 1) mask_tail(0, s_cur);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    float m = s_cur[qb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, s_cur[qb][r]);
    m_cur[qb] = pair_max(m);
  }
  __syncthreads();

  // One pipelined iteration. NEXT: compute S_{kt+1}; MASK: it is the last tile and
  // may be partial; LOADK / LOADV: fetch K_{kt+2} / V_{kt+1}.
  auto iteration = [&](int kt, auto next_t, auto mask_t, auto loadk_t, auto loadv_t) {
    constexpr bool NEXT = decltype(next_t)::value, MASK = decltype(mask_t)::value;
    constexpr bool LOADK = decltype(loadk_t)::value, LOADV = decltype(loadv_t)::value;

    // [rare] the running maximum grows by more than TAU: rescale O and l
    bool grow = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) grow |= (m_cur[qb] - m_run[qb]) * scale_log2 > kTauBf16;
    if (__builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float m_new = fmaxf(m_run[qb], m_cur[qb]);
        const float alpha = fast_exp2((m_run[qb] - m_new) * scale_log2);
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
        m_run[qb] = m_new;
      }
    }
    DIT_STEP_FENCE();

    // fragment reads for this iteration, then the global loads of later tiles
    bf16x8_t kf[KS];
    if constexpr (NEXT) read_kfrags(kbuf0 + ((kt + 1) & 1) * TB, kf);
    bf16x8_t vf[2][DB];
    read_vfrags(vbuf0 + (kt & 1) * TB, vf);
    if constexpr (LOADK) gload(K, kt + 2, stK);
    if constexpr (LOADV) gload(V, kt + 1, stV);
    DIT_STEP_FENCE();

    const float mc0 = m_run[0] * scale_log2, mc1 = m_run[1] * scale_log2;
    float ls0 = 0.f, ls1 = 0.f;
    float p[QB][16];
    auto softmax_slice = [&](int r0, int nr) {
#pragma unroll
      for (int r = r0; r < r0 + nr; ++r) {
        p[0][r] = fast_exp2(fmaf(s_cur[0][r], scale_log2, -mc0));
        p[1][r] = fast_exp2(fmaf(s_cur[1][r], scale_log2, -mc1));
        ls0 += p[0][r];
        ls1 += p[1][r];
      }
    };
    auto pack_p = [&](int half, bf16x8_t (&pb)[QB]) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        bf16x8_t v;
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] = (__bf16)p[qb][half * 8 + e];
        pb[qb] = v;
      }
    };

    // ---- phase A: S_{j+1} (MFMA) with the softmax of keys 0-15 of S_j (VALU)
    f32x16_t s_nxt[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s_nxt[qb][r] = 0.f;
    constexpr int kSliceA = 8 / KS;      // elements per qb per phase-A step (keys 0-15: regs 0-7)
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if constexpr (NEXT) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s_nxt[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[qb][ks], s_nxt[qb], 0, 0, 0);
      }
      softmax_slice(ks * kSliceA, kSliceA);
      DIT_STEP_FENCE();
    }
    bf16x8_t pb0[QB], pb1[QB];
    pack_p(0, pb0);

    // ---- phase B1: O^T += V^T P^T for keys 0-15 (MFMA) with the softmax of keys 16-31
    constexpr int kSliceB = 8 / DB;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0][db], pb0[qb], acc[qb][db], 0, 0, 0);
      softmax_slice(8 + db * kSliceB, kSliceB);
      DIT_STEP_FENCE();
    }
    pack_p(1, pb1);
    l_run[0] += ls0;
    l_run[1] += ls1;

    // ---- phase B2: keys 16-31 (MFMA) with the row maxima of S_{j+1} (VALU)
    if constexpr (NEXT && MASK) mask_tail(kt + 1, s_nxt);
    float mx0 = -INFINITY, mx1 = -INFINITY;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
        acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1][db], pb1[qb], acc[qb][db], 0, 0, 0);
      if constexpr (NEXT) {
        constexpr int kSliceM = 16 / DB;
#pragma unroll
        for (int r = db * kSliceM; r < (db + 1) * kSliceM; ++r) {
          mx0 = fmaxf(mx0, s_nxt[0][r]);
          mx1 = fmaxf(mx1, s_nxt[1][r]);
        }
      }
      DIT_STEP_FENCE();
    }
    if constexpr (NEXT) {
      m_cur[0] = pair_max(mx0);
      m_cur[1] = pair_max(mx1);
      s_cur[0] = s_nxt[0];
      s_cur[1] = s_nxt[1];
    }
    if constexpr (LOADK) lstore_k(kbuf0 + (kt & 1) * TB, stK);
    if constexpr (LOADV) lstore_v(vbuf0 + ((kt + 1) & 1) * TB, stV);
    __syncthreads();
  };

  using T = flag_t<true>;
  using F = flag_t<false>;
  int kt = 0;
  for (; kt + 2 < n_kt; ++kt) iteration(kt, T{}, F{}, T{}, T{});
  if (kt + 1 < n_kt) {          // second to last: S of the last tile, which may be partial
    iteration(kt, T{}, T{}, F{}, T{});
    ++kt;
  }
  iteration(kt, F{}, F{}, F{}, F{});

#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l_tot = pair_sum(l_run[qb]);
    const float inv = 1.0f / l_tot;
    const int row = q0 + qb * 32 + l32;
    if (row < N) {
      uint16_t* orow = Og + base + (size_t)row * D;
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
      if (LSEg != nullptr && hh == 0) LSEg[(size_t)bh * N + row] = m_run[qb] * scale + logf(l_tot);
    }
  }
}

#undef DIT_STEP_FENCE

}  // namespace ditattn
