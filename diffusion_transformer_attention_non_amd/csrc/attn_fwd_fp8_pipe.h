// fp8-e4m3 attention forward for gfx950, d = 128, bf16 out: 64 query rows per
// wave, software-pipelined, K/V tiles moved by LDS DMA.
//
// The structure follows attn_fwd_bf16_pipe.h (one wave per SIMD, 4 waves and
// 256 rows per workgroup, K in a ring of 4 LDS slots and V in a ring of 3,
// filled two tiles ahead by buffer_load ... lds, one barrier per tile, the
// running maximum moved only on a rare path, key-range split of the last
// round). What differs for e4m3:
// * both products run on the 32x32x64 f8f6f4 MFMA in its e4m3 x e4m3 form, so
//   a sub-tile is 64 keys (the k extent of the PV product) and an LDS tile 128;
// * K rows are 128 bytes padded to 144 (conflict-free ds_read_b128, additive
//   addresses); V rows keep 128 bytes with a transpose-read-aware XOR swizzle,
//   which the DMA applies by choosing each lane's source chunk. LDS serves
//   256 bytes (64 four-byte banks) per pass, so two 128-byte rows share a
//   pass; a ds_read_b64_tr_b8 pass covers rows {0-3, 8-11} (+4) and two
//   neighbouring 16-byte chunks c, c+1 (c even), and the 4 rows of each
//   parity need {c ^ f, c ^ f ^ 1} disjoint: chunk c of row r is stored at
//   c ^ f(r), f(r) = 2 ((r >> 1) & 1) + 4 ((r >> 3) & 1). V^T fragments come
//   from ds_read_b64_tr_b8 and P^T is packed from the S^T accumulators in the
//   matching key order;
// * probabilities are scaled by 2 before the e4m3 cast (the factor is added
//   to the exponent argument): p down to 2^-7 of the running maximum stays
//   in the normal e4m3 range (2 p >= 2^-6), and p up to 232 times it fits (the maximum of
//   the first sub-tile is usually a few bits below the row's). A power of
//   two cancels in O. The row sums are those of the e4m3 values,
//   taken on the matrix core (the output's denominator; the exact sums for
//   the log-sum-exp are fp32 adds, only in the EXACT_LSE form). The cast does
//   not saturate: past 464 (p > 232 relative to the running maximum) it gives
//   the e4m3 NaN, which makes the half-row sum NaN; that sends the sub-tile
//   down the rare path, which recomputes its logits from K in LDS, takes their
//   exact maximum and rescales. Large but representable p take no detour;
// * per-tensor descales dq, dk fold into the logit multiplier and dv into the
//   epilogue.
// Sub-iteration j (64 keys), two phases of 8 MFMAs each:
//   X: O^T += V_{j-1}^T P_{j-1}^T, with the softmax of S_j's first query block;
//      the K_{j+1} fragment reads are issued first.
//   Y: S_{j+1} = K_{j+1} Q^T, with the softmax of S_j's second query block (each
//      block of S_j is overwritten once consumed), the V_j fragment reads and
//      the tile DMA.
#pragma once
#include "attn_common.h"
#include "attn_fwd_bf16_pipe.h"   // dma_b128, flag_t, PipeSplit

namespace ditattn {

struct Fp8PipeCfg {
  static constexpr int kD = 128, kNW = 4, kThreads = 256, kBR = 256;
  static constexpr int kKRow = 144;                        // K row pitch in LDS: 128 bytes + 16 padding
  static constexpr int kTileKeys = 128;                    // keys per LDS tile (two 64-key sub-tiles)
  static constexpr int kKB = kTileKeys;                    // key-tile size for the split planner
  static constexpr int kKTile = kTileKeys * kKRow;         // 18432
  static constexpr int kVTile = kTileKeys * 128;           // 16384
  static constexpr int kDmaPerWave = 5;                    // 20 x 1 KB instructions per tile and tensor
  static constexpr int kSlot = kNW * kDmaPerWave * 1024;   // 20480
  static constexpr int kKSlots = 4, kVSlots = 3;
  static constexpr int kVBase = kKSlots * kSlot;
  static constexpr int kLdsBytes = kVBase + kVSlots * kSlot;   // 143360
  static_assert(kKTile <= kSlot && kVTile <= kSlot, "tile fits its slot");
  static constexpr int kORow = 272;                        // O staging pitch, as in the bf16 kernel
  static_assert(kNW * 64 * kORow <= kLdsBytes, "O staging fits the slots");
};

constexpr float kFp8PipePLog2 = 1.0f;          // P is scaled by 2 before the cast

#define DIT_FENCE() __builtin_amdgcn_sched_barrier(0)

// O^T += V^T P^T with the accumulator held in AGPRs. The builtin form would keep
// it in VGPRs, where its 128 registers per lane push the logits out to AGPR
// copies. The compiler does not model this instruction's latency: the
// accumulator's AGPRs are read by the VALU only after pv_drain(...) or after a
// full phase of other work, and its VGPR sources are not rewritten for a
// whole sub-iteration after issue.
__device__ __forceinline__ void pv_mfma(f32x16_t& acc, const i32x8_t& v, const i32x8_t& p) {
  asm("v_mfma_f32_32x32x64_f8f6f4 %0, %1, %2, %0" : "+a"(acc) : "v"(v), "v"(p));
}
// 32 wait states: more than a 16-pass MFMA needs before its result is read.
// The accumulators pass through it ("+a") and the products' sources are its
// inputs: otherwise the compiler may hoist it above the (non-volatile)
// products, read an accumulator right after the product that writes it, or
// reuse a source register while the product still runs.
__device__ __forceinline__ void pv_drain(f32x16_t (&acc)[2][4], const i32x8_t (&vf)[4], const i32x8_t (&p)[2],
                                         int sv, int sp) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
               : "+a"(acc[0][0]), "+a"(acc[0][1]), "+a"(acc[0][2]), "+a"(acc[0][3]), "+a"(acc[1][0]),
                 "+a"(acc[1][1]), "+a"(acc[1][2]), "+a"(acc[1][3])
               : "v"(vf[0]), "v"(vf[1]), "v"(vf[2]), "v"(vf[3]), "v"(p[0]), "v"(p[1]), "v"(sv), "v"(sp)
               : "memory");
}

// Block scales of the MX form, E8M0 bytes (value 2^(byte - 127)). q and k:
// one 32-bit word per row, byte j = d block j (d = 32 j .. 32 j + 31). v:
// [B*H][ceil(N/32)][32] words per 32-token block, byte j of word i = column
// 32 j + i.
struct MxScales {
  const uint8_t* q;
  const uint8_t* k;
  const uint8_t* v;
};

// The scaled 32x32x64 e4m3 MFMA. Lane l supplies one scale word per operand;
// byte OA (OB) of it scales row (column) l % 32 over k-block l / 32, and
// k-block b is bytes 16 b .. 16 b + 15 of the operand in both lane halves
// (k = 16 h + 0..15 in half h's bytes 0-15, 32 + 16 h + 0..15 in bytes 16-31).
template <int OA, int OB>
__device__ __forceinline__ f32x16_t mfma_mx_t(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OA, sa, OB, sb);
}
// oa, ob are constants once the caller's loops are unrolled
__device__ __forceinline__ f32x16_t mfma_mx(const i32x8_t& a, const i32x8_t& b, const f32x16_t& c, int sa, int oa,
                                            int sb, int ob) {
  switch (oa * 4 + ob) {
#define DIT_MX_CASE(A, B) \
  case A * 4 + B:         \
    return mfma_mx_t<A, B>(a, b, c, sa, sb);
    DIT_MX_CASE(0, 0) DIT_MX_CASE(0, 1) DIT_MX_CASE(0, 2) DIT_MX_CASE(0, 3)
    DIT_MX_CASE(1, 0) DIT_MX_CASE(1, 1) DIT_MX_CASE(1, 2) DIT_MX_CASE(1, 3)
    DIT_MX_CASE(2, 0) DIT_MX_CASE(2, 1) DIT_MX_CASE(2, 2) DIT_MX_CASE(2, 3)
    DIT_MX_CASE(3, 0) DIT_MX_CASE(3, 1) DIT_MX_CASE(3, 2) default: return mfma_mx_t<3, 3>(a, b, c, sa, sb);
#undef DIT_MX_CASE
  }
}
// DMA instruction 4 of a K tile in the MX form: waves 0 and 1 (b32 == 0) move
// K rows (16 bytes per lane); waves 2 and 3 move the tile's K scale words, 4
// bytes per lane to M0 + 4 lane, so that the range check at the end of the
// scale array works per word (a 16-byte chunk that straddles the end comes
// back as zeros). The instruction is chosen inside one asm block: b32 is
// uniform, and a branch in the C++ would split the scheduling region.
__device__ __forceinline__ void dma_k4_mx(i32x4_t rsrc, int voffset, unsigned lds_addr, int b32) {
  asm volatile(
      "s_cmp_eq_u32 %3, 0\n\t"
      "s_cbranch_scc1 1f\n\t"
      "buffer_load_dword %0, %1, 0 offen lds\n\t"
      "s_branch 2f\n"
      "1:\n\t"
      "buffer_load_dwordx4 %0, %1, 0 offen lds\n"
      "2:" ::"v"(voffset), "s"(rsrc), "{m0}"(lds_addr), "s"(b32)
      : "memory", "scc");
}

// pv_mfma with block scales: byte oa of sv for V^T, byte 0 of sp for P^T
__device__ __forceinline__ void pv_mfma_mx(f32x16_t& acc, const i32x8_t& v, const i32x8_t& p, int sv, int sp,
                                           int oa) {
  switch (oa) {
    case 0:
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[0,0,0]"
          : "+a"(acc) : "v"(v), "v"(p), "v"(sv), "v"(sp));
      break;
    case 1:
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,0,0] op_sel_hi:[0,0,0]"
          : "+a"(acc) : "v"(v), "v"(p), "v"(sv), "v"(sp));
      break;
    case 2:
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel_hi:[1,0,0]"
          : "+a"(acc) : "v"(v), "v"(p), "v"(sv), "v"(sp));
      break;
    default:
      asm("v_mfma_scale_f32_32x32x64_f8f6f4 %0, %1, %2, %0, %3, %4 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
          : "+a"(acc) : "v"(v), "v"(p), "v"(sv), "v"(sp));
      break;
  }
}

// EXACT_LSE: the caller wants the log-sum-exp; it is then summed from the
// unrounded fp32 probabilities as well (the output is normalised by the sums
// of the e4m3 values in both forms).
// MX: block-scaled inputs (scales in mxs, descale unused). Q and K fragments
// then hold d in the MFMA's k order (so that each k-block is one 32-wide d
// block), K scales ride in the K slot past the rows (in place of the two DMA
// instructions that would only zero-fill there) and V scales in a fifth V
// DMA instruction; both products use the scaled MFMA.
template <class C, bool EXACT_LSE, bool MX = false>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_fp8_pipe_kernel(const uint8_t* __restrict__ Qg, const uint8_t* __restrict__ Kg,
                              const uint8_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                              float* __restrict__ LSEg, const float* __restrict__ descale,
                              int N, int n_qtiles, float scale_log2, float scale, PipeSplit split, Layout L,
                              MxScales mxs = MxScales{nullptr, nullptr, nullptr}) {
  constexpr int D = C::kD, KROW = C::kKRow;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  float dq = 1.f, dk = 1.f, dv = 1.f;
  if (descale != nullptr) { dq = descale[0]; dk = descale[1]; dv = descale[2]; }
  const float c_log2 = scale_log2 * dq * dk;          // raw fp8 dot -> log2 units

  const int n_t = (N + C::kTileKeys - 1) / C::kTileKeys;
  int tile, u0 = 0, u1 = n_t, ws_index = -1;
  if ((int)blockIdx.x < split.n_full) {
    tile = xcd_remap(blockIdx.x, split.n_full);
  } else {
    const int sidx = xcd_remap(blockIdx.x - split.n_full, gridDim.x - split.n_full);
    const int part = sidx / split.n_split;
    const int ti = sidx - part * split.n_split;
    tile = split.n_full + ti;
    u0 = part * n_t / split.parts;
    u1 = (part + 1) * n_t / split.parts;
    ws_index = part * split.n_split + ti;
  }
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  const long long ibase = L.in_off(bh), obase = L.out_off(bh);
  const int rowb = (int)L.qn;             // bytes between consecutive tokens of q, k, v
  const char* Kh = reinterpret_cast<const char*>(Kg + ibase);
  const char* Vh = reinterpret_cast<const char*>(Vg + ibase);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * C::kBR + wave * 64;

  // Q^T fragments: query q0 + qb*32 + l32, d = ks*64 + hh*32 .. +31 (MX:
  // d = ks*64 + hh*16 .. +15 and ks*64 + 32 + hh*16 .. +15, the MFMA's k order)
  i32x8_t qf[2][2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      i32x4_t a = {0, 0, 0, 0}, b = {0, 0, 0, 0};
      if (row < N) {
        const uint8_t* p = Qg + ibase + (long long)row * L.qn + ks * 64;
        a = *(const i32x4_t*)(p + (MX ? hh * 16 : hh * 32));
        b = *(const i32x4_t*)(p + (MX ? 32 + hh * 16 : hh * 32 + 16));
      }
      qf[qb][ks] = i32x8_t{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
    }
  }
  // MX scale words of this lane: byte 2 x + ks = row block x (query block or
  // key block), d block 2 ks + hh; v_perm picks those bytes of two row words
  const int sc_sel = hh ? 0x07050301 : 0x06040200;
  int qsc = 0;
  if constexpr (MX) {
    int w[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int row = q0 + qb * 32 + l32;
      w[qb] = row < N ? *(const int*)(mxs.q + ((size_t)bh * N + row) * 4) : 0;
    }
    qsc = __builtin_amdgcn_perm(w[1], w[0], sc_sel);
  }

  // ---- DMA lane offsets: instruction i writes LDS bytes [1024 i, 1024 i + 1024)
  // of a slot; lane L covers 16-byte slot s = 64 i + L
  int kdo[C::kDmaPerWave], vdo[C::kDmaPerWave];
#pragma unroll
  for (int m = 0; m < C::kDmaPerWave; ++m) {
    const int s = 64 * (wave + 4 * m) + lane;
    const int kr = s / (KROW / 16), kc = s % (KROW / 16);
    kdo[m] = (kc < 8 && kr < C::kTileKeys) ? kr * rowb + kc * 16 : C::kTileKeys * rowb;   // past the tile: zeros
    const int vr = s >> 3, vs = s & 7;
    const int vc = vs ^ ((((vr >> 1) & 1) << 1) | (((vr >> 3) & 1) << 2));    // f(vr) is its own inverse
    vdo[m] = vr < C::kTileKeys ? vr * rowb + vc * 16 : C::kTileKeys * rowb;
  }
  // buffer descriptor of `rows` rows from address a: the range check
  // zero-fills rows past them. Descriptors of tiles past the end are built
  // but never read. Every field comes from the scalar unit: the inline-asm
  // DMA reads it with no wait states of the compiler's in between.
  auto make_rsrc = [&](unsigned long long a, int rows) __attribute__((always_inline)) {
    i32x4_t rs;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
    rs[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));   // stride 0
    rs[2] = __builtin_amdgcn_readfirstlane(min(C::kTileKeys, rows) * rowb);
    rs[3] = 0x00020000;
    return rs;
  };
  auto tile_rsrc = [&](const char* head, int t) __attribute__((always_inline)) {
    return make_rsrc((unsigned long long)(head + (long long)t * C::kTileKeys * rowb), N - t * C::kTileKeys);
  };
  // MX: instruction 4 of waves 2 and 3 (LDS bytes 18432.. and 19456.. of a K
  // slot) carries the tile's K scale words of keys 0-63 and 64-127, that of
  // every wave (16384.. of a V slot) its four V scale blocks; lanes past the
  // data zero-fill
  auto bytes_rsrc_at = [&](unsigned long long a, int bytes) __attribute__((always_inline)) {
    i32x4_t rs;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
    rs[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));
    rs[2] = __builtin_amdgcn_readfirstlane(max(bytes, 0));
    rs[3] = 0x00020000;
    return rs;
  };
  auto bytes_rsrc = [&](const uint8_t* base, long long off, int bytes) __attribute__((always_inline)) {
    return bytes_rsrc_at((unsigned long long)(base + off), bytes);
  };
  const int n_vb = (N + 31) / 32;
  auto kscale_rsrc = [&](int t) __attribute__((always_inline)) {
    return bytes_rsrc(mxs.k, ((long long)bh * N + (long long)t * C::kTileKeys) * 4,
                      min(C::kTileKeys, N - t * C::kTileKeys) * 4);
  };
  auto vscale_rsrc = [&](int t) __attribute__((always_inline)) {
    return bytes_rsrc(mxs.v, ((long long)bh * n_vb + (long long)t * 4) * 128, min(4, n_vb - t * 4) * 128);
  };
  if constexpr (MX) {
    static_assert(C::kKTile == 18 * 1024 && C::kVTile == 16 * 1024, "scale DMAs land past the tile rows");
    if (wave >= 2) kdo[4] = (wave - 2) * 256 + lane * 4;
    vdo[4] = wave * 1024 + lane * 16;
  }
  auto dma_one = [&](const i32x4_t& rs, const char* slot, const int (&off)[C::kDmaPerWave], int m)
      __attribute__((always_inline)) {
    const int i = wave + 4 * m;
    dma_b128(rs, off[m], __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)DIT_LDS(const char, slot) + i * 1024));
  };
  auto dma_k4 = [&](const i32x4_t& rs, const char* slot) __attribute__((always_inline)) {
    const int i = wave + 16;
    dma_k4_mx(rs, kdo[4], __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)DIT_LDS(const char, slot) + i * 1024),
              __builtin_amdgcn_readfirstlane(wave >= 2 ? 1 : 0));
  };
  auto dma_tile = [&](const char* head, int t, const char* slot, const int (&off)[C::kDmaPerWave])
      __attribute__((always_inline)) {
    const i32x4_t rs = tile_rsrc(head, t);
#pragma unroll
    for (int m = 0; m < C::kDmaPerWave; ++m) dma_one(rs, slot, off, m);
  };
  auto kslot = [&](int t) { return smem + __builtin_amdgcn_readfirstlane((t % C::kKSlots) * C::kSlot); };
  auto vslot = [&](int t) {
    return smem + __builtin_amdgcn_readfirstlane(C::kVBase + (t % C::kVSlots) * C::kSlot);
  };

  // ---- fragment reads
  const int k_rd = l32 * KROW + (MX ? hh * 16 : hh * 32);
  i32x8_t kf[2][2];                                     // [key block][d step]
  int ksc = 0;                                          // MX: the K scale word (bytes as qsc's)
  // K fragments of sub-tile `odd` (0, 1) of the 128-key tile in `slot`
  auto read_kfrags = [&](const char* slot, int odd) {
    // MX: the scale words are read first, so that their permute waits for
    // them alone (LDS reads complete in order), not for the fragments
    int w0 = 0, w1 = 0;
    if constexpr (MX) {
      const char* sb = slot + C::kKTile + odd * 1024 + l32 * 4;
      w0 = *(const int*)sb;
      w1 = *(const int*)(sb + 128);
    }
    const char* kb = slot + odd * 64 * KROW + k_rd;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const i32x4_t a0 = *(const i32x4_t*)(kb + b * 32 * KROW + ks * 64);
        const i32x4_t a1 = *(const i32x4_t*)(kb + b * 32 * KROW + ks * 64 + (MX ? 32 : 16));
        kf[b][ks] = i32x8_t{a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
      }
    if constexpr (MX) ksc = __builtin_amdgcn_perm(w1, w0, sc_sel);
  };
  // V^T gather (the key order of the P^T packing): lane pair gi>>1 addresses key
  // slot tr_e of an 8-key read; the XOR of the V swizzle depends on key bits
  // 1 and 3, which come from tr_key alone
  const int g = lane >> 4, gi = lane & 15;
  const int tr_e = gi >> 1;
  const int tr_key = (tr_e >> 2) * 8 + (g >> 1) * 4 + (tr_e & 3);
  const int tr_gk = (((tr_key >> 1) & 1) << 1) | (((tr_key >> 3) & 1) << 2);
  int v_rd[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) v_rd[db] = tr_key * 128 + (((2 * db) ^ tr_gk) + (g & 1)) * 16 + (gi & 1) * 8;
  i32x8_t vf[4];                                        // [d block]
  int vsc = 0;                                          // MX: V scale word, byte db = column 32 db + l32
  // V fragments of sub-tile `odd` of the tile in `slot`; half 0: d blocks 0, 1; half 1: 2, 3
  auto read_vfrags = [&](const char* slot, int odd, int half) {
    const char* vb = slot + odd * 64 * 128;
    if constexpr (MX) {
      if (half == 0) vsc = *(const int*)(slot + C::kVTile + (odd * 2 + hh) * 128 + l32 * 4);
    }
#pragma unroll
    for (int db = half * 2; db < half * 2 + 2; ++db) {
      // one lane address per d block; the four reads then differ by constants,
      // which the barrier keeps out of the sum so they land in the offset field
      uint32_t a = (uint32_t)(uintptr_t)DIT_LDS(const char, vb) + (uint32_t)v_rd[db];
      asm volatile("" : "+v"(a));
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const i32x2_t t = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2_t*)(uintptr_t)(a + ((u >> 1) * 32 + (u & 1) * 16) * 128));
        vf[db][2 * u] = t[0];
        vf[db][2 * u + 1] = t[1];
      }
    }
  };
  // keys of sub-tile j past N do not exist
  auto mask_keys = [&](int j, f32x16_t (&s)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = j * 64 + b * 32 + (r >> 2) * 8 + hh * 4 + (r & 3);
        s[b][r] = key < N ? s[b][r] : -INFINITY;
      }
  };
  auto s_chains = [&](int qb, f32x16_t (&s)[2]) {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int r = 0; r < 16; ++r) s[b][r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        if constexpr (MX)
          s[b] = mfma_mx(kf[b][ks], qf[qb][ks], s[b], ksc, 2 * b + ks, qsc, 2 * qb + ks);
        else
          s[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[b][ks], qf[qb][ks], s[b], 0, 0, 0, 0, 0, 0);
      }
    }
  };
  auto row_max = [&](const f32x16_t (&s)[2]) {
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, fmaxf(s[0][r], s[1][r]));
    return pair_max(mx) * c_log2;                     // c_log2 > 0
  };
  // one step of the softmax of one query block: 4 logits -> 8 p, one e4m3 word
  auto soft_step = [&](const f32x16_t (&s)[2], int w, float nm, i32x8_t& pout, float& ls) {
    const int b = w >> 2, r0 = (w & 3) * 4;
    float p[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = fast_exp2(fmaf(s[b][r0 + e], c_log2, nm));
      if constexpr (EXACT_LSE) ls += p[e];
    }
    // both halves of the word are written, so the first conversion may start
    // from any register content (an empty asm stands in for it, saving a clear)
    uint32_t any;
    asm volatile("" : "=v"(any));
    const uint32_t lo = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], any, false);
    pout[w] = (int)__builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], lo, true);
  };
  // Row sums of the e4m3 P^T on the matrix core. Read as the B operand of the
  // 16x16x128 product, lane 16 g + c of a P^T fragment is column c, k-group g;
  // A holds ones exactly where row r meets k-group r, so output row r, column
  // c is the sum of the 32 values in lane 16 r + c. Lanes 0..15 receive rows
  // 0..3: the half-row sums of queries c (rows 0, 2) and c + 16 (rows 1, 3).
  const int p_one = 0x7F7F7F7F;          // MX: scale 2^0 for P^T
  const int ones_w = (lane & 15) == (lane >> 4) ? 0x38383838 : 0;   // e4m3 1.0
  const i32x8_t ones = {ones_w, ones_w, ones_w, ones_w, ones_w, ones_w, ones_w, ones_w};
  auto psum = [&](const i32x8_t& pt) __attribute__((always_inline)) {
    const f32x4_t z = {0.f, 0.f, 0.f, 0.f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(ones, pt, z, 0, 0, 0, 0, 0, 0);
  };

  f32x16_t acc[2][4];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
  float mc[2];                        // running row maxima of the scaled logits, log2 units
  // sums of 8 p in lanes 0..15: query c of each block in l_lo, query c + 16 in l_hi
  float l_lo[2] = {0.f, 0.f}, l_hi[2] = {0.f, 0.f};
  float l_ex[2] = {0.f, 0.f};         // EXACT_LSE: this lane's sums of the unrounded 8 p
  f32x16_t s0[2], s1[2];              // raw logits of the current sub-tile [query block][key block]
  i32x8_t pA[2], pB[2];               // P^T of two consecutive sub-tiles [query block]

  // LDS byte offsets of the ring slots the iteration of tile u uses: K of
  // tiles u, u+1, u+3 and V of u, u+2. They rotate by one slot per iteration
  // (scalar adds instead of a modulo per use).
  struct Ring {
    int k0, k1, k3, v0, v2;
  };
  Ring ring;
  {
    auto rfl = [](int x) { return __builtin_amdgcn_readfirstlane(x); };
    ring.k0 = rfl((u0 % C::kKSlots) * C::kSlot);
    ring.k1 = rfl(((u0 + 1) % C::kKSlots) * C::kSlot);
    ring.k3 = rfl(((u0 + 3) % C::kKSlots) * C::kSlot);
    ring.v0 = rfl(C::kVBase + (u0 % C::kVSlots) * C::kSlot);
    ring.v2 = rfl(C::kVBase + ((u0 + 2) % C::kVSlots) * C::kSlot);
  }
  auto advance_ring = [&]() __attribute__((always_inline)) {
    ring.k3 = ring.k0;
    ring.k0 = ring.k1;
    ring.k1 = ring.k1 == (C::kKSlots - 1) * C::kSlot ? 0 : ring.k1 + C::kSlot;
    ring.v2 = ring.v0;
    ring.v0 = ring.v0 == C::kVBase + (C::kVSlots - 1) * C::kSlot ? C::kVBase : ring.v0 + C::kSlot;
  };

  // ---- prologue: K tiles u0..u0+2, V tiles u0, u0+1; the first sub-tile's logits
  auto dma_ktile = [&](int t) __attribute__((always_inline)) {
    if constexpr (MX) {
      const i32x4_t rs = tile_rsrc(Kh, t);
#pragma unroll
      for (int m = 0; m < 4; ++m) dma_one(rs, kslot(t), kdo, m);
      dma_k4(wave >= 2 ? kscale_rsrc(t) : rs, kslot(t));
    } else {
      dma_tile(Kh, t, kslot(t), kdo);
    }
  };
  auto dma_vtile = [&](int t) __attribute__((always_inline)) {
    if constexpr (MX) {
      const i32x4_t rs = tile_rsrc(Vh, t);
#pragma unroll
      for (int m = 0; m < 4; ++m) dma_one(rs, vslot(t), vdo, m);
      dma_one(vscale_rsrc(t), vslot(t), vdo, 4);
    } else {
      dma_tile(Vh, t, vslot(t), vdo);
    }
  };
  dma_ktile(u0);
  if (u0 + 1 < u1) dma_ktile(u0 + 1);
  if (u0 + 2 < u1) dma_ktile(u0 + 2);
  dma_vtile(u0);
  if (u0 + 1 < u1) dma_vtile(u0 + 1);
  __builtin_amdgcn_s_waitcnt(0x0F70);      // vmcnt(0)
  __syncthreads();
  read_kfrags(kslot(u0), 0);
  s_chains(0, s0);
  s_chains(1, s1);
  if (64 * (2 * u0 + 1) > N) { mask_keys(2 * u0, s0); mask_keys(2 * u0, s1); }
  mc[0] = row_max(s0);
  mc[1] = row_max(s1);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) pA[qb] = i32x8_t{};
#pragma unroll
  for (int db = 0; db < 4; ++db) vf[db] = i32x8_t{};

  // One sub-iteration: consumes P_{j-1} (pin) and S_j (s0, s1); produces P_j
  // (pout) and S_{j+1} (s0, s1), each S block written only after its old
  // values are consumed.
  auto sub = [&](int j, i32x8_t (&pin)[2], i32x8_t (&pout)[2], auto mask_c, auto&& dma)
      __attribute__((always_inline)) {
    constexpr bool MASK = decltype(mask_c)::value;
    f32x4_t rs0, rs1;
    float ls0 = 0.f, ls1 = 0.f;
    // ================= phase X: P_{j-1} V_{j-1}, softmax of S_j block 0
    // the second sub-tile of a tile (j odd) takes the next K tile's first half
    read_kfrags(smem + ((j & 1) ? ring.k1 : ring.k0), (j + 1) & 1);
    DIT_FENCE();
    {
      const float nm0 = kFp8PipePLog2 - mc[0];
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const int db = st >> 1, qb = st & 1;
        if constexpr (MX)
          pv_mfma_mx(acc[qb][db], vf[db], pin[qb], vsc, p_one, db);
        else
          pv_mfma(acc[qb][db], vf[db], pin[qb]);
        soft_step(s0, st, nm0, pout[0], ls0);
        DIT_FENCE();
      }
    }
    // ================= phase Y: S_{j+1}, softmax of S_j block 1
    {
      const float nm1 = kFp8PipePLog2 - mc[1];
      auto smfma = [&](f32x16_t& dst, int b, int qb, int ks) __attribute__((always_inline)) {
        if (ks == 0) {
#pragma unroll
          for (int r = 0; r < 16; ++r) dst[r] = 0.f;
        }
        if constexpr (MX)
          dst = mfma_mx(kf[b][ks], qf[qb][ks], dst, ksc, 2 * b + ks, qsc, 2 * qb + ks);
        else
          dst = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kf[b][ks], qf[qb][ks], dst, 0, 0, 0, 0, 0, 0);
      };
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        if (st < 4) {
          smfma(s0[st >> 1], st >> 1, 0, st & 1);          // block 0 (consumed in phase X)
          if (st == 0) rs0 = psum(pout[0]);
        } else if (st < 6) {
          // words 4-7 of S_j block 1 by step 5, two a step: key block 0 is
          // free after words 0-3 (steps 0-3), key block 1 after these
          soft_step(s1, st, nm1, pout[1], ls1);
          soft_step(s1, st + 2, nm1, pout[1], ls1);
          smfma(s1[0], 0, 1, st - 4);
        } else if (st == 6) {
          // two S MFMAs ahead of the range test that reads these sums
          rs1 = psum(pout[1]);
          DIT_FENCE();
          smfma(s1[1], 1, 1, 0);
        } else {
          smfma(s1[1], 1, 1, 1);
        }
        if (st < 4) soft_step(s1, st, nm1, pout[1], ls1);
        // the V_j fragment reads go behind the first MFMAs (the K fragments
        // were read a phase earlier); 8 at a time, lgkmcnt counts at most 15
        if (st < 2) {
          DIT_FENCE();
          read_vfrags(smem + ring.v0, j & 1, st);
          DIT_FENCE();
        }
        if (st >= 4) dma(st - 4);
        DIT_FENCE();
      }
      if constexpr (MASK) {
        if (64 * (j + 2) > N) { mask_keys(j + 1, s0); mask_keys(j + 1, s1); }
      }
    }
    // The packed P must exist here: without this the compiler sinks the e4m3
    // conversions past the rare-path branch, out of the MFMA phases.
    asm volatile("" ::"v"(pout[0]), "v"(pout[1]));
    // ---- rare path: some p passed the e4m3 range (its NaN made a half-row
    // sum NaN). The sums are >= +0 or NaN, so their bit patterns order like
    // the values, with every NaN above +inf: one unsigned maximum decides.
    auto u = [](float x) { return __float_as_uint(x); };
    const uint32_t big = max(max(max(u(rs0[0]), u(rs0[1])), max(u(rs0[2]), u(rs0[3]))),
                             max(max(u(rs1[0]), u(rs1[1])), max(u(rs1[2]), u(rs1[3]))));
    if (__builtin_amdgcn_ballot_w64(big > 0x7F800000u) != 0) {
      // Recompute S_j from K in LDS into the registers of S_{j+1}, take its
      // exact row maxima, rescale, redo P_j; then recompute S_{j+1}. Reusing
      // those registers keeps this path's working set to one accumulator
      // block, which keeps it from crowding the steady loop's registers.
      DIT_FENCE();
      read_kfrags(smem + ring.k0, j & 1);  // K tiles j/2 and (j+1)/2 are still in their slots
      s_chains(0, s0);
      s_chains(1, s1);
      if constexpr (MASK) {
        if (64 * (j + 1) > N) { mask_keys(j, s0); mask_keys(j, s1); }
      }
      DIT_FENCE();
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const f32x16_t (&s)[2] = qb == 0 ? s0 : s1;
        const float m_new = fmaxf(mc[qb], row_max(s));
        const float alpha = fast_exp2(mc[qb] - m_new);
        l_lo[qb] *= __shfl(alpha, lane & 15);
        l_hi[qb] *= __shfl(alpha, (lane & 15) + 16);
        l_ex[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < 4; ++db) {          // one block at a time, AGPRs to AGPRs
          asm volatile("" : "+a"(acc[qb][db]));
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
          asm volatile("" : "+a"(acc[qb][db]));
          DIT_FENCE();
        }
        mc[qb] = m_new;
        const float nm = kFp8PipePLog2 - m_new;
        float& ls = qb == 0 ? ls0 : ls1;
        ls = 0.f;
#pragma unroll
        for (int w = 0; w < 8; ++w) soft_step(s, w, nm, pout[qb], ls);
        DIT_FENCE();
      }
      rs0 = psum(pout[0]);
      rs1 = psum(pout[1]);
      read_kfrags(smem + ((j & 1) ? ring.k1 : ring.k0), (j + 1) & 1);
      s_chains(0, s0);
      s_chains(1, s1);
      if constexpr (MASK) {
        if (64 * (j + 2) > N) { mask_keys(j + 1, s0); mask_keys(j + 1, s1); }
      }
      DIT_FENCE();
    }
    l_ex[0] += ls0;
    l_ex[1] += ls1;
    l_lo[0] += rs0[0] + rs0[2];
    l_hi[0] += rs0[1] + rs0[3];
    l_lo[1] += rs1[0] + rs1[2];
    l_hi[1] += rs1[1] + rs1[3];
  };

  // One 128-key tile u: streams in K tile u+3 (first sub-iteration) and V tile
  // u+2 (second), one DMA instruction per phase-Y step, then waits for the
  // tiles issued one iteration earlier before the barrier that publishes them.
  // rk, rv: the descriptors of the tiles at u + 3 (K) and u + 2 (V); rk4,
  // rvs: those of the MX scale instructions; before_wait() runs after the
  // compute, ahead of the wait (the next iteration's scalar bookkeeping goes
  // there, behind the last MFMAs in flight).
  auto iteration = [&](int u, auto tail_c, const i32x4_t& rk, const i32x4_t& rv, const i32x4_t& rk4,
                       const i32x4_t& rvs, auto&& before_wait) __attribute__((always_inline)) {
    constexpr bool TAIL = decltype(tail_c)::value;
    const bool k_next = !TAIL || u + 3 < u1, v_next = !TAIL || u + 2 < u1;
    const char* sk = smem + ring.k3;
    const char* sv = smem + ring.v2;
    DIT_FENCE();
    static_assert(C::kDmaPerWave == 5, "DMA hook spreads 5 instructions over 4 steps");
    sub(2 * u, pA, pB, tail_c, [&](int st) __attribute__((always_inline)) {
      if (k_next) {
        dma_one(rk, sk, kdo, st);
        if (st == 0) {
          if constexpr (MX)
            dma_k4(rk4, sk);
          else
            dma_one(rk, sk, kdo, 4);
        }
      }
    });
    sub(2 * u + 1, pB, pA, tail_c, [&](int st) __attribute__((always_inline)) {
      // a V tile is 16 KB: instructions 16-19 (m = 4) would only zero-fill
      // rows that are never read; the MX form sends its scales with them
      if (v_next) {
        dma_one(rv, sv, vdo, st);
        if (MX && st == 0) dma_one(rvs, sv, vdo, 4);
      }
    });
    DIT_FENCE();
    before_wait();
    advance_ring();
    if (TAIL)
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    else if (MX)
      __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10): 5 K and 5 V instructions may stay in flight
    else
      __builtin_amdgcn_s_waitcnt(0x0F79);  // vmcnt(9): this iteration's 9 DMAs (5 K, 4 V) may stay in flight
    __syncthreads();
    DIT_FENCE();
  };
  // the tiles at u + 3 (K) and u + 2 (V): addresses and rows left, and the
  // MX scale blocks' addresses and bytes left, advanced by one tile per
  // iteration
  const unsigned long long tile_bytes = (unsigned long long)C::kTileKeys * rowb;
  unsigned long long ka = (unsigned long long)(Kh + (long long)(u0 + 3) * C::kTileKeys * rowb);
  unsigned long long va = (unsigned long long)(Vh + (long long)(u0 + 2) * C::kTileKeys * rowb);
  int kr = N - (u0 + 3) * C::kTileKeys, vr = N - (u0 + 2) * C::kTileKeys;
  unsigned long long ksa = 0, vsa = 0;
  int vbr = 0;
  if constexpr (MX) {
    ksa = (unsigned long long)(mxs.k + ((long long)bh * N + (long long)(u0 + 3) * C::kTileKeys) * 4);
    vsa = (unsigned long long)(mxs.v + ((long long)bh * n_vb + (long long)(u0 + 2) * 4) * 128);
    vbr = n_vb - (u0 + 2) * 4;
  }
  auto advance = [&]() __attribute__((always_inline)) {
    ka += tile_bytes;
    va += tile_bytes;
    kr -= C::kTileKeys;
    vr -= C::kTileKeys;
    if constexpr (MX) {
      ksa += C::kTileKeys * 4;
      vsa += 4 * 128;
      vbr -= 4;
    }
  };
  auto run = [&](int u, auto tail_c) __attribute__((always_inline)) {
    const i32x4_t rk = make_rsrc(ka, kr), rv = make_rsrc(va, vr);
    i32x4_t rk4 = rk, rvs = rv;          // MX: the scale instructions' sources
    if constexpr (MX) {
      rk4 = wave >= 2 ? bytes_rsrc_at(ksa, min(C::kTileKeys, kr) * 4) : rk;
      rvs = bytes_rsrc_at(vsa, min(4, vbr) * 128);
    }
    iteration(u, tail_c, rk, rv, rk4, rvs, advance);
  };
  int u = u0;
  for (; u + 3 < u1; ++u) run(u, flag_t<false>{});
  for (; u < u1; ++u) run(u, flag_t<true>{});

  // ---- P V of the last sub-tile (its V fragments were read in the last phase Y)
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      if constexpr (MX)
        pv_mfma_mx(acc[qb][db], vf[db], pA[qb], vsc, p_one, db);
      else
        pv_mfma(acc[qb][db], vf[db], pA[qb]);
    }
  pv_drain(acc, vf, pA, vsc, p_one);

  // l sums 8 p, and so does acc: their ratio needs no further scaling
  float l_q[2];                        // the row sum of this lane's query
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lo = __shfl(l_lo[qb], l32 & 15), hi = __shfl(l_hi[qb], l32 & 15);
    l_q[qb] = l32 < 16 ? lo : hi;
  }
  if (ws_index >= 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = l_q[qb];
      const float mul = dv / l_tot;
      const int r = wave * 64 + qb * 32 + l32;
      float* orow = split.ws_o + ((size_t)ws_index * C::kBR + r) * D;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + i * 8 + hh * 4;
          f32x4_t w = {acc[qb][db][i * 4 + 0] * mul, acc[qb][db][i * 4 + 1] * mul, acc[qb][db][i * 4 + 2] * mul,
                       acc[qb][db][i * 4 + 3] * mul};
          *(f32x4_t*)(orow + d0) = w;
        }
      if (hh == 0) split.ws_lse[(size_t)ws_index * C::kBR + r] = mc[qb] + __log2f(l_tot) - kFp8PipePLog2;
      if constexpr (EXACT_LSE) {
        const float l_exact = pair_sum(l_ex[qb]);
        if (hh == 0) split.ws_lse_out[(size_t)ws_index * C::kBR + r] = mc[qb] + __log2f(l_exact) - kFp8PipePLog2;
      }
    }
    return;
  }
  // O goes to HBM through LDS, over the K/V slots (no DMA is in flight after
  // the last iteration), so that each store instruction writes 4 whole rows
  // instead of 8-byte pieces of 32 rows; each wave stages its own 64 rows.
  __syncthreads();
  char* ost = smem + wave * (64 * C::kORow);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float l_tot = l_q[qb];
    const float mul = dv / l_tot;
    char* srow = ost + (qb * 32 + l32) * C::kORow;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + hh * 4;
        uint2 w;
        w.x = pack_bf16x2(acc[qb][db][i * 4 + 0] * mul, acc[qb][db][i * 4 + 1] * mul);
        w.y = pack_bf16x2(acc[qb][db][i * 4 + 2] * mul, acc[qb][db][i * 4 + 3] * mul);
        *(uint2*)(srow + d0 * 2) = w;
      }
    if constexpr (EXACT_LSE) {
      const float l_exact = pair_sum(l_ex[qb]);
      const int row = q0 + qb * 32 + l32;
      if (hh == 0 && row < N)
        LSEg[(size_t)bh * N + row] = (mc[qb] + __log2f(l_exact) - kFp8PipePLog2) * 0.6931471805599453f;
    }
  }
  // other lanes of the same wave read the staged rows: one wave's LDS
  // operations complete in order, and the wait pins the reads after the writes
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  const int chunk = lane & 15;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rl = r * 4 + (lane >> 4);
    const i32x4_t x = *(const i32x4_t*)(ost + rl * C::kORow + chunk * 16);
    const int row = q0 + rl;
    if (row < N) *(i32x4_t*)(Og + obase + (long long)row * L.on + chunk * 8) = x;
  }
}

#undef DIT_FENCE

}  // namespace ditattn
