// bf16 attention forward for gfx950, d = 128: 64 query rows per wave,
// software-pipelined, K/V tiles moved by LDS DMA.
//
// Shape. A wave owns 64 query rows (two 32-row blocks), so every K or V
// fragment it reads from LDS feeds two MFMAs; with 32 rows per wave the LDS
// would have to deliver twice the bytes per flop. The O accumulator is then
// 128 registers per lane and one wave runs per SIMD (4 waves, 256 rows per
// workgroup), so the wave interleaves its own MFMA, VALU and LDS work.
//
// Data movement. K and V tiles of 64 keys go from HBM to LDS with
// buffer_load_dwordx4 ... lds: no staging registers, no LDS store
// instructions, and rows past N arrive as zeros from the buffer range check.
// Rows are padded (K 272 bytes, V 320 bytes) so that every fragment read is
// free of bank conflicts and addressed by one register plus an immediate; the
// DMA writes 1 KB of consecutive LDS per instruction, and lanes that land on
// padding are pointed past the tile, so the range check zero-fills them
// without a memory access. K lives in a ring of 4 tile slots and V in a ring
// of 3: while tile u is computed on, K tile u+3 and V tile u+2 stream in (one
// DMA instruction on every other step of phase X), and one s_waitcnt +
// barrier per 64 keys publishes the tiles issued an iteration earlier.
//
// Sub-iteration j (32 keys), two phases of 8 steps. Each step is one
// O^T += V_{j-1}^T P_{j-1}^T MFMA and one S_{j+1} = K_{j+1} Q^T MFMA (a chain
// over d), with a fixed VALU mix split around the two MFMAs: two exponentials
// of P_j and two FMAs forming exponent arguments (of S_j's second query block
// in phase X, of S_{j+1}'s first in phase Y) behind the first, the row-sum
// adds and the bf16 pack of those two exponentials behind the second, so that
// no instruction waits on the transcendental unit's result. Fragment reads
// from LDS follow the MFMA that last reads the register they fill: V_j over
// both phases, K_{j+2} over phase Y. P alternates between two register sets
// over the two sub-iterations of a tile, so nothing is copied at the loop
// edge. Row sums are of the rounded P (the values O is multiplied with), on
// the matrix core: a 16x16x32 product of the packed P with a lane-selected
// ones operand.
//
// Softmax without a per-tile maximum. The running maximum m (log2 units, per
// query row) starts at the exact maximum of the first 32 keys. bf16 keeps
// 8 significant bits at any scale, so probabilities relative to a stale m lose
// nothing as long as nothing overflows. A tile first runs with m fixed and no
// test in the loop; its row sums are tested once at the end, and if any is
// not finite or exceeds 2^64 the workgroup runs the tile again with the
// checked loop, in which m moves whenever a sum of 16 of a sub-tile's
// probabilities exceeds 2^64 (or is not finite): that rare path recomputes
// the sub-tile's logits from K (still in LDS), takes their exact maximum,
// rescales O and l and recomputes P.
//
// Row sums. O is divided by the sum of the bf16-rounded probabilities that
// the P V products multiply V with, so every output row is a convex
// combination of rows of V; a row that one key dominates then keeps nothing
// of that key's rounding error. The sums come from the matrix core: one
// 16x16x32 product of each packed P^T fragment with a ones operand (no VALU
// adds), which also feeds the overflow test. The EXACT_LSE form, used when a
// log-sum-exp is requested, adds fp32 sums of the unrounded probabilities for
// it, so the log-sum-exp is the exact one; O is the same in both forms.
//
// Schedules. pipe_tile runs one query tile over a range of key tiles.
// attn_fwd_bf16_pipe_kernel gives each workgroup a whole tile, or one key
// range of a tile of the last, partly filled round (merged afterwards by
// attn_split_combine_kernel); attn_fwd_bf16_streamk_kernel gives each of one
// workgroup per CU an equal contiguous range of (tile, key tile) pairs
// (merged by attn_streamk_combine_kernel). The SPARSE form takes its key
// tiles from a per-tile list instead of 0 .. n_t - 1.
// Layout conventions (S^T = K Q^T, O^T = V^T P^T, V^T by transpose reads)
// are those of attn_fwd_bf16.h. Built with -mllvm -amdgpu-mfma-vgpr-form.
#pragma once
#include <type_traits>

#include "attn_common.h"

namespace ditattn {

struct PipeCfg {
  static constexpr int kD = 128, kNW = 4, kThreads = 256, kBR = 256;
  static constexpr int kKS = 8, kDB = 4;
  static constexpr int kKRow = 272, kVRow = 320;          // padded row pitch in LDS (bytes)
  static constexpr int kKTile = 64 * kKRow;               // 17408 bytes of K rows
  static constexpr int kVTile = 64 * kVRow;               // 20480 bytes of V rows
  // Both tiles move as 20 DMA instructions of 1 KB, 5 per wave, so every wave
  // issues the same count; the last 3 K instructions land past the K rows, in
  // the slot's slack, and read nothing (their offsets are past the tile).
  static constexpr int kDmaPerWave = 5;
  static constexpr int kSlot = kNW * kDmaPerWave * 1024;  // 20480
  static constexpr int kKSlots = 4, kVSlots = 3;
  static constexpr int kVBase = kKSlots * kSlot;
  // past the slots: one word per wave, whether its unchecked pass overflowed
  static constexpr int kFlagOff = kVBase + kVSlots * kSlot;   // 143360
  static constexpr int kLdsBytes = kFlagOff + 16;
  static_assert(kKTile <= kSlot && kVTile <= kSlot, "tile fits its slot");
  // The bf16 O rows of a finished tile are staged in LDS (over the K/V slots,
  // 64 rows per wave, padded pitch) on their way to HBM.
  static constexpr int kORow = 272;
  static_assert(kNW * 64 * kORow <= kLdsBytes, "O staging fits the slots");
  static constexpr int kWsRow = 528;                       // fp32 partial rows of a split tile
  static_assert(kNW * 64 * kWsRow <= kLdsBytes, "partial-row staging fits the slots");
};

constexpr float kPipeSumLimit = 0x1p64f;   // overflow guard: far below FLT_MAX / N

// Key-range split of the last, partly filled round of workgroups. The first
// n_full workgroups each take one 256-row query tile over all keys. The next
// n_split * parts workgroups take the remaining n_split query tiles, each
// split into `parts` contiguous ranges of 64-key tiles; they write their rows
// normalised over their own keys (fp32, ws_o) with the log2-sum-exp of that
// range (ws_lse), and attn_split_combine_kernel merges the parts.
struct PipeSplit {
  int n_full, n_split, parts;
  float* ws_o;      // [n_split * parts][256][128]
  float* ws_lse;    // [n_split * parts][256], log2 units: the merge weights of O
  float* ws_lse_out;  // NULL, or [n_split * parts][256]: a different log2 sum for the LSE output
};

template <bool B>
using flag_t = std::integral_constant<bool, B>;

// Block-sparse visiting: for query tile t of head bh (t over 256-row tiles),
// the 64-key tiles list[(bh * n_qtiles + t) * max_blocks + i], i < count, in
// ascending order, with count = counts[bh * n_qtiles + t] (at most
// max_blocks). Unused by the dense form.
struct KvBlocks {
  const int* list;
  const int* counts;
  int max_blocks;
};

// 16 bytes per lane from a buffer into LDS at M0 + 16 * lane. Written as asm
// so that the compiler does not order every later LDS read behind it (it
// would wait for all loads in flight); completion is awaited explicitly with
// s_waitcnt vmcnt before the barrier that publishes the tile.
__device__ __forceinline__ void dma_b128(i32x4_t rsrc, int voffset, unsigned lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voffset), "s"(rsrc), "{m0}"(lds_addr) : "memory");
}

#define DIT_FENCE() __builtin_amdgcn_sched_barrier(0)

// One query tile over the key tiles [u0, u1) (dense) or over list positions
// (SPARSE: the key tiles come from a KvBlocks list instead of 0 .. n_t - 1;
// a split tile's part `part` of split.parts takes its share of the list).
// ws_index >= 0: write the rows normalised over this range, with their
// log2-sum-exp, to workspace slot ws_index; otherwise write O (and the LSE).
template <class C, bool SPARSE, bool EXACT_LSE>
__device__ __forceinline__ void pipe_tile(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                                          const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                                          float* __restrict__ LSEg, int N, int n_qtiles, float scale_log2,
                                          const PipeSplit& split, const Layout& L, const KvBlocks& kvb, int tile,
                                          int u0, int u1, int ws_index, int part) {
  constexpr int D = C::kD, KS = C::kKS, DB = C::kDB;
  constexpr int KROW = C::kKRow, VROW = C::kVRow;
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int n_t = (N + 63) / 64;          // 64-key tiles
  const int bh = tile / n_qtiles;
  const int qt = tile - bh * n_qtiles;
  // key tile at pipeline position p: p itself, or the p-th listed one. The
  // pipeline looks up to three positions past the end; those clamp to the
  // last entry (their data is never used).
  // The list is read through the constant address space: scalar loads, which
  // do not count against the vector-memory counter that orders the tile DMAs.
  using cint = const __attribute__((address_space(4))) int;
  cint* klist = nullptr;
  if constexpr (SPARSE) {
    // a split tile's parts take contiguous ranges of list positions
    const int cnt = *(cint*)(kvb.counts + tile);
    const int c = cnt < 0 ? 0 : (cnt > kvb.max_blocks ? kvb.max_blocks : cnt);
    const int parts = ws_index >= 0 ? split.parts : 1;   // an unsplit tile takes the whole list
    u0 = part * c / parts;
    u1 = (part + 1) * c / parts;
    klist = (cint*)(kvb.list + (size_t)tile * kvb.max_blocks);
  }
  auto ktile = [&](int p) __attribute__((always_inline)) {
    if constexpr (SPARSE) return klist[p < u1 ? p : u1 - 1];
    else return p;
  };
  // first key of sub-tile j (32 keys) of the pipeline
  auto ksub = [&](int j) __attribute__((always_inline)) { return ktile(j >> 1) * 64 + (j & 1) * 32; };
  const long long ibase = L.in_off(bh), obase = L.out_off(bh);
  const int rowb = (int)(L.qn * 2);       // bytes between consecutive tokens of q, k, v
  const char* Kh = reinterpret_cast<const char*>(Kg + ibase);
  const char* Vh = reinterpret_cast<const char*>(Vg + ibase);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31, hh = lane >> 5;
  const int q0 = qt * C::kBR + wave * 64;

  if constexpr (SPARSE) {
    if (u1 <= u0) {
      // no listed key: attention over the empty set gives O = 0, LSE = -inf
      // (for a part of a split tile: zero rows of weight 2^-inf)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const int row = q0 + qb * 32 + l32;
        if (ws_index >= 0) {
          const int r = wave * 64 + qb * 32 + l32;
          float* orow = split.ws_o + ((size_t)ws_index * C::kBR + r) * D + hh * (D / 2);
#pragma unroll
          for (int c = 0; c < D / 2; c += 4) *(f32x4_t*)(orow + c) = f32x4_t{0.f, 0.f, 0.f, 0.f};
          if (hh == 0) split.ws_lse[(size_t)ws_index * C::kBR + r] = -INFINITY;
          if (EXACT_LSE && hh == 0) split.ws_lse_out[(size_t)ws_index * C::kBR + r] = -INFINITY;
        } else if (row < N) {
          uint16_t* orow = Og + obase + (long long)row * L.on + hh * (D / 2);
#pragma unroll
          for (int c = 0; c < D / 2; c += 8) *(i32x4_t*)(orow + c) = i32x4_t{0, 0, 0, 0};
          if (LSEg != nullptr && hh == 0) LSEg[(size_t)bh * N + row] = -INFINITY;
        }
      }
      return;
    }
  }

  bf16x8_t qf[2][KS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const uint16_t* Q = Qg + ibase;
    const int row = q0 + qb * 32 + l32;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      i32x4_t raw = {0, 0, 0, 0};
      if (row < N) raw = *(const i32x4_t*)(Q + (long long)row * L.qn + ks * 16 + hh * 8);
      qf[qb][ks] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // ---- DMA: instruction i of a tile writes LDS bytes [1024 i, 1024 i + 1024);
  // lane L covers 16-byte slot 64 i + L of the padded tile
  int kdo[C::kDmaPerWave], vdo[C::kDmaPerWave];
#pragma unroll
  for (int m = 0; m < C::kDmaPerWave; ++m) {
    const int s = 64 * (wave + 4 * m) + lane;
    const int kr = s / (KROW / 16), kc = s % (KROW / 16);
    const int vr = s / (VROW / 16), vc = s % (VROW / 16);
    // padding slots get an offset past any tile (64 rows), so the range check
    // zero-fills them without a memory access
    kdo[m] = kc < D / 8 ? kr * rowb + kc * 16 : 64 * rowb;
    vdo[m] = vc < D / 8 ? vr * rowb + vc * 16 : 64 * rowb;
  }
  // buffer descriptor of `rows` rows from address a: the range check
  // zero-fills rows past them. Only descriptors of tiles that exist are used
  // (rows >= 1); others are built but never read. Every field must come from
  // the scalar unit: a VALU write of an SGPR (v_readfirstlane of a VALU
  // result, a VALU min/max/med3) needs 5 wait states before a vector-memory
  // instruction reads that SGPR, and the compiler does not insert them for
  // the inline-asm DMA (the build refuses ISA with such a hazard). A plain
  // min keeps it on the scalar unit, with its SCC use known to the compiler.
  auto make_rsrc = [&](unsigned long long a, int rows) __attribute__((always_inline)) {
    i32x4_t rs;
    rs[0] = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
    rs[1] = __builtin_amdgcn_readfirstlane((int)((a >> 32) & 0xffffu));   // stride 0
    rs[2] = __builtin_amdgcn_readfirstlane(min(64, rows) * rowb);          // bytes in range
    rs[3] = 0x00020000;
    return rs;
  };
  // buffer descriptor of one 64-key tile: the range check zero-fills rows past N
  auto tile_rsrc = [&](const char* head, int t) __attribute__((always_inline)) {
    int rows = N - t * 64;
    if constexpr (SPARSE) {
      // a listed index outside [0, n_t) (a malformed list) reads zeros
      const bool inside = t >= 0 && t < n_t;
      rows = inside ? rows : 0;
      t = inside ? t : 0;
    }
    return make_rsrc((unsigned long long)(head + (long long)t * 64 * rowb), rows);
  };
  // the m-th DMA instruction of this wave for one tile (instruction wave + 4 m)
  auto dma_one = [&](const i32x4_t& rs, const char* slot, const int (&off)[C::kDmaPerWave], int m)
      __attribute__((always_inline)) {
    const int i = wave + 4 * m;
    dma_b128(rs, off[m], __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)DIT_LDS(const char, slot) + i * 1024));
  };
  auto dma_tile = [&](const char* head, int t, const char* slot, const int (&off)[C::kDmaPerWave])
      __attribute__((always_inline)) {
    const i32x4_t rs = tile_rsrc(head, t);
#pragma unroll
    for (int m = 0; m < C::kDmaPerWave; ++m) dma_one(rs, slot, off, m);
  };
  // Slot offsets pass through readfirstlane so that the compiler keeps them in
  // an SGPR instead of folding the V base into every read's immediate offset,
  // which exceeds the 16-bit field and costs a VALU add per read.
  auto kslot = [&](int t) { return smem + __builtin_amdgcn_readfirstlane((t % C::kKSlots) * C::kSlot); };
  auto vslot = [&](int t) {
    return smem + __builtin_amdgcn_readfirstlane(C::kVBase + (t % C::kVSlots) * C::kSlot);
  };

  // ---- fragment reads
  const int k_rd = l32 * KROW + hh * 16;
  const int g = lane >> 4, gi = lane & 15;
  const int v_rd = ((g >> 1) * 4 + (gi >> 2)) * VROW + (g & 1) * 32 + (gi & 3) * 8;
  bf16x8_t kf[KS];
  auto kbase = [&](int j) { return kslot(j >> 1) + (j & 1) * 32 * KROW + k_rd; };
  auto read_kfrag = [&](const char* kb, int ks) __attribute__((always_inline)) {
    kf[ks] = __builtin_bit_cast(bf16x8_t, *(const i32x4_t*)(kb + ks * 32));
  };
  auto read_kfrags_at = [&](const char* kb) __attribute__((always_inline)) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) read_kfrag(kb, ks);
  };
  auto read_kfrags = [&](int j) { read_kfrags_at(kbase(j)); };
  bf16x8_t vf[2][DB];
  auto read_vfrag = [&](const char* vb, int half, int db) __attribute__((always_inline)) {
    const char* p = vb + half * 16 * VROW + db * 64;
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(DIT_LDS(i16x4_t, p));
    const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(DIT_LDS(i16x4_t, (p + 8 * VROW)));
    const i32x2_t lo2 = __builtin_bit_cast(i32x2_t, lo), hi2 = __builtin_bit_cast(i32x2_t, hi);
    const i32x4_t a4 = {lo2[0], lo2[1], hi2[0], hi2[1]};
    vf[half][db] = __builtin_bit_cast(bf16x8_t, a4);
  };
  // keys of sub-tile j past N do not exist
  auto mask_keys = [&](int j, f32x16_t& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = ksub(j) + (r >> 2) * 8 + hh * 4 + (r & 3);
      s[r] = key < N ? s[r] : -INFINITY;
    }
  };
  auto s_chain = [&](int qb, f32x16_t& s) {
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[qb][ks], s, 0, 0, 0);
  };
  auto row_max = [&](const f32x16_t& s) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    return pair_max(mx) * scale_log2;      // scale_log2 > 0
  };
  // p = 2^t[i] (EXACT_LSE: also summed unrounded into ls); pack_word puts
  // two p as bf16 word e & 3 of out[e >> 2].
  auto exp_one = [&](const f32x16_t& t, int i, float& ls) __attribute__((always_inline)) {
    const float p = fast_exp2(t[i]);
    if constexpr (EXACT_LSE) {
      ls += p;
      asm volatile("" : "+v"(ls));     // keeps the add in this step
    }
    return p;
  };
  // exp2 now, its row-sum add later: the add waits on the transcendental unit
  auto exp_raw = [&](const f32x16_t& t, int i) __attribute__((always_inline)) {
    float p = fast_exp2(t[i]);
    asm volatile("" : "+v"(p));
    return p;
  };
  auto pack_word = [&](float a, float b, int e, bf16x8_t (&out)[2]) __attribute__((always_inline)) {
    const bf16x2_t pk = {(__bf16)a, (__bf16)b};
    int word = __builtin_bit_cast(int, pk);
    asm volatile("" : "+v"(word));     // keeps the pack in this step
    i32x4_t w = __builtin_bit_cast(i32x4_t, out[e >> 2]);
    w[e & 3] = word;
    out[e >> 2] = __builtin_bit_cast(bf16x8_t, w);
  };
  // the pack of two p (EXACT_LSE: and their unrounded adds), placed at this point
  auto sum_pack = [&](float& ls, float a, float b, int e, bf16x8_t (&out)[2]) __attribute__((always_inline)) {
    asm volatile("" : "+v"(a), "+v"(b));
    if constexpr (EXACT_LSE) {
      ls += a;
      ls += b;
      asm volatile("" : "+v"(ls));
    }
    pack_word(a, b, e, out);
  };
  // Row sums of the packed P on the matrix core. Read as the B operand of the
  // 16x16x32 product, lane 16 g + c of a P^T fragment is column c, k-group g
  // (query c + 16 (g & 1), 8 of the fragment's 16 keys); A holds ones exactly
  // where row r meets k-group r, so output row r, column c sums the 8 values
  // of lane 16 r + c. Lanes 0..15 receive the sums of queries c (rows 0, 2)
  // and c + 16 (rows 1, 3); the other lanes' rows are zero.
  const int one_w = (lane & 15) == (lane >> 4) ? 0x3F803F80 : 0;        // two bf16 1.0
  const bf16x8_t ones = __builtin_bit_cast(bf16x8_t, i32x4_t{one_w, one_w, one_w, one_w});
  auto psum = [&](const bf16x8_t& pt, const f32x4_t& c) __attribute__((always_inline)) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pt, c, 0, 0, 0);
  };

  // The state a pass over the tile's keys leaves for the epilogue.
  f32x16_t acc[2][DB];
  float mc[2];                 // running row maxima, log2 units
  // row sums of the rounded P in lanes 0..15: query c of each block in l_lo,
  // query c + 16 in l_hi; EXACT_LSE: this lane's sums of the unrounded p
  float l_lo[2], l_hi[2], l_ex[2];

  // One pass over the tile's keys. CHECKED: the running maximum moves when
  // a sub-tile's sums of 16 p pass 2^64 or are not finite (the rare path
  // below). Not CHECKED: it stays at the first sub-tile's exact maximum, the
  // row-sum products of a sub-tile go back to back into running sums that
  // nothing reads in the loop, and the caller tests the final sums once; a
  // tile whose sums are not all finite and at most 2^64 runs again CHECKED.
  auto pass = [&](auto checked_c) __attribute__((always_inline)) {
    constexpr bool CHECKED = decltype(checked_c)::value;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[qb][db][r] = 0.f;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) l_lo[qb] = l_hi[qb] = l_ex[qb] = 0.f;
    f32x4_t lrun[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};   // not CHECKED: running sums
    f32x16_t t0;                 // exponent arguments of the current sub-tile, query block 0
    f32x16_t s1;                 // raw logits of the current sub-tile, query block 1
    bf16x8_t pA[2][2], pB[2][2]; // P of two consecutive sub-tiles [query block][key half]
    // LDS byte offsets of the ring slots the iteration of pipeline position u
    // uses: K of positions u, u+1, u+3 and V of u, u+2. They rotate by one
    // slot per iteration (scalar adds instead of a modulo per use).
    struct Ring {
      int k0, k1, k3, v0, v2;
    };
    Ring ring;

    // ---- prologue: K tiles u0..u0+2, V tiles u0, u0+1; the first sub-tile's
    // logits and their exact row maxima. The first iteration reads K u0, K u0+1
    // and V u0 only, so K u0+2 and V u0+1 go last and stay in flight (their 10
    // instructions) until that iteration's own wait; the Q loads, issued before
    // all of them, are complete once those are the only ones left.
    dma_tile(Kh, ktile(u0), kslot(u0), kdo);
    dma_tile(Vh, ktile(u0), vslot(u0), vdo);
    if (u0 + 1 < u1) dma_tile(Kh, ktile(u0 + 1), kslot(u0 + 1), kdo);
    if (u0 + 2 < u1) {
      dma_tile(Kh, ktile(u0 + 2), kslot(u0 + 2), kdo);
      dma_tile(Vh, ktile(u0 + 1), vslot(u0 + 1), vdo);
      __builtin_amdgcn_s_waitcnt(0x0F7A);    // vmcnt(10)
    } else {
      if (u0 + 1 < u1) dma_tile(Vh, ktile(u0 + 1), vslot(u0 + 1), vdo);
      __builtin_amdgcn_s_waitcnt(0x0F70);    // vmcnt(0)
    }
    __syncthreads();
    read_kfrags(2 * u0);
    {
      f32x16_t s0;
      s_chain(0, s0);
      s_chain(1, s1);
      if (ksub(2 * u0) + 32 > N) { mask_keys(2 * u0, s0); mask_keys(2 * u0, s1); }
      mc[0] = row_max(s0);
      mc[1] = row_max(s1);
  #pragma unroll
      for (int r = 0; r < 16; ++r) t0[r] = fmaf(s0[r], scale_log2, -mc[0]);
    }
    read_kfrags(2 * u0 + 1);          // the K fragments a sub-iteration starts with are those of the next sub-tile
    // the first phase X adds 0 * 0: no previous sub-tile yet
  #pragma unroll
    for (int h = 0; h < 2; ++h)
  #pragma unroll
      for (int x = 0; x < 2; ++x) pA[h][x] = bf16x8_t{};
  #pragma unroll
    for (int h = 0; h < 2; ++h)
  #pragma unroll
      for (int db = 0; db < DB; ++db) vf[h][db] = bf16x8_t{};

    // One sub-iteration j. On entry: P_{j-1} (pin), V_{j-1} fragments (vf),
    // K_{j+1} fragments (kf), S_j's exponent arguments for query block 0 (t0)
    // and raw logits for query block 1 (s1). Two phases of 8 steps; each step
    // is one P V MFMA (independent accumulators) and one S_{j+1} MFMA (a chain),
    // with half of the same VALU mix behind each: two exponentials of P_j with
    // their row-sum adds and bf16 pack, and two FMAs. The LDS reads of the next
    // fragments follow the MFMA that last reads the register: V_j during both
    // phases, K_{j+2} during phase Y. On exit the state holds sub-tile j+1.
    // MASK: keys of S_{j+1} (and, on the rare path, of S_j) may lie past N.
    // dma(m) issues this sub-iteration's share of the tile DMA at phase-X step 2 m.
    auto sub = [&](int j, bf16x8_t (&pin)[2][2], bf16x8_t (&pout)[2][2], auto mask_c, auto&& dma)
        __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_c)::value;
      float ls0 = 0.f, ls1 = 0.f;   // EXACT_LSE only
      const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
      f32x4_t rs0, rs1;          // matrix-core sums of P_j, query blocks 0 and 1
      f32x16_t& t1 = s1;         // in place
      f32x16_t sa, sb;           // S_{j+1} of query blocks 0 and 1
      const char* vb = smem + ring.v0 + (j & 1) * 32 * VROW + v_rd;      // V of position j / 2
      const char* kb2 = smem + ring.k1 + (j & 1) * 32 * KROW + k_rd;     // K of sub-tile j + 2
      // ================= phase X: P_{j-1} V_{j-1} (keys 0-15), S_{j+1} block 0, P_j block 0
      {
        const float m1 = mc[1];
  #pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int qb = st & 1, db = st >> 1;
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[0][db], pin[qb][0], acc[qb][db], 0, 0, 0);
          const float pa = exp_raw(t0, 2 * st), pb = exp_raw(t0, 2 * st + 1);
          t1[2 * st] = fmaf(s1[2 * st], scale_log2, -m1);
          t1[2 * st + 1] = fmaf(s1[2 * st + 1], scale_log2, -m1);
          if ((st & 1) == 0) dma(st >> 1);
          DIT_FENCE();
          if (st == 0) {
  #pragma unroll
            for (int r = 0; r < 16; ++r) sa[r] = 0.f;
          }
          sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[0][st], sa, 0, 0, 0);
          if (CHECKED && st == 4) rs0 = psum(pout[0][0], zero4);   // words 0-3 were packed in steps 0-3
          sum_pack(ls0, pa, pb, st, pout[0]);
          if (st & 1) read_vfrag(vb, 0, db);      // both query blocks have used vf[0][db]
          DIT_FENCE();
        }
      }
      if constexpr (MASK) {
        if (ksub(j + 1) + 32 > N) mask_keys(j + 1, sa);
      }
      // ================= phase Y: P_{j-1} V_{j-1} (keys 16-31), S_{j+1} block 1, P_j block 1
      {
        const float m0 = mc[0];
  #pragma unroll
        for (int st = 0; st < 8; ++st) {
          const int qb = st & 1, db = st >> 1;
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[1][db], pin[qb][1], acc[qb][db], 0, 0, 0);
          const float pa = exp_raw(t1, 2 * st), pb = exp_raw(t1, 2 * st + 1);
          t0[2 * st] = fmaf(sa[2 * st], scale_log2, -m0);        // S_{j+1}'s arguments
          t0[2 * st + 1] = fmaf(sa[2 * st + 1], scale_log2, -m0);
          DIT_FENCE();
          if (st == 0) {
  #pragma unroll
            for (int r = 0; r < 16; ++r) sb[r] = 0.f;
          }
          sb = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[st], qf[1][st], sb, 0, 0, 0);
          if (CHECKED && st == 0) rs0 = psum(pout[0][1], rs0);
          if (CHECKED && st == 4) rs1 = psum(pout[1][0], zero4);
          sum_pack(ls1, pa, pb, st, pout[1]);
          read_kfrag(kb2, st);                     // kf[st] is free: K_{j+2}
          if (st & 1) read_vfrag(vb, 1, db);
          DIT_FENCE();
        }
      }
      if constexpr (MASK) {
        if (ksub(j + 1) + 32 > N) mask_keys(j + 1, sb);
      }
      s1 = sb;
      // The packed P must exist here: without this the compiler sinks the bf16
      // packs past the rare-path branch, out of the MFMA phases.
      asm volatile("" ::"v"(pout[0][0]), "v"(pout[0][1]), "v"(pout[1][0]), "v"(pout[1][1]));
      if constexpr (CHECKED) {
        rs1 = psum(pout[1][1], rs1);
        // ---- rare path: a sum of 16 of sub-tile j's p passed 2^64 or is not
        // finite. The sums are >= +0 or NaN, so their bit patterns order like the
        // values, with every NaN above +inf: one unsigned maximum decides.
        auto bits = [](float x) { return __float_as_uint(x); };
        const uint32_t big = max(max(max(bits(rs0[0]), bits(rs0[1])), max(bits(rs0[2]), bits(rs0[3]))),
                                 max(max(bits(rs1[0]), bits(rs1[1])), max(bits(rs1[2]), bits(rs1[3]))));
        if (__builtin_expect(__builtin_amdgcn_ballot_w64(big > __float_as_uint(kPipeSumLimit)) != 0, 0)) {
          read_kfrags_at(smem + ring.k0 + (j & 1) * 32 * KROW + k_rd);   // K tiles j/2 and (j+2)/2 are still in their slots
    #pragma unroll
          for (int qb = 0; qb < 2; ++qb) {
            f32x16_t s;
            s_chain(qb, s);
            if constexpr (MASK) {
              if (ksub(j) + 32 > N) mask_keys(j, s);
            }
            const float m_new = fmaxf(mc[qb], row_max(s));
            const float alpha = fast_exp2(mc[qb] - m_new);
            l_lo[qb] *= __shfl(alpha, lane & 15);
            l_hi[qb] *= __shfl(alpha, (lane & 15) + 16);
            if constexpr (EXACT_LSE) l_ex[qb] *= alpha;
    #pragma unroll
            for (int db = 0; db < DB; ++db)
    #pragma unroll
              for (int r = 0; r < 16; ++r) acc[qb][db][r] *= alpha;
            if (qb == 0) {
              const float shift = m_new - mc[0];
    #pragma unroll
              for (int r = 0; r < 16; ++r) t0[r] -= shift;    // S_{j+1}'s arguments used the old maximum
            }
            mc[qb] = m_new;
    #pragma unroll
            for (int r = 0; r < 16; ++r) s[r] = fmaf(s[r], scale_log2, -m_new);
            float& ls = qb == 0 ? ls0 : ls1;
            ls = 0.f;
    #pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pa = exp_one(s, 2 * e, ls);
              pack_word(pa, exp_one(s, 2 * e + 1, ls), e, pout[qb]);
            }
          }
          rs0 = psum(pout[0][1], psum(pout[0][0], zero4));
          rs1 = psum(pout[1][1], psum(pout[1][0], zero4));
          read_kfrags_at(kb2);
        }
        l_lo[0] += rs0[0] + rs0[2];
        l_hi[0] += rs0[1] + rs0[3];
        l_lo[1] += rs1[0] + rs1[2];
        l_hi[1] += rs1[1] + rs1[3];
      } else {
        // the four row-sum products of P_j back to back, into the running sums
        lrun[0] = psum(pout[0][0], lrun[0]);
        lrun[1] = psum(pout[1][0], lrun[1]);
        lrun[0] = psum(pout[0][1], lrun[0]);
        lrun[1] = psum(pout[1][1], lrun[1]);
        (void)rs0;
        (void)rs1;
      }
      if constexpr (EXACT_LSE) {
        l_ex[0] += ls0;
        l_ex[1] += ls1;
      }
    };

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

    // One 64-key tile u. It streams in K tile u+3 (during its first
    // sub-iteration) and V tile u+2 (during its second), one DMA instruction on
    // every other phase-X step, and then waits for the tiles issued one iteration earlier
    // (K u+2, V u+1) before the barrier that publishes them. In the steady
    // state (TAIL false) both DMAs exist and no key of tiles u, u+1 lies past N,
    // so the body has no branch but the rare path: a branch would let the
    // compiler sink the softmax work out of the MFMA phases.
    // rk, rv: the descriptors of the key tiles at positions u + 3 (K) and u + 2
    // (V); before_wait() runs after the compute, ahead of the wait for the
    // tiles (the next iteration's scalar bookkeeping goes there, behind the
    // last MFMAs in flight).
    auto iteration = [&](int u, auto tail_c, const i32x4_t& rk, const i32x4_t& rv, auto&& before_wait)
        __attribute__((always_inline)) {
      constexpr bool TAIL = decltype(tail_c)::value;
      const bool k_next = !TAIL || u + 3 < u1, v_next = !TAIL || u + 2 < u1;
      const char* sk = smem + ring.k3;
      const char* sv = smem + ring.v2;
      DIT_FENCE();
      // hook steps st = 0..3 issue instructions m = st, and m = 4 at st = 0
      static_assert(C::kDmaPerWave == 5, "DMA hook spreads 5 instructions over 4 steps");
      sub(2 * u, pA, pB, tail_c, [&](int st) __attribute__((always_inline)) {
        if (k_next) {
          dma_one(rk, sk, kdo, st);
          if (st == 0) dma_one(rk, sk, kdo, 4);
        }
      });
      sub(2 * u + 1, pB, pA, tail_c, [&](int st) __attribute__((always_inline)) {
        if (v_next) {
          dma_one(rv, sv, vdo, st);
          if (st == 0) dma_one(rv, sv, vdo, 4);
        }
      });
      DIT_FENCE();
      before_wait();
      advance_ring();
      if (TAIL)
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
      else
        __builtin_amdgcn_s_waitcnt(0x0F7A);  // vmcnt(10): this iteration's 10 DMAs may stay in flight
      __syncthreads();
      DIT_FENCE();
    };
    // Sub-tiles past u1 that the pipeline touches (S of sub-tile 2 u1) read a
    // slot that is stale or zero: their values are never used.
    int u = u0;
    if constexpr (SPARSE) {
      // A steady-state iteration loads the next one's K tile index while it
      // waits for its DMAs (a scalar load waited for at the top of the loop
      // would stall every wave there).
      int tk = ktile(u0 + 3), tv = ktile(u0 + 2);
      for (; u + 3 < u1; ++u) {
        int tk_next;
        iteration(u, flag_t<false>{}, tile_rsrc(Kh, tk), tile_rsrc(Vh, tv), [&] {
          tk_next = ktile(u + 4);
          asm volatile("" : "+s"(tk_next));
        });
        tv = tk;
        tk = tk_next;
      }
      for (; u < u1; ++u) iteration(u, flag_t<true>{}, tile_rsrc(Kh, ktile(u + 3)), tile_rsrc(Vh, ktile(u + 2)), [] {});
    } else {
      // the tiles at positions u + 3 (K) and u + 2 (V): addresses and rows left,
      // advanced by one tile per iteration
      const unsigned long long tile_bytes = (unsigned long long)64 * rowb;
      unsigned long long ka = (unsigned long long)(Kh + (long long)(u0 + 3) * 64 * rowb);
      unsigned long long va = (unsigned long long)(Vh + (long long)(u0 + 2) * 64 * rowb);
      int kr = N - (u0 + 3) * 64, vr = N - (u0 + 2) * 64;
      auto advance = [&]() __attribute__((always_inline)) {
        ka += tile_bytes;
        va += tile_bytes;
        kr -= 64;
        vr -= 64;
      };
      for (; u + 3 < u1; ++u) iteration(u, flag_t<false>{}, make_rsrc(ka, kr), make_rsrc(va, vr), advance);
      for (; u < u1; ++u) iteration(u, flag_t<true>{}, make_rsrc(ka, kr), make_rsrc(va, vr), advance);
    }

    // ---- P V of the last sub-tile (its V fragments were read in the last phase Y)
  #pragma unroll
    for (int half = 0; half < 2; ++half)
  #pragma unroll
      for (int db = 0; db < DB; ++db)
  #pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[half][db], pA[qb][half], acc[qb][db], 0, 0, 0);
    if constexpr (!CHECKED) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        l_lo[qb] = lrun[qb][0] + lrun[qb][2];
        l_hi[qb] = lrun[qb][1] + lrun[qb][3];
      }
    }
  };
  pass(flag_t<false>{});
  {
    // the workgroup runs the tile again, checked, if a wave's sums overflowed
    // (every lane: those of lanes 16..63 are zero); NaN fails the test
    bool ok = l_lo[0] <= kPipeSumLimit && l_hi[0] <= kPipeSumLimit && l_lo[1] <= kPipeSumLimit &&
              l_hi[1] <= kPipeSumLimit;
    if constexpr (EXACT_LSE) ok = ok && l_ex[0] <= kPipeSumLimit && l_ex[1] <= kPipeSumLimit;
    int* flags = reinterpret_cast<int*>(smem + C::kFlagOff);
    // every lane votes: a ballot inside the lane-0 branch would see lane 0 only
    const int overflowed = __builtin_amdgcn_ballot_w64(!ok) != 0 ? 1 : 0;
    if (lane == 0) flags[wave] = overflowed;
    __syncthreads();
    if ((flags[0] | flags[1] | flags[2] | flags[3]) != 0) pass(flag_t<true>{});
  }

  // The results go to memory through LDS. In the MFMA layout a lane holds
  // pieces of 32 different rows, so a direct store instruction touches 32 rows
  // and the memory pipeline takes it one cache line at a time; staged, each
  // store instruction writes whole rows (1 KB). The staging reuses the K/V
  // slots: no DMA is in flight after the last iteration, and the barrier waits
  // until every wave has read its last fragments. Each wave stages and reads
  // back only its own 64 rows; one wave's LDS operations complete in order, and
  // the waits keep the compiler from moving the reads above the writes.
  // the rounded-P row sum of this lane's query, from lanes 0..15
  float l_q[2];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float lo = __shfl(l_lo[qb], l32 & 15), hi = __shfl(l_hi[qb], l32 & 15);
    l_q[qb] = l32 < 16 ? lo : hi;
  }
  __syncthreads();
  if (ws_index >= 0) {
    // one key range of a split tile: fp32 rows normalised over the range
    char* wst = smem + wave * (64 * C::kWsRow);
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const float l_tot = l_q[qb];
      const float inv = 1.0f / l_tot;
      char* srow = wst + (qb * 32 + l32) * C::kWsRow;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + i * 8 + hh * 4;
          f32x4_t w = {acc[qb][db][i * 4 + 0] * inv, acc[qb][db][i * 4 + 1] * inv, acc[qb][db][i * 4 + 2] * inv,
                       acc[qb][db][i * 4 + 3] * inv};
          *(f32x4_t*)(srow + d0 * 4) = w;
        }
      const size_t r = (size_t)ws_index * C::kBR + wave * 64 + qb * 32 + l32;
      if (hh == 0) split.ws_lse[r] = mc[qb] + __log2f(l_tot);
      if constexpr (EXACT_LSE) {
        const float l_exact = pair_sum(l_ex[qb]);
        if (hh == 0) split.ws_lse_out[r] = mc[qb] + __log2f(l_exact);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    float* wrows = split.ws_o + ((size_t)ws_index * C::kBR + wave * 64) * D;
    const int c32 = lane & 31;
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const int rl = r * 2 + (lane >> 5);
      *(f32x4_t*)(wrows + rl * D + c32 * 4) = *(const f32x4_t*)(wst + rl * C::kWsRow + c32 * 16);
    }
    return;
  }
  char* ost = smem + wave * (64 * C::kORow);
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float inv = 1.0f / l_q[qb];
    char* srow = ost + (qb * 32 + l32) * C::kORow;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + hh * 4;
        uint2 w;
        w.x = pack_bf16x2(acc[qb][db][i * 4 + 0] * inv, acc[qb][db][i * 4 + 1] * inv);
        w.y = pack_bf16x2(acc[qb][db][i * 4 + 2] * inv, acc[qb][db][i * 4 + 3] * inv);
        *(uint2*)(srow + d0 * 2) = w;
      }
    if constexpr (EXACT_LSE) {
      const float l_exact = pair_sum(l_ex[qb]);
      const int row = q0 + qb * 32 + l32;
      if (hh == 0 && row < N) LSEg[(size_t)bh * N + row] = (mc[qb] + __log2f(l_exact)) * 0.6931471805599453f;
    }
  }
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

// EXACT_LSE: the form that writes a log-sum-exp (LSEg non-null).
template <class C, bool SPARSE, bool EXACT_LSE>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_bf16_pipe_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                               const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                               float* __restrict__ LSEg, int N, int n_qtiles, float scale_log2, float scale,
                               PipeSplit split, Layout L, KvBlocks kvb = KvBlocks{nullptr, nullptr, 0}) {
  const int n_t = (N + 63) / 64;
  // query tile and key-tile range [u0, u1) of this workgroup
  int tile, u0 = 0, u1 = n_t, ws_index = -1, part = 0;
  if ((int)blockIdx.x < split.n_full) {
    tile = xcd_remap(blockIdx.x, split.n_full);
  } else {
    // neighbouring indices (one XCD) share a key range: K/V reuse in L2
    const int sidx = xcd_remap(blockIdx.x - split.n_full, gridDim.x - split.n_full);
    part = sidx / split.n_split;
    const int ti = sidx - part * split.n_split;
    tile = split.n_full + ti;
    u0 = part * n_t / split.parts;
    u1 = (part + 1) * n_t / split.parts;
    ws_index = part * split.n_split + ti;
  }
  pipe_tile<C, SPARSE, EXACT_LSE>(Qg, Kg, Vg, Og, LSEg, N, n_qtiles, scale_log2, split, L, kvb, tile, u0, u1,
                                  ws_index, part);
}

// Stream-K schedule: `groups` workgroups (one per CU) cut the tiles * n_t
// (query tile, key tile) pairs of the call into equal contiguous ranges, so
// that every CU does the same work whatever the tile count. A range meets at
// most two tiles partly: the rows of its first tile (if partial) go to
// workspace slot 2 g, those of its last (if partial, and another tile) to
// 2 g + 1, and attn_streamk_combine_kernel merges each cut tile; tiles the
// range covers whole are written directly.
struct StreamK {
  float* ws_o;     // [2 groups][256][128]
  float* ws_lse;   // [2 groups][256], log2 units: the merge weights of O (rounded-P sums)
  float* ws_lse_out;  // NULL, or [2 groups][256]: the exact sums, for the LSE output
  int groups;
  int tiles;       // query tiles of the call
};

template <class C, bool EXACT_LSE>
__global__ __launch_bounds__(C::kThreads) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_fwd_bf16_streamk_kernel(const uint16_t* __restrict__ Qg, const uint16_t* __restrict__ Kg,
                                  const uint16_t* __restrict__ Vg, uint16_t* __restrict__ Og,
                                  float* __restrict__ LSEg, int N, int n_qtiles, float scale_log2, StreamK sk,
                                  Layout L) {
  const int n_t = (N + 63) / 64;
  const long long work = (long long)sk.tiles * n_t;
  // neighbouring groups (one XCD) share the tile cut between them: K/V reuse in L2
  const int g = xcd_remap(blockIdx.x, gridDim.x);
  const long long s = work * g / sk.groups, e = work * (g + 1) / sk.groups;
  const PipeSplit ws{0, 0, 1, sk.ws_o, sk.ws_lse, sk.ws_lse_out};
  for (long long pos = s; pos < e;) {
    const int tile = (int)(pos / n_t);
    const int u0 = (int)(pos - (long long)tile * n_t);
    const int u1 = (int)min((long long)n_t, (long long)u0 + (e - pos));
    const int slot = (u0 == 0 && u1 == n_t) ? -1 : (pos == s ? 2 * g : 2 * g + 1);
    pipe_tile<C, false, EXACT_LSE>(Qg, Kg, Vg, Og, LSEg, N, n_qtiles, scale_log2, ws, L,
                                   KvBlocks{nullptr, nullptr, 0}, tile, u0, u1, slot, 0);
    __syncthreads();       // every wave is done with the LDS slots before the next tile's DMA
    pos += u1 - u0;
  }
}

// Merges the tiles cut by stream-K range boundaries. Block (b, 64-row chunk):
// boundary b (1 .. groups - 1) starts group b; the first boundary inside a
// tile merges that tile's parts, from the group whose range holds the tile's
// first key tile to the one holding its last. A group's part is slot 2 g if
// the part starts the group's range, else 2 g + 1. The boundary arithmetic
// is done once per block; each thread then takes 4 values of 8 rows, four
// rows' loads in flight at a time.
constexpr int kStreamKMergeRows = 64;
constexpr int kStreamKMaxParts = 16;          // parts of one cut tile; the planner keeps ranges long enough
__global__ __launch_bounds__(256) void attn_streamk_combine_kernel(uint16_t* __restrict__ Og, float* __restrict__ LSEg,
                                                                   int N, int n_qtiles, StreamK sk, Layout L) {
  constexpr int D = PipeCfg::kD, BR = PipeCfg::kBR, CHUNKS = BR / kStreamKMergeRows;
  constexpr int kMaxParts = kStreamKMaxParts;
  const int b = blockIdx.x / CHUNKS + 1;
  const int chunk = blockIdx.x % CHUNKS;
  const int n_t = (N + 63) / 64;
  const long long work = (long long)sk.tiles * n_t;
  auto start = [&](int g) { return work * g / sk.groups; };
  const long long pb = start(b);
  const int tile = (int)(pb / n_t);
  const long long t0 = (long long)tile * n_t, t1 = t0 + n_t;
  if (pb == t0) return;                       // the boundary falls on a tile edge
  if (start(b - 1) > t0) return;              // an earlier boundary in this tile merges it
  // the parts: group b - 1 (its range reaches into the tile from before, or
  // starts at its first key tile), then b, b + 1, ... while they start in it
  int slots[kMaxParts];
  int n_parts = 0;
  slots[n_parts++] = start(b - 1) >= t0 ? 2 * (b - 1) : 2 * (b - 1) + 1;
  for (int g = b; g < sk.groups && n_parts < kMaxParts; ++g) {
    const long long sg = start(g);
    if (sg >= t1) break;
    if (start(g + 1) > sg) slots[n_parts++] = 2 * g;     // a group with no work has no part
  }
  const int bh = tile / n_qtiles, qt = tile - bh * n_qtiles;
  const int c = (threadIdx.x & 31) * 4;
#pragma unroll 4
  for (int rr = 0; rr < kStreamKMergeRows / 8; ++rr) {
    const int r = chunk * kStreamKMergeRows + rr * 8 + (threadIdx.x >> 5);
    const int row = qt * BR + r;
    if (row >= N) break;
    float mx = -INFINITY;
    for (int i = 0; i < n_parts; ++i) mx = fmaxf(mx, sk.ws_lse[(size_t)slots[i] * BR + r]);
    float wsum = 0.f;
    f32x4_t o = {0.f, 0.f, 0.f, 0.f};
    for (int i = 0; i < n_parts; ++i) {
      const size_t idx = (size_t)slots[i] * BR + r;
      const float w = fast_exp2(sk.ws_lse[idx] - mx);
      wsum += w;
      o += w * *(const f32x4_t*)(sk.ws_o + idx * D + c);
    }
    const float inv = 1.0f / wsum;
    uint2 out;
    out.x = pack_bf16x2(o[0] * inv, o[1] * inv);
    out.y = pack_bf16x2(o[2] * inv, o[3] * inv);
    *(uint2*)(Og + L.out_off(bh) + (long long)row * L.on + c) = out;
    if (LSEg != nullptr && c == 0) {
      // the exact sums of the parts (the merge weights above are the rounded-P sums)
      float lmx = -INFINITY, lsum = 0.f;
      for (int i = 0; i < n_parts; ++i) lmx = fmaxf(lmx, sk.ws_lse_out[(size_t)slots[i] * BR + r]);
      for (int i = 0; i < n_parts; ++i) lsum += fast_exp2(sk.ws_lse_out[(size_t)slots[i] * BR + r] - lmx);
      LSEg[(size_t)bh * N + row] = (lmx + __log2f(lsum)) * 0.6931471805599453f;
    }
  }
}

#undef DIT_FENCE

// Merges the key-range parts of the split query tiles: per row,
// O = sum_p w_p O_p / sum_p w_p with w_p = 2^(lse_p - max_p lse_p). Eight
// rows per 256-thread block, four d values per thread.
__global__ __launch_bounds__(256) void attn_split_combine_kernel(const float* __restrict__ ws_o,
                                                                 const float* __restrict__ ws_lse,
                                                                 uint16_t* __restrict__ Og, float* __restrict__ LSEg,
                                                                 int N, int n_qtiles, PipeSplit split, Layout L) {
  constexpr int D = PipeCfg::kD, BR = PipeCfg::kBR;
  const int ti = blockIdx.x / (BR / 8);
  const int r = (blockIdx.x % (BR / 8)) * 8 + (threadIdx.x >> 5);
  const int c = (threadIdx.x & 31) * 4;
  const int tile = split.n_full + ti;
  const int bh = tile / n_qtiles, qt = tile - bh * n_qtiles;
  const int row = qt * BR + r;
  if (row >= N) return;
  float mx = -INFINITY;
  for (int p = 0; p < split.parts; ++p) mx = fmaxf(mx, ws_lse[(size_t)(p * split.n_split + ti) * BR + r]);
  if (mx == -INFINITY) {
    // every part empty (block-sparse lists only): attention over no key
    *(uint2*)(Og + L.out_off(bh) + (long long)row * L.on + c) = uint2{0u, 0u};
    if (LSEg != nullptr && c == 0) LSEg[(size_t)bh * N + row] = -INFINITY;
    return;
  }
  float wsum = 0.f;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  float lse_mx = mx, lse_sum = 0.f;    // the LSE output's own sums when ws_lse_out is given
  if (LSEg != nullptr && split.ws_lse_out != nullptr && c == 0) {
    lse_mx = -INFINITY;
    for (int p = 0; p < split.parts; ++p)
      lse_mx = fmaxf(lse_mx, split.ws_lse_out[(size_t)(p * split.n_split + ti) * BR + r]);
    for (int p = 0; p < split.parts; ++p)
      lse_sum += fast_exp2(split.ws_lse_out[(size_t)(p * split.n_split + ti) * BR + r] - lse_mx);
  }
  for (int p = 0; p < split.parts; ++p) {
    const size_t idx = (size_t)(p * split.n_split + ti) * BR + r;
    const float w = fast_exp2(ws_lse[idx] - mx);
    wsum += w;
    const f32x4_t x = *(const f32x4_t*)(ws_o + idx * D + c);
    o += w * x;
  }
  const float inv = 1.0f / wsum;
  uint2 out;
  out.x = pack_bf16x2(o[0] * inv, o[1] * inv);
  out.y = pack_bf16x2(o[2] * inv, o[3] * inv);
  *(uint2*)(Og + L.out_off(bh) + (long long)row * L.on + c) = out;
  if (LSEg != nullptr && c == 0)
    LSEg[(size_t)bh * N + row] =
        (split.ws_lse_out != nullptr ? lse_mx + __log2f(lse_sum) : mx + __log2f(wsum)) * 0.6931471805599453f;
}

}  // namespace ditattn
