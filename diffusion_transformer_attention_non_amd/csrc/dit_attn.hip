// C ABI of the gfx950 DiT attention library: argument checks, device check,
// kernel selection and launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "dit_attn.h"
#include "attn_fwd_bf16.h"
#include "attn_fwd_bf16_pipe.h"
#include "attn_fwd_fp8_pipe.h"
#include "quant_e4m3.h"
#include "quant_mx.h"
#include "mfma_ceiling.h"

using namespace ditattn;

namespace {

constexpr int kMaxDevices = 64;
// 0 = not checked yet, 1 = gfx950 and kernels configured, 2 = unsupported device
std::atomic<int> g_device_state[kMaxDevices];
// compute units per device (set with the device state)
std::atomic<int> g_num_cu[kMaxDevices];   // published by g_device_state's release

// Kernel configurations. bf16 d = 128 runs the 64-rows-per-wave pipelined
// kernel (256 rows per workgroup); d = 64 the 32-rows-per-wave kernel with
// BR = NW * QB * 32 rows per workgroup.
using CfgBf16D128 = PipeCfg;
using CfgBf16D64 = Bf16Cfg<64, 1, 8, 64, 2>;
using CfgFp8D128 = Fp8PipeCfg;

template <class C>
hipError_t allow_lds_bf16() {
  return hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_fwd_bf16_kernel<C>),
                             hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
}
template <class C>
hipError_t allow_lds_pipe() {
  const void* kernels[6] = {reinterpret_cast<const void*>(&attn_fwd_bf16_pipe_kernel<C, false, false>),
                            reinterpret_cast<const void*>(&attn_fwd_bf16_pipe_kernel<C, false, true>),
                            reinterpret_cast<const void*>(&attn_fwd_bf16_pipe_kernel<C, true, false>),
                            reinterpret_cast<const void*>(&attn_fwd_bf16_pipe_kernel<C, true, true>),
                            reinterpret_cast<const void*>(&attn_fwd_bf16_streamk_kernel<C, false>),
                            reinterpret_cast<const void*>(&attn_fwd_bf16_streamk_kernel<C, true>)};
  for (const void* k : kernels) {
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
template <class C>
hipError_t allow_lds_fp8() {
  const void* kernels[4] = {reinterpret_cast<const void*>(&attn_fwd_fp8_pipe_kernel<C, false, false>),
                            reinterpret_cast<const void*>(&attn_fwd_fp8_pipe_kernel<C, true, false>),
                            reinterpret_cast<const void*>(&attn_fwd_fp8_pipe_kernel<C, false, true>),
                            reinterpret_cast<const void*>(&attn_fwd_fp8_pipe_kernel<C, true, true>)};
  for (const void* k : kernels) {
    const hipError_t e = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, C::kLdsBytes);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return DIT_ATTN_EDEVICE;
  int state = dev < kMaxDevices ? g_device_state[dev].load(std::memory_order_acquire) : 0;
  if (state == 1) return DIT_ATTN_OK;
  if (state == 2) return DIT_ATTN_EDEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DIT_ATTN_EDEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (ok) {
    if (allow_lds_pipe<CfgBf16D128>() != hipSuccess || allow_lds_bf16<CfgBf16D64>() != hipSuccess ||
        allow_lds_fp8<CfgFp8D128>() != hipSuccess)
      return DIT_ATTN_EDEVICE;
    for (const void* k : {reinterpret_cast<const void*>(&mfma_ceiling_kernel<false>),
                          reinterpret_cast<const void*>(&mfma_ceiling_kernel<true>)})
      if (hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, kCeilingLds) != hipSuccess)
        return DIT_ATTN_EDEVICE;
  }
  if (ok && dev < kMaxDevices) {
    int n_cu = 0;
    if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n_cu <= 0)
      return DIT_ATTN_EDEVICE;
    g_num_cu[dev].store(n_cu, std::memory_order_relaxed);
  }
  if (dev < kMaxDevices) g_device_state[dev].store(ok ? 1 : 2, std::memory_order_release);
  return ok ? DIT_ATTN_OK : DIT_ATTN_EDEVICE;
}

int cu_count() {
  int dev = 0;
  (void)hipGetDevice(&dev);
  const int n = dev >= 0 && dev < kMaxDevices ? g_num_cu[dev].load(std::memory_order_relaxed) : 0;
  return n > 0 ? n : 256;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, uint64_t na, const void* b, uint64_t nb) {
  const uintptr_t pa = reinterpret_cast<uintptr_t>(a), pb = reinterpret_cast<uintptr_t>(b);
  return pa < pb + nb && pb < pa + na;
}

// Checks one tensor's (batch, head, token) element strides and returns the
// byte span its rows cover from the base pointer. Rows are d contiguous
// elements; every row start must stay 16-byte aligned; a token stride below d
// would overlap rows. For an output the map (b, h, n) -> row must be one to
// one: taken by increasing stride, each dimension of size > 1 must step past
// everything the smaller ones cover. Inputs may repeat rows (stride 0 shares
// one head's K and V among heads).
bool check_strides(const int64_t* s, int B, int H, int N, int d, unsigned esize, bool output, uint64_t* span) {
  for (int i = 0; i < 3; ++i)
    if (s[i] < 0 || s[i] > ((int64_t)1 << 40) || (s[i] * (int64_t)esize) % 16 != 0) return false;
  if (s[2] < d) return false;
  const unsigned __int128 last = (unsigned __int128)(B - 1) * (uint64_t)s[0] + (unsigned __int128)(H - 1) * (uint64_t)s[1] +
                                 (unsigned __int128)(N - 1) * (uint64_t)s[2] + (unsigned)d;
  if (last * esize >= ((unsigned __int128)1 << 62)) return false;
  *span = (uint64_t)(last * esize);
  if (output) {
    int64_t st[3] = {s[0], s[1], s[2]};
    int64_t sz[3] = {B, H, N};
    for (int i = 0; i < 3; ++i)          // sort by stride
      for (int j = i + 1; j < 3; ++j)
        if (st[j] < st[i]) { std::swap(st[i], st[j]); std::swap(sz[i], sz[j]); }
    unsigned __int128 cover = (unsigned)d;
    for (int i = 0; i < 3; ++i) {
      if (sz[i] == 1) continue;
      if ((unsigned __int128)st[i] < cover) return false;
      cover = (unsigned __int128)st[i] * (uint64_t)(sz[i] - 1) + cover;
    }
  }
  return true;
}

template <class C>
int launch_bf16(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                float scale, hipStream_t st, const Layout& L) {
  const int n_qtiles = (N + C::kBR - 1) / C::kBR;
  const long long grid = (long long)n_qtiles * BH;
  if (grid > 0x7fffffffLL) return DIT_ATTN_EINVAL;
  const float scale_log2 = scale * 1.4426950408889634f;
  hipLaunchKernelGGL(attn_fwd_bf16_kernel<C>, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qtiles,
                     scale_log2, scale, L);
  return hipGetLastError() == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

// One workgroup (256 query rows) runs per CU, so a grid of T tiles takes
// ceil(T / n_cu) rounds and the last round holds rem = T mod n_cu tiles. Those
// are split into `parts` contiguous key ranges that run side by side, and a
// combine kernel merges them; the fp32 partial rows live in a stream-ordered
// allocation freed after the merge. `parts` minimises the modelled time of
// the last round, ceil(rem * parts / n_cu) * (1/parts + kPartOverhead / n_t)
// in units of one full tile (each range pays about kPartOverhead key tiles of
// prologue and epilogue), with at least 4 key tiles per range and at most
// kMaxSplitRows partial rows. parts = 1 (no split) when nothing is gained.
constexpr double kPartOverhead = 2.0;
// Partial rows of one call, split or stream-K: 128 Ki rows x 129 floats =
// 67.6 MB (+ 0.5 MB of exact LSE sums for fp8 with an LSE output).
constexpr long long kMaxSplitRows = 1 << 17;

int plan_split(int BH, int n_qtiles, int N, int key_tile, int n_cu, PipeSplit* sp) {
  const int tiles = BH * n_qtiles;
  *sp = PipeSplit{tiles, 0, 1, nullptr, nullptr};
  const int rem = tiles % n_cu;
  const int n_t = (N + key_tile - 1) / key_tile;
  if (rem == 0) return 0;
  int best = 1;
  double best_cost = 1.0;
  const int max_parts = std::min<long long>(n_t / 4, kMaxSplitRows / (256LL * rem));
  for (int parts = 2; parts <= max_parts; ++parts) {
    const long long waves = ((long long)rem * parts + n_cu - 1) / n_cu;
    const double cost = (double)waves * (1.0 / parts + kPartOverhead / n_t);
    if (cost < best_cost * 0.98) { best_cost = cost; best = parts; }   // more parts only for a clear gain
  }
  if (best < 2) return 0;
  sp->n_full = tiles - rem;
  sp->n_split = rem;
  sp->parts = best;
  return 1;
}

// Cost of a schedule in key tiles on the busiest CU, each tile a workgroup
// touches adding kPartOverhead (prologue, epilogue). The split plan: its full
// rounds, then the last round's parts. Stream-K: the equal share, touching
// share / n_t + 1 tiles.
double split_cost(const PipeSplit& sp, int tiles, int n_t, int n_cu) {
  if (sp.n_split == 0) return (double)((tiles + n_cu - 1) / n_cu) * (n_t + kPartOverhead);
  const long long waves = ((long long)sp.n_split * sp.parts + n_cu - 1) / n_cu;
  return (double)(sp.n_full / n_cu) * (n_t + kPartOverhead) + (double)waves * ((double)n_t / sp.parts + kPartOverhead);
}
double streamk_cost(int tiles, int n_t, int groups) {
  const double share = (double)tiles * n_t / groups;
  return share + kPartOverhead * (share / n_t + 1.0);
}
constexpr int kStreamKMinKeyTiles = 4;        // per group

// The schedule of one call, decided on the host from its shape alone (never
// from the data). Both the launch and dit_attn_plan use this.
enum PlanKind { kPlanBf16D128 = 0, kPlanBf16D128Sparse = 1, kPlanFp8D128 = 2, kPlanBf16D64 = 3 };
struct Plan {
  int schedule;          // DIT_ATTN_SCHED_*
  PipeSplit sp;          // split: n_full, n_split, parts (workspace pointers unset)
  int groups;            // stream-K workgroups
  long long workgroups;  // of the attention kernel
  size_t units;          // partial rows in the workspace
  size_t ws_floats;      // workspace size in floats
  int best_schedule;     // the fastest schedule (what a large enough workspace buys)
  size_t wanted_floats;  // its workspace size in floats
};

int make_plan(int kind, long long BH, int N, int n_cu, int max_blocks, bool lse, Plan* p) {
  const int br = kind == kPlanBf16D64 ? CfgBf16D64::kBR : CfgBf16D128::kBR;
  const long long n_qtiles = (N + br - 1) / br;
  const long long tiles = n_qtiles * BH;
  if (tiles > 0x7fffffffLL / 8) return DIT_ATTN_EINVAL;
  *p = Plan{DIT_ATTN_SCHED_TILE, PipeSplit{(int)tiles, 0, 1, nullptr, nullptr, nullptr}, 0, tiles, 0, 0,
            DIT_ATTN_SCHED_TILE, 0};
  if (kind == kPlanBf16D64) return DIT_ATTN_OK;
  constexpr int kD = CfgBf16D128::kD, kBR = CfgBf16D128::kBR;
  if (kind == kPlanBf16D128) {
    const int n_t = (N + 63) / 64;
    // ranges of at least 4 key tiles, and long enough that a tile meets at
    // most kStreamKMaxParts - 1 of them (the merge's limit): boundaries in a
    // tile are a range apart, so a range of ceil(n_t / (max - 3)) key tiles
    // puts at most max - 2 of them inside it
    const long long min_range =
        std::max<long long>(kStreamKMinKeyTiles, (n_t + kStreamKMaxParts - 4) / (kStreamKMaxParts - 3));
    const int groups = (int)std::min<long long>(std::min<long long>(n_cu, kMaxSplitRows / (2 * kBR)),
                                                tiles * n_t / min_range);
    PipeSplit alt;
    plan_split((int)tiles, 1, N, 64, n_cu, &alt);
    // Stream-K only up to two rounds of tiles: a CU's range then stays in
    // one or two heads. With more rounds the ranges run through every head at
    // once and K/V stop fitting the caches (measured 7-8% slower at H = 12
    // and 24 of the 16896-token call, where the split plan does well).
    if (groups >= 2 && tiles <= 2LL * n_cu &&
        streamk_cost((int)tiles, n_t, groups) < split_cost(alt, (int)tiles, n_t, n_cu)) {
      p->schedule = DIT_ATTN_SCHED_STREAMK;
      p->groups = groups;
      p->workgroups = groups;
      p->units = (size_t)2 * groups * kBR;
      // with an LSE output, exact sums of their own besides the rounded-P merge weights
      p->ws_floats = p->units * (kD + 1) + (lse ? p->units : 0);
      return DIT_ATTN_OK;
    }
  }
  const int keys = kind == kPlanBf16D128Sparse ? max_blocks * 64 : N;
  const int key_tile = kind == kPlanFp8D128 ? CfgFp8D128::kKB : 64;
  if (plan_split((int)BH, (int)n_qtiles, keys, key_tile, n_cu, &p->sp)) {
    p->schedule = DIT_ATTN_SCHED_SPLIT;
    p->workgroups = (long long)p->sp.n_full + (long long)p->sp.n_split * p->sp.parts;
    p->units = (size_t)p->sp.n_split * p->sp.parts * kBR;
    // with an LSE output: O's merge weights come from the sums of the rounded
    // P (bf16 or e4m3), the LSE from exact sums of its own
    p->ws_floats = p->units * (kD + 1) + (lse ? p->units : 0);
  }
  return DIT_ATTN_OK;
}

// The plan of a call given `ws_bytes` of caller workspace: the fastest
// schedule if the workspace holds its partial rows, one workgroup per tile
// if no workspace is given, DIT_ATTN_EWORKSPACE for a workspace that is given
// but too small (a caller that passes one expects it to be used).
int resolve_plan(int kind, long long BH, int N, int n_cu, int max_blocks, bool lse, int64_t ws_bytes, Plan* p) {
  if (ws_bytes < 0) return DIT_ATTN_EINVAL;
  const int st = make_plan(kind, BH, N, n_cu, max_blocks, lse, p);
  if (st != DIT_ATTN_OK) return st;
  p->best_schedule = p->schedule;
  p->wanted_floats = p->ws_floats;
  const uint64_t need = (uint64_t)p->ws_floats * sizeof(float);
  if (need == 0 || (uint64_t)ws_bytes >= need) return DIT_ATTN_OK;
  if (ws_bytes != 0) return DIT_ATTN_EWORKSPACE;
  const long long tiles = p->sp.n_full + (long long)p->sp.n_split;
  p->schedule = DIT_ATTN_SCHED_TILE;
  p->sp = PipeSplit{(int)tiles, 0, 1, nullptr, nullptr, nullptr};
  p->groups = 0;
  p->workgroups = tiles;
  p->units = 0;
  p->ws_floats = 0;
  return DIT_ATTN_OK;
}

// Dense bf16 d = 128 under stream-K: `groups` workgroups, partial rows in the
// workspace's 2 groups slots, merged by the combine kernel.
template <class C>
int launch_streamk(const void* q, const void* k, const void* v, void* o, float* lse, int tiles, int N,
                   int n_qtiles, float scale_log2, hipStream_t st, int groups, const Layout& L, void* ws) {
  const size_t units = (size_t)2 * groups * C::kBR;
  float* wsf = static_cast<float*>(ws);
  StreamK sk{wsf, wsf + units * C::kD, lse != nullptr ? wsf + units * (C::kD + 1) : nullptr, groups, tiles};
  auto* kernel = lse != nullptr ? &attn_fwd_bf16_streamk_kernel<C, true> : &attn_fwd_bf16_streamk_kernel<C, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)groups), dim3(C::kThreads), C::kLdsBytes, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qtiles, scale_log2, sk,
                     L);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && groups > 1) {
    hipLaunchKernelGGL(attn_streamk_combine_kernel, dim3((unsigned)((groups - 1) * (C::kBR / kStreamKMergeRows))),
                       dim3(256), 0, st,
                       static_cast<uint16_t*>(o), lse, N, n_qtiles, sk, L);
    err = hipGetLastError();
  }
  return err == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

// SPARSE: block lists in kvb; the split planner then takes max_blocks as
// the key-tile count (the host never reads the lists). `plan` comes from
// resolve_plan; ws holds its partial rows (unused without them).
template <class C, bool SPARSE = false>
int launch_pipe(const void* q, const void* k, const void* v, void* o, float* lse, int BH, int N,
                float scale, hipStream_t st, const Plan& plan, void* ws, const Layout& L,
                const KvBlocks& kvb = KvBlocks{}) {
  const int n_qtiles = (N + C::kBR - 1) / C::kBR;
  const int tiles = n_qtiles * BH;
  const float scale_log2 = scale * 1.4426950408889634f;
  if (plan.schedule == DIT_ATTN_SCHED_STREAMK)
    return launch_streamk<C>(q, k, v, o, lse, tiles, N, n_qtiles, scale_log2, st, plan.groups, L, ws);
  PipeSplit sp = plan.sp;
  if (plan.schedule == DIT_ATTN_SCHED_SPLIT) {
    sp.ws_o = static_cast<float*>(ws);
    sp.ws_lse = sp.ws_o + plan.units * C::kD;
    sp.ws_lse_out = lse != nullptr ? sp.ws_lse + plan.units : nullptr;
  }
  const long long grid = (long long)sp.n_full + (long long)sp.n_split * sp.parts;
  auto* kernel = lse != nullptr ? &attn_fwd_bf16_pipe_kernel<C, SPARSE, true> : &attn_fwd_bf16_pipe_kernel<C, SPARSE, false>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, st,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(o), lse, N, n_qtiles,
                     scale_log2, scale, sp, L, kvb);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && plan.schedule == DIT_ATTN_SCHED_SPLIT) {
    hipLaunchKernelGGL(attn_split_combine_kernel, dim3((unsigned)(sp.n_split * (C::kBR / 8))), dim3(256), 0, st,
                       sp.ws_o, sp.ws_lse, static_cast<uint16_t*>(o), lse, N, n_qtiles, sp, L);
    err = hipGetLastError();
  }
  return err == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

// MX: block-scaled inputs with their scales in mxs (descale unused)
template <class C, bool MX = false>
int launch_fp8(const void* q, const void* k, const void* v, void* o, float* lse, const float* descale,
               int BH, int N, float scale, hipStream_t st, const Plan& plan, void* ws, const Layout& L,
               const MxScales& mxs = MxScales{nullptr, nullptr, nullptr}) {
  static_assert(C::kBR == PipeCfg::kBR && C::kD == PipeCfg::kD, "the merge kernel assumes 256 x 128 tiles");
  const int n_qtiles = (N + C::kBR - 1) / C::kBR;
  const float scale_log2 = scale * 1.4426950408889634f;
  PipeSplit sp = plan.sp;
  if (plan.schedule == DIT_ATTN_SCHED_SPLIT) {
    sp.ws_o = static_cast<float*>(ws);
    sp.ws_lse = sp.ws_o + plan.units * C::kD;
    sp.ws_lse_out = lse != nullptr ? sp.ws_lse + plan.units : nullptr;
  }
  const long long grid = (long long)sp.n_full + (long long)sp.n_split * sp.parts;
  auto* kernel = lse != nullptr ? &attn_fwd_fp8_pipe_kernel<C, true, MX> : &attn_fwd_fp8_pipe_kernel<C, false, MX>;
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(C::kThreads), C::kLdsBytes, st,
                     static_cast<const uint8_t*>(q), static_cast<const uint8_t*>(k),
                     static_cast<const uint8_t*>(v), static_cast<uint16_t*>(o), lse, descale, N, n_qtiles,
                     scale_log2, scale, sp, L, mxs);
  hipError_t err = hipGetLastError();
  if (err == hipSuccess && plan.schedule == DIT_ATTN_SCHED_SPLIT) {
    hipLaunchKernelGGL(attn_split_combine_kernel, dim3((unsigned)(sp.n_split * (C::kBR / 8))), dim3(256), 0, st,
                       sp.ws_o, sp.ws_lse, static_cast<uint16_t*>(o), lse, N, n_qtiles, sp, L);
    err = hipGetLastError();
  }
  return err == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

// What check_call derives from valid arguments.
struct Checked {
  Layout L;
  int bh;
  uint64_t in_bytes, out_bytes, lse_bytes;   // byte spans of q (k, v), o, lse
};

// Host checks shared by the attention entry points; no device call.
int check_call(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, float scale,
               int dtype, const int64_t* qkv_strides, const int64_t* o_strides, const float* descale_qkv,
               float* lse, Checked* c) {
  if (!q || !k || !v || !o) return DIT_ATTN_EINVAL;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16)) return DIT_ATTN_EINVAL;
  if (lse && !aligned(lse, 4)) return DIT_ATTN_EINVAL;
  if (descale_qkv && !aligned(descale_qkv, 4)) return DIT_ATTN_EINVAL;
  if (B < 1 || H < 1 || N < 1) return DIT_ATTN_EINVAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return DIT_ATTN_EINVAL;
  if (dtype != DIT_ATTN_BF16 && dtype != DIT_ATTN_FP8_E4M3) return DIT_ATTN_EUNSUPPORTED;
  if (dtype == DIT_ATTN_BF16 && d != 64 && d != 128) return DIT_ATTN_EUNSUPPORTED;
  if (dtype == DIT_ATTN_FP8_E4M3 && d != 128) return DIT_ATTN_EUNSUPPORTED;
  const long long bh = (long long)B * H;
  if (bh > 0x7fffffffLL) return DIT_ATTN_EINVAL;
  // contiguous [B][H][N][d] unless strides are given (larger than any valid
  // stride when H N d does not fit, which check_strides then rejects)
  const unsigned __int128 hnd = (unsigned __int128)(unsigned)H * (unsigned)N * (unsigned)d;
  const int64_t big = (int64_t)1 << 41;
  const int64_t contig[3] = {hnd < (unsigned __int128)big ? (int64_t)hnd : big, (int64_t)N * d, d};
  const int64_t* si = qkv_strides ? qkv_strides : contig;
  const int64_t* so = o_strides ? o_strides : contig;
  const unsigned in_size = dtype == DIT_ATTN_BF16 ? 2u : 1u;
  uint64_t in_bytes = 0, out_bytes = 0;
  if (!check_strides(si, B, H, N, d, in_size, false, &in_bytes)) return DIT_ATTN_EINVAL;
  if (!check_strides(so, B, H, N, d, 2u, true, &out_bytes)) return DIT_ATTN_EINVAL;
  // a 128-key tile of q, k or v must span < 2^31 bytes (32-bit DMA offsets)
  if (si[2] * (int64_t)in_size * 128 >= ((int64_t)1 << 31)) return DIT_ATTN_EINVAL;
  if (overlap(o, out_bytes, q, in_bytes) || overlap(o, out_bytes, k, in_bytes) ||
      overlap(o, out_bytes, v, in_bytes))
    return DIT_ATTN_EINVAL;
  const uint64_t lse_bytes = (uint64_t)bh * (uint64_t)N * 4u;
  if (lse) {
    if (overlap(lse, lse_bytes, q, in_bytes) || overlap(lse, lse_bytes, k, in_bytes) ||
        overlap(lse, lse_bytes, v, in_bytes) || overlap(lse, lse_bytes, o, out_bytes))
      return DIT_ATTN_EINVAL;
  }
  *c = Checked{Layout{si[0], si[1], si[2], so[0], so[1], so[2], H}, (int)bh, in_bytes, out_bytes, lse_bytes};
  return DIT_ATTN_OK;
}

// A workspace of ws_bytes > 0 must be a 16-byte aligned pointer that overlaps
// none of the n buffers (pointer, byte span; NULL pointers are skipped).
// ws_bytes == 0 means no workspace, whatever the pointer.
int check_workspace(const void* ws, int64_t ws_bytes, const void* const* bufs, const uint64_t* spans, int n) {
  if (ws_bytes < 0) return DIT_ATTN_EINVAL;
  if (ws_bytes == 0) return DIT_ATTN_OK;
  if (ws == nullptr || !aligned(ws, 16)) return DIT_ATTN_EINVAL;
  for (int i = 0; i < n; ++i)
    if (bufs[i] != nullptr && overlap(ws, (uint64_t)ws_bytes, bufs[i], spans[i])) return DIT_ATTN_EINVAL;
  return DIT_ATTN_OK;
}

// The library's own scratch for dit_attn_fwd_noalloc: every plan's partial
// rows fit (kMaxSplitRows rows of kD + 1 floats, plus kMaxSplitRows floats of
// exact LSE sums for fp8). Each GPU the library runs on holds one copy until
// the process ends. Host code never uses the array's name as an address: the
// kernels get the device address hipGetSymbolAddress returns for the current
// device, looked up once per device on the entry point's first call there.
constexpr size_t kScratchBytes = (size_t)kMaxSplitRows * (PipeCfg::kD + 1) * sizeof(float) +
                                 (size_t)kMaxSplitRows * sizeof(float);   // 65 MiB
static_assert(kScratchBytes == DIT_ATTN_NOALLOC_SCRATCH_BYTES, "the header states the scratch size");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::atomic<void*> g_scratch_ptr[kMaxDevices];

// Device address of the current device's scratch array, or nullptr.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr != nullptr) return ptr;
  if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  return ptr;
}

int plan_kind(int d, int dtype, int max_blocks) {
  return dtype == DIT_ATTN_FP8_E4M3 ? kPlanFp8D128
         : d == 64                  ? kPlanBf16D64
         : max_blocks > 0           ? kPlanBf16D128Sparse
                                    : kPlanBf16D128;
}

}  // namespace

extern "C" {

int dit_attn_version(void) { return (2 << 16) | 1; }

int dit_attn_mfma_ceiling(int dtype, int rounds, int workgroups, void* record, int64_t record_bytes,
                          int* wall_clock_khz, void* stream) {
  if (rounds < 1 || workgroups < 0 || workgroups > (1 << 20) || record == nullptr || record_bytes < 0 ||
      !aligned(record, 8))
    return DIT_ATTN_EINVAL;
  if (dtype != DIT_ATTN_BF16 && dtype != DIT_ATTN_FP8_E4M3) return DIT_ATTN_EUNSUPPORTED;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  const int wg = workgroups > 0 ? workgroups : cu_count();
  if (record_bytes < (int64_t)wg * 4 * 2 * (int64_t)sizeof(long long)) return DIT_ATTN_EWORKSPACE;
  if (wall_clock_khz != nullptr) {
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
      return DIT_ATTN_EDEVICE;
    *wall_clock_khz = khz;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  long long* rec = static_cast<long long*>(record);
  if (dtype == DIT_ATTN_FP8_E4M3)
    hipLaunchKernelGGL(mfma_ceiling_kernel<true>, dim3((unsigned)wg), dim3(256), kCeilingLds, st, rec, rounds);
  else
    hipLaunchKernelGGL(mfma_ceiling_kernel<false>, dim3((unsigned)wg), dim3(256), kCeilingLds, st, rec, rounds);
  return hipGetLastError() == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

const char* dit_attn_strerror(int status) {
  switch (status) {
    case DIT_ATTN_OK: return "ok";
    case DIT_ATTN_EINVAL: return "invalid argument";
    case DIT_ATTN_EUNSUPPORTED: return "unsupported head dimension or dtype";
    case DIT_ATTN_EDEVICE: return "no gfx950 HIP device is current";
    case DIT_ATTN_ELAUNCH: return "kernel launch failed";
    case DIT_ATTN_EWORKSPACE: return "workspace smaller than the call's plan needs";
    default: return "unknown status";
  }
}

int dit_attn_fwd_strided(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                         float scale, int dtype, const int64_t* qkv_strides, const int64_t* o_strides,
                         const float* descale_qkv, float* lse, void* workspace, int64_t workspace_bytes,
                         void* stream) {
  Checked c;
  const int status = check_call(q, k, v, o, B, H, N, d, scale, dtype, qkv_strides, o_strides, descale_qkv, lse, &c);
  if (status != DIT_ATTN_OK) return status;
  const void* bufs[5] = {q, k, v, o, lse};
  const uint64_t spans[5] = {c.in_bytes, c.in_bytes, c.in_bytes, c.out_bytes, c.lse_bytes};
  const int ws_status = check_workspace(workspace, workspace_bytes, bufs, spans, 5);
  if (ws_status != DIT_ATTN_OK) return ws_status;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  Plan plan;
  const int pst = resolve_plan(plan_kind(d, dtype, 0), c.bh, N, cu_count(), 0, lse != nullptr, workspace_bytes, &plan);
  if (pst != DIT_ATTN_OK) return pst;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == DIT_ATTN_BF16) {
    if (d == 128) return launch_pipe<CfgBf16D128>(q, k, v, o, lse, c.bh, N, scale, st, plan, workspace, c.L);
    return launch_bf16<CfgBf16D64>(q, k, v, o, lse, c.bh, N, scale, st, c.L);
  }
  return launch_fp8<CfgFp8D128>(q, k, v, o, lse, descale_qkv, c.bh, N, scale, st, plan, workspace, c.L);
}

int dit_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                         float scale, int dtype, const int64_t* qkv_strides, const int64_t* o_strides,
                         const float* descale_qkv, float* lse, void* stream) {
  Checked c;
  const int status = check_call(q, k, v, o, B, H, N, d, scale, dtype, qkv_strides, o_strides, descale_qkv, lse, &c);
  if (status != DIT_ATTN_OK) return status;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  Plan plan;
  // the scratch array stands in for a workspace of its size: a plan that needs
  // more is refused (DIT_ATTN_EWORKSPACE), never run on a smaller schedule
  const int pst = resolve_plan(plan_kind(d, dtype, 0), c.bh, N, cu_count(), 0, lse != nullptr,
                               (int64_t)kScratchBytes, &plan);
  if (pst != DIT_ATTN_OK) return pst;
  void* ws = nullptr;
  if (plan.ws_floats > 0) {
    ws = scratch_address();
    if (ws == nullptr) return DIT_ATTN_EDEVICE;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (dtype == DIT_ATTN_BF16) {
    if (d == 128) return launch_pipe<CfgBf16D128>(q, k, v, o, lse, c.bh, N, scale, st, plan, ws, c.L);
    return launch_bf16<CfgBf16D64>(q, k, v, o, lse, c.bh, N, scale, st, c.L);
  }
  return launch_fp8<CfgFp8D128>(q, k, v, o, lse, descale_qkv, c.bh, N, scale, st, plan, ws, c.L);
}

int dit_attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                             float scale, int dtype, const int32_t* kv_blocks, const int32_t* kv_counts,
                             int max_blocks, const int64_t* qkv_strides, const int64_t* o_strides, float* lse,
                             void* workspace, int64_t workspace_bytes, void* stream) {
  Checked c;
  const int status = check_call(q, k, v, o, B, H, N, d, scale, dtype, qkv_strides, o_strides, nullptr, lse, &c);
  if (status != DIT_ATTN_OK) return status;
  if (dtype != DIT_ATTN_BF16 || d != 128) return DIT_ATTN_EUNSUPPORTED;
  if (!kv_blocks || !kv_counts || !aligned(kv_blocks, 4) || !aligned(kv_counts, 4)) return DIT_ATTN_EINVAL;
  const int n_qtiles = (N + DIT_ATTN_SPARSE_Q_BLOCK - 1) / DIT_ATTN_SPARSE_Q_BLOCK;
  const int n_t = (N + DIT_ATTN_SPARSE_KV_BLOCK - 1) / DIT_ATTN_SPARSE_KV_BLOCK;
  if (max_blocks < 1 || max_blocks > n_t) return DIT_ATTN_EINVAL;
  const long long tiles = (long long)c.bh * n_qtiles;
  if (tiles > 0x7fffffffLL / 8) return DIT_ATTN_EINVAL;
  const uint64_t count_bytes = (uint64_t)tiles * 4u, list_bytes = count_bytes * (uint64_t)max_blocks;
  // the lists are read-only inputs: they may share memory with q, k, v, not with what the call writes
  if (overlap(o, c.out_bytes, kv_blocks, list_bytes) || overlap(o, c.out_bytes, kv_counts, count_bytes))
    return DIT_ATTN_EINVAL;
  if (lse && (overlap(lse, c.lse_bytes, kv_blocks, list_bytes) || overlap(lse, c.lse_bytes, kv_counts, count_bytes)))
    return DIT_ATTN_EINVAL;
  const void* bufs[7] = {q, k, v, o, lse, kv_blocks, kv_counts};
  const uint64_t spans[7] = {c.in_bytes, c.in_bytes, c.in_bytes, c.out_bytes, c.lse_bytes, list_bytes, count_bytes};
  const int ws_status = check_workspace(workspace, workspace_bytes, bufs, spans, 7);
  if (ws_status != DIT_ATTN_OK) return ws_status;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  Plan plan;
  const int pst =
      resolve_plan(kPlanBf16D128Sparse, c.bh, N, cu_count(), max_blocks, lse != nullptr, workspace_bytes, &plan);
  if (pst != DIT_ATTN_OK) return pst;
  using C = CfgBf16D128;
  static_assert(C::kBR == DIT_ATTN_SPARSE_Q_BLOCK, "query block = the kernel's query tile");
  const KvBlocks kvb{kv_blocks, kv_counts, max_blocks};
  return launch_pipe<C, true>(q, k, v, o, lse, c.bh, N, scale, static_cast<hipStream_t>(stream), plan, workspace,
                              c.L, kvb);
}

int dit_attn_plan(int B, int H, int N, int d, int dtype, int max_blocks, int lse, int n_cu, int64_t workspace_bytes,
                  dit_attn_plan_t* plan) {
  if (!plan || B < 1 || H < 1 || N < 1 || n_cu < 0 || max_blocks < 0 || workspace_bytes < 0) return DIT_ATTN_EINVAL;
  if (dtype != DIT_ATTN_BF16 && dtype != DIT_ATTN_FP8_E4M3) return DIT_ATTN_EUNSUPPORTED;
  if (dtype == DIT_ATTN_BF16 && d != 64 && d != 128) return DIT_ATTN_EUNSUPPORTED;
  if (dtype == DIT_ATTN_FP8_E4M3 && d != 128) return DIT_ATTN_EUNSUPPORTED;
  if (max_blocks > 0 && (dtype != DIT_ATTN_BF16 || d != 128)) return DIT_ATTN_EUNSUPPORTED;
  if (max_blocks > (N + 63) / 64) return DIT_ATTN_EINVAL;
  const long long bh = (long long)B * H;
  if (bh > 0x7fffffffLL) return DIT_ATTN_EINVAL;
  if (n_cu == 0) {
    const int dev_status = check_device();
    if (dev_status != DIT_ATTN_OK) return dev_status;
    n_cu = cu_count();
  }
  Plan p;
  const int st = resolve_plan(plan_kind(d, dtype, max_blocks), bh, N, n_cu, max_blocks, lse != 0, workspace_bytes, &p);
  if (st != DIT_ATTN_OK) return st;
  plan->schedule = p.schedule;
  plan->workgroups = (int32_t)p.workgroups;
  plan->parts = p.schedule == DIT_ATTN_SCHED_SPLIT ? p.sp.parts : 1;
  plan->split_tiles = p.schedule == DIT_ATTN_SCHED_SPLIT ? p.sp.n_split : 0;
  plan->workspace_bytes = (int64_t)(p.ws_floats * sizeof(float));
  plan->workspace_wanted = (int64_t)(p.wanted_floats * sizeof(float));
  plan->best_schedule = p.best_schedule;
  plan->reserved = 0;
  return DIT_ATTN_OK;
}

int dit_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                    float scale, int dtype, const float* descale_qkv, float* lse, void* stream) {
  return dit_attn_fwd_strided(q, k, v, o, B, H, N, d, scale, dtype, nullptr, nullptr, descale_qkv, lse, nullptr, 0,
                              stream);
}

int dit_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d, float scale,
                 int dtype, void* stream) {
  return dit_attn_fwd_ex(q, k, v, o, B, H, N, d, scale, dtype, nullptr, nullptr, stream);
}

int dit_attn_fwd_mx(const void* q8, const void* k8, const void* v8, const void* q_scales, const void* k_scales,
                    const void* v_scales, void* o, int B, int H, int N, int d, float scale, float* lse,
                    void* workspace, int64_t workspace_bytes, void* stream) {
  Checked c;
  const int status = check_call(q8, k8, v8, o, B, H, N, d, scale, DIT_ATTN_FP8_E4M3, nullptr, nullptr, nullptr, lse, &c);
  if (status != DIT_ATTN_OK) return status;
  if (!q_scales || !k_scales || !v_scales) return DIT_ATTN_EINVAL;
  if (!aligned(q_scales, 16) || !aligned(k_scales, 16) || !aligned(v_scales, 16)) return DIT_ATTN_EINVAL;
  const uint64_t row_scale_bytes = (uint64_t)c.bh * (uint64_t)N * 4u;
  const uint64_t v_scale_bytes = (uint64_t)c.bh * (uint64_t)((N + 31) / 32) * 128u;
  const void* sc[3] = {q_scales, k_scales, v_scales};
  const uint64_t sb[3] = {row_scale_bytes, row_scale_bytes, v_scale_bytes};
  for (int i = 0; i < 3; ++i) {
    if (overlap(o, c.out_bytes, sc[i], sb[i])) return DIT_ATTN_EINVAL;
    if (lse && overlap(lse, c.lse_bytes, sc[i], sb[i])) return DIT_ATTN_EINVAL;
  }
  const void* bufs[8] = {q8, k8, v8, o, lse, q_scales, k_scales, v_scales};
  const uint64_t spans[8] = {c.in_bytes, c.in_bytes, c.in_bytes, c.out_bytes, c.lse_bytes, sb[0], sb[1], sb[2]};
  const int ws_status = check_workspace(workspace, workspace_bytes, bufs, spans, 8);
  if (ws_status != DIT_ATTN_OK) return ws_status;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  Plan plan;
  const int pst = resolve_plan(kPlanFp8D128, c.bh, N, cu_count(), 0, lse != nullptr, workspace_bytes, &plan);
  if (pst != DIT_ATTN_OK) return pst;
  const MxScales mxs{static_cast<const uint8_t*>(q_scales), static_cast<const uint8_t*>(k_scales),
                     static_cast<const uint8_t*>(v_scales)};
  return launch_fp8<CfgFp8D128, true>(q8, k8, v8, o, lse, nullptr, c.bh, N, scale, static_cast<hipStream_t>(stream),
                                      plan, workspace, c.L, mxs);
}

int dit_attn_quantize_mx(const void* x, int B, int H, int N, int d, int along, void* x8, void* scales,
                         void* stream) {
  if (!x || !x8 || !scales) return DIT_ATTN_EINVAL;
  if (!aligned(x, 16) || !aligned(x8, 16)) return DIT_ATTN_EINVAL;
  if (B < 1 || H < 1 || N < 1 || d < 32 || d % 32 != 0 || d > 1024) return DIT_ATTN_EINVAL;
  if (along != DIT_ATTN_MX_ALONG_D && along != DIT_ATTN_MX_ALONG_TOKENS) return DIT_ATTN_EINVAL;
  const long long bh = (long long)B * H;
  if (bh > 65535) return DIT_ATTN_EINVAL;                 // grid y of the token-blocked kernel
  const unsigned __int128 n = (unsigned __int128)bh * (unsigned)N * (unsigned)d;
  if (n >= ((unsigned __int128)1 << 62)) return DIT_ATTN_EINVAL;
  const uint64_t n_el = (uint64_t)n;
  const uint64_t scale_bytes = along == DIT_ATTN_MX_ALONG_D ? n_el / 32
                                                          : (uint64_t)bh * (uint64_t)((N + 31) / 32) * (uint64_t)d;
  if (overlap(x, n_el * 2u, x8, n_el) || overlap(x, n_el * 2u, scales, scale_bytes) ||
      overlap(x8, n_el, scales, scale_bytes))
    return DIT_ATTN_EINVAL;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  if (along == DIT_ATTN_MX_ALONG_D) {
    const int64_t n_blocks = (int64_t)(n_el / 32);
    const int64_t want = (n_blocks + kQuantThreads - 1) / kQuantThreads;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(quant_mx_rows_kernel, dim3(blocks), dim3(kQuantThreads), 0, st, xb, n_blocks,
                       static_cast<uint8_t*>(x8), static_cast<uint8_t*>(scales));
  } else {
    hipLaunchKernelGGL(quant_mx_tokens_kernel, dim3((unsigned)((N + 31) / 32), (unsigned)bh), dim3(d), 0, st, xb, N,
                       d, static_cast<uint8_t*>(x8), static_cast<uint8_t*>(scales));
  }
  return hipGetLastError() == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

int dit_attn_quantize_e4m3(const void* x, int64_t n, void* x8, float* descale, uint32_t* amax_ws,
                           void* stream) {
  if (!x || !x8 || !descale || !amax_ws) return DIT_ATTN_EINVAL;
  if (!aligned(x, 16) || !aligned(x8, 16) || !aligned(descale, 4) || !aligned(amax_ws, 4)) return DIT_ATTN_EINVAL;
  if (n < 1 || n % 8 != 0 || n >= ((int64_t)1 << 62)) return DIT_ATTN_EINVAL;
  if (overlap(x, (uint64_t)n * 2u, x8, (uint64_t)n) || overlap(descale, 4, x, (uint64_t)n * 2u) ||
      overlap(descale, 4, x8, (uint64_t)n) || overlap(amax_ws, 4, x, (uint64_t)n * 2u) ||
      overlap(amax_ws, 4, x8, (uint64_t)n) || overlap(amax_ws, 4, descale, 4))
    return DIT_ATTN_EINVAL;
  const int dev_status = check_device();
  if (dev_status != DIT_ATTN_OK) return dev_status;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t n8 = n / 8;
  const int64_t want = (n8 + kQuantThreads - 1) / kQuantThreads;
  const unsigned blocks = (unsigned)(want < 2048 ? want : 2048);
  const uint16_t* xb = static_cast<const uint16_t*>(x);
  hipLaunchKernelGGL(amax_clear_kernel, dim3(1), dim3(64), 0, st, amax_ws);
  hipLaunchKernelGGL(amax_kernel, dim3(blocks), dim3(kQuantThreads), 0, st, xb, n8, amax_ws);
  hipLaunchKernelGGL(quant_e4m3_kernel, dim3(blocks), dim3(kQuantThreads), 0, st, xb, n8,
                     static_cast<uint8_t*>(x8), descale, static_cast<const uint32_t*>(amax_ws));
  return hipGetLastError() == hipSuccess ? DIT_ATTN_OK : DIT_ATTN_ELAUNCH;
}

}  // extern "C"
