/*
 * dit_attn.h - C ABI of the MI355X (gfx950) DiT joint-attention library.
 *
 * The operation is the dense, non-causal multi-head attention of a diffusion
 * transformer over the concatenated text and image token sequence:
 *
 *     O[b,h] = softmax(Q[b,h] K[b,h]^T * scale) V[b,h]
 *
 * The pages this library follows name it only as the DiT's dense BF16
 * attention, about 60% of DiT kernel time at 2048x2048 ("Speed Up Image
 * Generation with FLUX 3 Image Klein on NVIDIA Blackwell GPUs", "Key
 * takeaways"; Italian commentary, section "NVFP4, attention e caching"), and
 * report FP8 attention variants beside it (Japanese summary, third paragraph).
 * No mask is applied: every token attends to every token (the card's
 * glossary entry for the transformer).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout:    q, k, v, o are contiguous row-major [B][H][N][d] tensors, d
 *            innermost, in device memory. o is always bfloat16.
 * Ownership: the caller allocates, owns and frees every buffer it passes,
 *            and the library never allocates, frees or retains device or
 *            host memory. Some shapes run faster with a workspace: when a
 *            bf16 d = 128 or fp8 call would leave the GPU's last round of
 *            workgroups partly filled, its query tiles are split along the
 *            keys (the last round's tiles, or, for calls of at most two
 *            rounds, every CU taking an equal share of all (query tile, key
 *            tile) pairs) and the fp32 partial rows are merged afterwards.
 *            Those rows live in a caller-owned workspace, passed to the
 *            entry points that take one and sized by dit_attn_plan (at most
 *            2^17 partial rows of 129 floats, plus 2^17 floats for an fp8
 *            call with an LSE output: 68.2 MB).
 *            Without a workspace (the short forms dit_attn_fwd and
 *            dit_attn_fwd_ex, or a NULL workspace) the call runs one
 *            workgroup per query tile; dit_attn_plan reports which schedule
 *            a call takes. The library keeps no state beyond its loaded code
 *            objects and a per-device record (gfx950 or not, CU count).
 * Streams:   work is enqueued on `stream` (a hipStream_t; NULL = the null
 *            stream) and the call returns at once. The calls contain no host
 *            synchronisation, device-to-host read, allocation or memset, so
 *            they can be captured in a HIP graph (kernel nodes only).
 * Errors:    every entry point returns DIT_ATTN_OK or a negative status, and
 *            launches nothing when it returns an error other than
 *            DIT_ATTN_ELAUNCH. Faults inside a kernel are not seen by the
 *            call; the caller sees them when it synchronises the stream.
 * Threads:   re-entrant; any number of host threads may call on their own
 *            streams. Calls that overlap in time must not share a workspace.
 */
#ifndef DIT_ATTN_H
#define DIT_ATTN_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define DIT_ATTN_API __attribute__((visibility("default")))
#else
#define DIT_ATTN_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    DIT_ATTN_BF16 = 0,      /* q, k, v bfloat16 */
    DIT_ATTN_FP8_E4M3 = 1   /* q, k, v OCP FP8 E4M3FN bytes with per-tensor descales */
} dit_attn_dtype_t;

enum {
    DIT_ATTN_OK = 0,
    DIT_ATTN_EINVAL = -1,        /* NULL / misaligned / aliasing pointer, B, H or N < 1, bad scale, size overflow */
    DIT_ATTN_EUNSUPPORTED = -2,  /* head dimension or dtype not implemented */
    DIT_ATTN_EDEVICE = -3,       /* no HIP device, or the current device is not gfx950 */
    DIT_ATTN_ELAUNCH = -4,       /* the kernel launch itself failed */
    DIT_ATTN_EWORKSPACE = -5     /* a workspace was given but is smaller than the call's plan needs */
};

/*
 * dit_attn_fwd - attention forward.
 *
 * q, k, v : device pointers, [B][H][N][d], bfloat16 (dtype = DIT_ATTN_BF16)
 *           or e4m3 bytes (dtype = DIT_ATTN_FP8_E4M3, descales taken as 1).
 *           16-byte aligned.
 * o       : device pointer, [B][H][N][d] bfloat16, 16-byte aligned, must not
 *           overlap q, k or v.
 * B, H, N : batch entries, heads, tokens (text + image [+ reference image]);
 *           each >= 1, and B*H*N*d < 2^62.
 * d       : head dimension. bf16: 64 or 128. fp8: 128.
 * scale   : logit multiplier (1/sqrt(d) for standard attention); finite, > 0.
 * dtype   : a dit_attn_dtype_t value.
 * stream  : hipStream_t or NULL.
 *
 * Runs without a workspace: one workgroup per query tile. The same call
 * through dit_attn_fwd_strided (NULL strides) with a workspace takes the
 * faster schedules that split query tiles along the keys.
 *
 * Status: DIT_ATTN_EINVAL, _EUNSUPPORTED or _EDEVICE before any launch;
 * DIT_ATTN_ELAUNCH if hipLaunchKernel reports an error.
 */
DIT_ATTN_API int dit_attn_fwd(const void* q, const void* k, const void* v, void* o,
                 int B, int H, int N, int d, float scale, int dtype, void* stream);

/*
 * dit_attn_fwd_ex - dit_attn_fwd plus the inputs the short form cannot carry.
 *
 * descale_qkv : device float[3] {dq, dk, dv}: the fp8 dequantisation factors
 *               (real value = code value * descale). NULL means 1, 1, 1.
 *               Ignored for bf16. The logits use scale*dq*dk and O carries dv.
 * lse         : device float[B*H*N] or NULL. When given, row i of head (b,h)
 *               receives the natural-log normaliser
 *               log(sum_j exp(s_ij)), s_ij the scaled logits, at [b*H*N + h*N + i].
 *               Must not overlap any other buffer. 4-byte aligned.
 */
DIT_ATTN_API int dit_attn_fwd_ex(const void* q, const void* k, const void* v, void* o,
                    int B, int H, int N, int d, float scale, int dtype,
                    const float* descale_qkv, float* lse, void* stream);

/*
 * dit_attn_fwd_strided - dit_attn_fwd_ex for rows that are not packed as
 * [B][H][N][d]: the layout a fused QKV projection or a sequence-to-head
 * all-to-all emits, e.g. [B][N][H][d] or [B][N][3][H][d].
 *
 * qkv_strides : host int64[3] {batch, head, token}: element strides shared by
 *               q, k and v (the d values of a row are contiguous). NULL means
 *               contiguous [B][H][N][d]: {H*N*d, N*d, d}. token >= d; batch and
 *               head may be 0 (rows shared across heads or batch entries).
 * o_strides   : host int64[3], the same for o; NULL means contiguous. The map
 *               (b, h, n) -> row must be one to one (checked).
 * Every stride times the element size (2 bytes bf16, 1 byte e4m3 for q, k, v;
 * 2 bytes for o) must be a multiple of 16 bytes, each stride at most 2^40, and
 * the token stride of q, k, v below 2^31 / (128 * element size). The
 * aliasing checks of dit_attn_fwd use the byte spans the strides cover. lse
 * stays packed as [B][H][N]. Other arguments and statuses as for
 * dit_attn_fwd_ex (DIT_ATTN_EINVAL for a stride that breaks these rules).
 *
 * workspace       : device memory owned by the caller, 16-byte aligned, or
 *                   NULL. Must not overlap q, k, v, o or lse. Its contents on
 *                   entry do not matter and are undefined afterwards; calls
 *                   in flight at the same time need their own.
 * workspace_bytes : its size. 0 (with any pointer): run without a workspace,
 *                   one workgroup per query tile. Otherwise it must be at
 *                   least dit_attn_plan's workspace_wanted for this shape
 *                   (else DIT_ATTN_EWORKSPACE and nothing is launched), and
 *                   the call takes the plan's fastest schedule.
 */
DIT_ATTN_API int dit_attn_fwd_strided(const void* q, const void* k, const void* v, void* o,
                         int B, int H, int N, int d, float scale, int dtype,
                         const int64_t* qkv_strides, const int64_t* o_strides,
                         const float* descale_qkv, float* lse,
                         void* workspace, int64_t workspace_bytes, void* stream);

/*
 * dit_attn_fwd_noalloc - dit_attn_fwd_strided without a workspace argument,
 * for callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation) but want the schedules a
 * workspace buys. The split rows live in the library's own static device
 * array of DIT_ATTN_NOALLOC_SCRATCH_BYTES (65 MiB; each GPU the library runs
 * on holds one copy until the process ends), found with hipGetSymbolAddress
 * on the first call on each device. The call allocates nothing.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other host threads) race and give undefined
 * results; serialise them (one stream, or events). Nothing in the array needs
 * to start at zero, and its contents after a call are undefined.
 * A plan that needs more than the array holds returns DIT_ATTN_EWORKSPACE
 * (no shape does on a device of at most 256 CUs). Arguments and other
 * statuses as for dit_attn_fwd_strided; DIT_ATTN_EDEVICE also if the array's
 * address cannot be had.
 */
#define DIT_ATTN_NOALLOC_SCRATCH_BYTES 68157440
DIT_ATTN_API int dit_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o,
                         int B, int H, int N, int d, float scale, int dtype,
                         const int64_t* qkv_strides, const int64_t* o_strides,
                         const float* descale_qkv, float* lse, void* stream);

/* Tile sizes of dit_attn_fwd_blocksparse: query rows per list, keys per listed block. */
#define DIT_ATTN_SPARSE_Q_BLOCK 256
#define DIT_ATTN_SPARSE_KV_BLOCK 64

/*
 * dit_attn_fwd_blocksparse - attention in which each block of queries visits
 * only a listed set of key/value blocks.
 *
 * The pages report a sparse attention mode for the DiT (Sol-Attention), run
 * with the first 12 or 16 denoising steps dense, whose block-selection rule
 * they do not give (Japanese summary, third paragraph). This call is the execution side only: the caller
 * chooses the blocks; a dense step calls dit_attn_fwd instead. For query row
 * i in query block t = i / 256 of head (b, h), with S the union of the listed
 * key blocks (block u = keys 64u .. min(64u + 63, N - 1)):
 *
 *     O[b,h,i] = sum_{j in S} softmax_S(s_i)_j V[b,h,j],   s_ij = scale q_i . k_j
 *
 * and the LSE output is log(sum_{j in S} exp(s_ij)). An empty list gives
 * O = 0 and LSE = -inf (attention over no keys).
 *
 * kv_counts  : device int32[B*H*ceil(N/256)]; entry (b*H + h)*ceil(N/256) + t
 *              is the number of blocks listed for query block t of head (b, h).
 *              Values above max_blocks are taken as max_blocks, negative ones
 *              as 0. 4-byte aligned.
 * kv_blocks  : device int32[B*H*ceil(N/256)][max_blocks]; the first count
 *              entries of row (b*H + h)*ceil(N/256) + t are that list's key
 *              block indices, strictly increasing, each in [0, ceil(N/64)).
 *              Entries past the count are not read. 4-byte aligned.
 * max_blocks : row length of kv_blocks, 1 <= max_blocks <= ceil(N/64).
 * Neither list may overlap o or lse; they may share memory with q, k, v.
 * Only dtype = DIT_ATTN_BF16 with d = 128 is implemented (else
 * DIT_ATTN_EUNSUPPORTED). With a workspace, the last, partly filled round of
 * workgroups is split as in dit_attn_fwd_strided, over list positions
 * instead of key tiles (the planner takes max_blocks as the list length, as
 * the host never reads the lists). The workspace must not overlap the lists
 * either. Other arguments, layouts (qkv_strides, o_strides may be NULL),
 * workspace rules and statuses as for dit_attn_fwd_strided. A list that
 * breaks the rules above cannot make the kernel access memory outside q, k,
 * v, o, lse, the lists and the workspace (a block index out of range reads
 * zero rows), but its result is unspecified.
 */
DIT_ATTN_API int dit_attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o,
                             int B, int H, int N, int d, float scale, int dtype,
                             const int32_t* kv_blocks, const int32_t* kv_counts, int max_blocks,
                             const int64_t* qkv_strides, const int64_t* o_strides,
                             float* lse, void* workspace, int64_t workspace_bytes, void* stream);

/* Block axis of dit_attn_quantize_mx. */
#define DIT_ATTN_MX_ALONG_D 0       /* 32 consecutive d values of a row (Q, K) */
#define DIT_ATTN_MX_ALONG_TOKENS 1  /* 32 consecutive tokens of a column (V) */

/*
 * dit_attn_fwd_mx - attention on block-scaled e4m3 inputs (MX style), with
 * the scaled e4m3 matrix product of gfx950.
 *
 * The pages report fp8 attention variants (Japanese summary, third
 * paragraph) without their scaling. Here every 32 consecutive values of an
 * input share one power-of-two scale 2^e, held as the E8M0 byte e + 127:
 * along d for q and k, along the tokens for v, so that each block lies in one
 * 32-wide slice of the contraction it enters. Real values are code * 2^e;
 * dit_attn_quantize_mx produces all three. The rest is the fp8 pipeline of
 * dit_attn_fwd with DIT_ATTN_FP8_E4M3 (logits from the dequantised values
 * times scale, P rounded to e4m3, O divided by the sum of the rounded P).
 *
 * q8, k8, v8 : device e4m3 codes, contiguous [B][H][N][d], 16-byte aligned.
 * q_scales,
 * k_scales   : device bytes [B][H][N][d/32]: byte j of row n scales d = 32 j
 *              .. 32 j + 31. 16-byte aligned.
 * v_scales   : device bytes [B][H][ceil(N/32)][32][d/32]: entry (t, i, j)
 *              scales column 32 j + i over tokens 32 t .. 32 t + 31.
 *              16-byte aligned.
 * o, lse, B, H, N, scale, stream: as for dit_attn_fwd_ex. d must be 128
 * (else DIT_ATTN_EUNSUPPORTED). o and lse must not overlap any input or
 * scale array. workspace, workspace_bytes: as for dit_attn_fwd_strided (it
 * must not overlap the scale arrays either); the plan is that of a
 * DIT_ATTN_FP8_E4M3 call. Statuses as for dit_attn_fwd_strided.
 */
DIT_ATTN_API int dit_attn_fwd_mx(const void* q8, const void* k8, const void* v8,
                    const void* q_scales, const void* k_scales, const void* v_scales, void* o,
                    int B, int H, int N, int d, float scale, float* lse,
                    void* workspace, int64_t workspace_bytes, void* stream);

/*
 * dit_attn_quantize_mx - block-scaled e4m3 quantisation of a bf16 tensor.
 *
 * x      : device bfloat16, contiguous [B][H][N][d], 16-byte aligned;
 *          32 <= d <= 1024, d a multiple of 32; B*H <= 65535.
 * along  : DIT_ATTN_MX_ALONG_D (scales [B][H][N][d/32]) or
 *          DIT_ATTN_MX_ALONG_TOKENS (scales [B][H][ceil(N/32)][32][d/32], the
 *          layouts dit_attn_fwd_mx reads).
 * For each block of 32 values: amax = max |x|; e = the smallest integer with
 * amax / 2^e <= 448, at least -127 (an all-zero block takes -127); the scale
 * byte is e + 127; each code is the e4m3 value nearest to x / 2^e (ties to
 * even). Nothing saturates. (The OCP Microscaling MXFP8 conversion takes
 * e = floor(log2 amax) - 8 and clips the block maximum instead; this rule is
 * one exponent step larger for blocks whose maximum's significand exceeds
 * 1.75.)
 * x8     : device uint8, same shape as x, 16-byte aligned; must not overlap x.
 * scales : device uint8 array of the size above; must not overlap x or x8.
 * Statuses: DIT_ATTN_EINVAL for bad pointers or sizes, _EDEVICE, _ELAUNCH.
 */
DIT_ATTN_API int dit_attn_quantize_mx(const void* x, int B, int H, int N, int d, int along, void* x8,
                         void* scales, void* stream);

/*
 * dit_attn_quantize_e4m3 - per-tensor absmax quantisation of a bf16 tensor.
 *
 * Produces the fp8 inputs of the DIT_ATTN_FP8_E4M3 path on the device:
 *   amax = max |x|;  s = fp32(448 / amax)  (s = 1 if amax is 0 or s is not finite)
 *   x8[i] = e4m3 round-to-nearest-even of clamp(fp32(x[i] * s), -448, 448)
 *   *descale = fp32(1 / s)
 *
 * x        : device bfloat16[n], 16-byte aligned.
 * n        : element count, 1 <= n < 2^62, a multiple of 8.
 * x8       : device uint8[n], 16-byte aligned, not overlapping x.
 * descale  : device float[1]: receives 1/s.
 * amax_ws  : device uint32[1] workspace owned by the caller; the call clears
 *            it itself (with a kernel), then reduces into it. Two calls in
 *            flight at once must not share it.
 * stream   : hipStream_t or NULL.
 */
DIT_ATTN_API int dit_attn_quantize_e4m3(const void* x, int64_t n, void* x8, float* descale,
                           uint32_t* amax_ws, void* stream);

/* Schedules of an attention call (dit_attn_plan_t.schedule). */
#define DIT_ATTN_SCHED_TILE 0     /* one workgroup per query tile */
#define DIT_ATTN_SCHED_SPLIT 1    /* the last round's query tiles split along the keys, then merged */
#define DIT_ATTN_SCHED_STREAMK 2  /* every CU takes an equal share of (query tile, key tile) pairs */

typedef struct {
    int32_t schedule;         /* DIT_ATTN_SCHED_* the call takes with the workspace given */
    int32_t workgroups;       /* workgroups of the attention kernel */
    int32_t parts;            /* key ranges per split query tile (SPLIT), else 1 */
    int32_t split_tiles;      /* query tiles split along the keys (SPLIT), else 0 */
    int64_t workspace_bytes;  /* workspace bytes that schedule uses, 0 if none */
    int64_t workspace_wanted; /* workspace bytes of the fastest schedule, 0 if it needs none */
    int32_t best_schedule;    /* DIT_ATTN_SCHED_* of the fastest schedule */
    int32_t reserved;
} dit_attn_plan_t;

/*
 * dit_attn_plan - the schedule an attention call of this shape would use.
 *
 * The launch decides its schedule from the shape and the workspace size
 * alone (never from the data); this returns that decision without launching
 * anything, so a caller can size the workspace or check the plan. B, H, N,
 * d, dtype as for dit_attn_fwd; max_blocks > 0 describes a
 * dit_attn_fwd_blocksparse call with that list length (bf16, d = 128 only),
 * 0 a dense call (the block-scaled fp8 call plans as DIT_ATTN_FP8_E4M3);
 * lse != 0 if an LSE output is requested.
 * n_cu            : compute units to plan for; 0 means the current device's
 *                   (then a gfx950 device must be current, else
 *                   DIT_ATTN_EDEVICE).
 * workspace_bytes : the workspace the call will be given (0: none, as for
 *                   dit_attn_fwd and dit_attn_fwd_ex). A call without one
 *                   reports schedule DIT_ATTN_SCHED_TILE and, in
 *                   best_schedule / workspace_wanted, what a workspace would
 *                   buy.
 * plan            : host pointer, filled on DIT_ATTN_OK.
 * Status: DIT_ATTN_EINVAL (NULL plan, sizes < 1, n_cu < 0, workspace_bytes
 * < 0, max_blocks out of range), DIT_ATTN_EUNSUPPORTED (d, dtype),
 * DIT_ATTN_EDEVICE, DIT_ATTN_EWORKSPACE (0 < workspace_bytes <
 * workspace_wanted, as the call itself would return).
 */
DIT_ATTN_API int dit_attn_plan(int B, int H, int N, int d, int dtype, int max_blocks, int lse, int n_cu,
                  int64_t workspace_bytes, dit_attn_plan_t* plan);

/* Human-readable name of a status code (static string, never NULL). */
DIT_ATTN_API const char* dit_attn_strerror(int status);

/*
 * dit_attn_mfma_ceiling - the matrix-core rate this card sustains on
 * attention-like operands, for setting an attention call against it.
 *
 * The dense MFMA peaks assume the 2.4 GHz peak engine clock. A stream of
 * products whose operands change from product to product drives the part to
 * its power limit below that clock, by an amount that depends on the data;
 * the attention kernels run into the same limit. This launches `workgroups`
 * workgroups of four waves (one wave per SIMD; 0 = one per CU), each wave
 * issuing rounds x 16 independent products back to back on operands drawn
 * once from a fixed counter hash: v_mfma_f32_32x32x16_bf16 on bf16 values of
 * about unit variance (dtype DIT_ATTN_BF16, 32768 flop per product) or
 * v_mfma_scale_f32_32x32x64_f8f6f4 on normal e4m3 codes at scale 2^0 (dtype
 * DIT_ATTN_FP8_E4M3, 131072 flop per product). It measures no attention
 * and follows no passage of the pages: it is the reference point for the
 * measurement of the attention calls.
 * record         : device buffer of at least workgroups x 64 bytes (int64,
 *                  8-byte aligned), caller-owned. Wave w = 4 workgroup +
 *                  wave index writes record[2 w] = shader-clock cycles
 *                  (s_memtime) and record[2 w + 1] = wall-clock ticks
 *                  (s_memrealtime) over its product loop; cycles / ticks x
 *                  wall_clock_khz is the shader clock in kHz.
 * wall_clock_khz : host pointer or NULL; receives the wall-clock tick rate.
 * The caller times the launch (events on `stream`) for the rate in flop/s.
 * Status: DIT_ATTN_EINVAL (rounds < 1, workgroups < 0 or > 2^20, NULL or
 * misaligned record), DIT_ATTN_EUNSUPPORTED (dtype), DIT_ATTN_EDEVICE,
 * DIT_ATTN_EWORKSPACE (record smaller than workgroups x 64 bytes),
 * DIT_ATTN_ELAUNCH.
 */
DIT_ATTN_API int dit_attn_mfma_ceiling(int dtype, int rounds, int workgroups, void* record, int64_t record_bytes,
                          int* wall_clock_khz, void* stream);

/* Library ABI version: (major << 16) | minor. 2.0: caller-owned workspaces
   (dit_attn_fwd_strided, _blocksparse and _mx take one; dit_attn_plan takes
   its size and reports the schedule it buys); nothing allocates. 2.1:
   dit_attn_mfma_ceiling. */
DIT_ATTN_API int dit_attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* DIT_ATTN_H */
