/*
 * flashmask.h -- C ABI of the FlashMask forward pass for AMD Instinct MI355X (gfx950).
 *
 * The method (web page "FlashMask技术：大模型训练中的高效注意力掩码优化", the
 * FlashMask article):
 *   - the attention mask is not stored as an N x N matrix; each query row i
 *     attends the inclusive key range [col_start[i], col_end[i]] (§1, §2.1,
 *     and the inclusive element compare of §4.1 item 3);
 *   - every (query block, key/value block) pair is classified as skip, full
 *     or partial (§2.2); skipped blocks are never loaded (§4.1 item 2), full
 *     blocks run the plain fused product, partial blocks also apply the
 *     element compare fused into the score (§4.1 item 3);
 *   - the softmax is the max-subtracted one of the FlashAttention article
 *     ("FlashAttention优化：高效训练长上下文GPT的技术突破", §2 item 2), evaluated
 *     blockwise with rescaling so the result equals dense masked attention
 *     (FlashMask article §2.2, last paragraph).
 *
 * Conventions shared by every entry point
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *     owned by the caller.  The library keeps no pointer after returning.
 *   - Return value: an fm_status code.  No call throws or aborts.
 *   - Intervals are int32; row r of batch b is element b*N + r.
 */
#ifndef FLASHMASK_H
#define FLASHMASK_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define FM_API __attribute__((visibility("default")))
#else
#define FM_API
#endif

typedef enum fm_status {
    FM_OK = 0,
    FM_ERR_INVALID_ARG = 1,   /* null pointer, bad size, misaligned pointer, bad scale   */
    FM_ERR_UNSUPPORTED = 2,   /* head dimension other than 64 or 128                      */
    FM_ERR_BAD_INTERVAL = 3,  /* fm_classify_tiles: some row violates 0 <= s <= e <= N-1  */
    FM_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed               */
    FM_ERR_TOO_LARGE = 5      /* fm_attn_fwd_noalloc: the problem exceeds its scratch     */
} fm_status;

/* Tile classes, in the order the FlashMask article §2.2 lists the cases. */
enum { FM_TILE_SKIP = 0, FM_TILE_FULL = 1, FM_TILE_PARTIAL = 2 };

/*
 * fm_classify_tiles -- the tile-class table of one sequence (FlashMask article §2.2).
 *
 *   col_start, col_end : int32[N] device, the intervals of one sequence
 *                        (for batch b pass col_start + b*N).
 *   N                  : sequence length, N >= 1.
 *   Br, Bc             : query and key block sizes, >= 1 (any value, not only
 *                        the attention kernel's own).
 *   class_out          : uint8[ceil(N/Br)][ceil(N/Bc)] device, row-major.
 *
 * For query block t (rows t*Br .. min(t*Br+Br, N)-1) and key block j
 * (klo = j*Bc, khi = min(klo+Bc, N)-1):
 *   SKIP    if khi < min col_start  or  klo > max col_end over the block's rows,
 *   FULL    if klo >= max col_start and khi <= min col_end,
 *   PARTIAL otherwise.
 * Synchronous: runs on the null stream and returns after the table is
 * written, so the caller must have finished writing the intervals.
 * Returns FM_ERR_BAD_INTERVAL when any row breaks 0 <= s <= e <= N-1 (the
 * table is still written, from the intervals clamped to [0, N-1]).
 */
FM_API int fm_classify_tiles(const int32_t* col_start, const int32_t* col_end, int64_t N,
                             int32_t Br, int32_t Bc, uint8_t* class_out);

/*
 * fm_attn_fwd -- masked attention forward: O = softmax(scale * Q K^T + M) V and
 * LSE = ln sum_j exp(scale * q_i . k_j) over the attended keys.
 *
 *   q, k, v   : bfloat16 [B][H][N][d] device, contiguous, 16-byte aligned.
 *   col_start, col_end : int32 [B][N] device, shared by all H heads; row i of
 *               batch b attends keys j in [0, N) with col_start <= j <= col_end.
 *               Any int32 values are accepted: a row whose range holds no key
 *               of [0, N) attends nothing and gets O = 0, LSE = -inf.
 *   B, H, N   : >= 1, N <= 2^22, B*H*ceil(N/128) < 2^31.
 *   d         : head dimension, 64 or 128 (else FM_ERR_UNSUPPORTED).
 *   scale     : finite and > 0 (typically 1/sqrt(d)).
 *   out       : bfloat16 [B][H][N][d] device, 16-byte aligned (round to nearest even).
 *   lse       : float32  [B][H][N] device, natural log.
 *   stream    : HIP stream the work is queued on (0 = null stream).
 *
 * Asynchronous on `stream`: returns once its kernels (interval preprocessing
 * and work ordering, then attention) are queued.  Inputs must not alias the
 * outputs.  The library keeps a small internal workspace per (device, stream),
 * grown in stream order; the call never synchronizes the device.
 * Errors: argument checks happen on the host before any HIP call
 * (FM_ERR_INVALID_ARG / FM_ERR_UNSUPPORTED); a failed allocation or launch
 * returns FM_ERR_HIP (see fm_last_hip_error).
 */
FM_API int fm_attn_fwd(const void* q, const void* k, const void* v,
                       const int32_t* col_start, const int32_t* col_end,
                       int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       void* out, float* lse, hipStream_t stream);

/*
 * fm_attn_fwd_noalloc -- fm_attn_fwd_multi (bf16, [B][n_ranges][N] intervals
 * shared by all heads) that allocates nothing: for callers that cannot call
 * hipMalloc, such as code under HIP graph capture, tight serving loops, or
 * harnesses that forbid allocation.  The caller still provides the inputs and
 * outputs.  Its workspace (per query block: 16 B of tile metadata per range,
 * a work count and a place in the order, plus the order's sort scratch on
 * very long problems) lives in a static device array of
 * FM_NOALLOC_SCRATCH_BYTES (4 MiB) that each GPU holds until the process ends;
 * one range per row fits up to about 170,000 query blocks of 128 rows
 * (B * ceil(N/128)), four ranges about 58,000.
 *   Arguments, results, asynchrony and errors as fm_attn_fwd_multi.  The
 * results are bit-identical to fm_attn_fwd_multi's except where that call
 * splits a small problem's key ranges over several workgroups
 * (FM_OPT_SPLIT_KEYS), which this one never does: there they differ only by
 * the order of fp32 additions.  FM_ERR_TOO_LARGE (nothing queued) when the
 * problem needs more scratch than that.  No kernel timing is recorded.
 *   Every call on one GPU uses that GPU's one array, which keeps the last
 * call's contents (nothing in it needs clearing: each call writes what it
 * reads).  Calls in order on one stream are safe; calls that can overlap on
 * one GPU (other streams, other host threads) race on the array and give
 * undefined results.
 */
#define FM_NOALLOC_SCRATCH_BYTES (4u << 20)
FM_API int fm_attn_fwd_noalloc(const void* q, const void* k, const void* v,
                               const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                               int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                               void* out, float* lse, hipStream_t stream);

/*
 * Rows with several key ranges.  The FlashMask article lists, as an
 * extension, rows whose attended keys are several disjoint column ranges
 * (§6.1 item 1), and as a use, attention sinks next to a sliding window
 * (§5.2 item 4), which one range per row cannot express.  Here each query
 * row holds n_ranges inclusive ranges, 1 <= n_ranges <= FM_MAX_RANGES, and
 * attends their union (ranges may overlap, touch, or be empty).
 *
 * Layout: col_start, col_end are int32 [B][n_ranges][N] device: range k of
 * row r of batch b is element (b*n_ranges + k)*N + r.  With n_ranges = 1
 * this is the [B][N] layout of the single-range calls, and the results are
 * bit-identical to them.
 *
 * Tile classes of a union (reading of §2.2 for several ranges): SKIP when
 * every range alone skips the tile, FULL when one range alone makes it FULL
 * (that range then covers every row of the tile, so the union does too),
 * PARTIAL otherwise.
 */
#define FM_MAX_RANGES 4

/*
 * fm_attn_fwd_multi -- fm_attn_fwd for rows with n_ranges key ranges.
 * Arguments, outputs, asynchrony and errors as fm_attn_fwd; additionally
 * FM_ERR_INVALID_ARG when n_ranges is outside [1, FM_MAX_RANGES].  Any int32
 * values are accepted; a range with no key of [0, N) adds nothing, and a row
 * whose ranges all hold no key gets O = 0, LSE = -inf.
 */
FM_API int fm_attn_fwd_multi(const void* q, const void* k, const void* v,
                             const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                             void* out, float* lse, hipStream_t stream);

/*
 * fm_attn_fwd_per_head -- fm_attn_fwd_multi with one interval set per head.
 * The FlashMask article varies the mask across layers (§3.4 item 1, a window
 * size per layer; §6.1 item 3, a mask kind per layer), which needs no
 * interface: each layer's call passes its own intervals.  This call carries
 * the same idea inside one layer, across heads (e.g. a different window per
 * head).  col_start, col_end are int32 [B][H][n_ranges][N]
 * device: range k of row r of head h of batch b is element
 * ((b*H + h)*n_ranges + k)*N + r.  With every head's set equal, the results
 * are bit-identical to fm_attn_fwd_multi's.  Other arguments, asynchrony and
 * errors as fm_attn_fwd_multi.
 */
FM_API int fm_attn_fwd_per_head(const void* q, const void* k, const void* v,
                                const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                                int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                void* out, float* lse, hipStream_t stream);

/*
 * fm_attn_fwd_fp8 -- the forward pass on FP8 inputs.  The FlashMask article
 * names an FP8 mode of its H100 path (§4.2) without saying which products run
 * in FP8.  Readings used here: Q, K and V are stored as OCP FP8 e4m3 (the
 * "e4m3fn" encoding: bias 7, no infinities, 0x7F/0xFF NaN) with one
 * dequantization scale per tensor (the real value of a code x is
 * scale * e4m3(x)); the score product Q K^T runs on the FP8 matrix units with
 * fp32 accumulation.  Then, by mode:
 *   FM_FP8_SCORES -- V is widened exactly to bf16 and the weights and the P V
 *     product stay bf16, as in fm_attn_fwd: the result is fm_attn_fwd's for
 *     the dequantized inputs, to the same accuracy.
 *   FM_FP8_ALL -- the P V product runs on the FP8 units as well: each weight
 *     (its row's running maximum subtracted, times 2^8) is rounded to e4m3
 *     (nearest even; relative error <= 2^-4 above 2^-14 of the row maximum)
 *     and the output divides by the sum of the rounded weights.  LSE stays
 *     the fp32 weights' (identical in both modes).
 *
 *   q8, k8, v8 : uint8 (e4m3) [B][H][N][d] device, contiguous, 16-byte aligned.
 *   q_scale, k_scale, v_scale : dequantization scales, finite and > 0.
 *   mode : FM_FP8_SCORES or FM_FP8_ALL.
 *   col_start, col_end, n_ranges : as fm_attn_fwd_multi ([B][n_ranges][N]).
 *   B, H, N, d, scale, out, lse, stream : as fm_attn_fwd (out is bfloat16).
 * Errors as fm_attn_fwd_multi; FM_ERR_INVALID_ARG for a bad scale or mode.
 */
#define FM_FP8_SCORES 0
#define FM_FP8_ALL 1
FM_API int fm_attn_fwd_fp8(const void* q8, const void* k8, const void* v8,
                           float q_scale, float k_scale, float v_scale, int32_t mode,
                           const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                           int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                           void* out, float* lse, hipStream_t stream);

/*
 * fm_classify_tiles_multi -- fm_classify_tiles for one sequence whose rows
 * hold n_ranges ranges: col_start, col_end are int32 [n_ranges][N] device
 * (for batch b pass col_start + b*n_ranges*N).  Classes as stated above.
 * Synchronous.  FM_ERR_BAD_INTERVAL when any range of any row breaks
 * 0 <= s <= e <= N-1 (the table is still written).
 */
FM_API int fm_classify_tiles_multi(const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                                   int64_t N, int32_t Br, int32_t Bc, uint8_t* class_out);

/*
 * fm_tile_schedule_multi -- fm_tile_schedule for [B][n_ranges][N] intervals.
 * work_out counts the key blocks of the union of the ranges' non-skip blocks
 * (the non-SKIP tiles of the query block's row of the class table).
 */
FM_API int fm_tile_schedule_multi(const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                                  int64_t B, int64_t N, int64_t d,
                                  int32_t* work_out, int32_t* order_out);

/*
 * fm_attn_bwd -- gradients of fm_attn_fwd: given dO = dL/dO, the gradients
 * dL/dQ, dL/dK, dL/dV.  The pages give the forward only and place the method
 * in training (FlashMask abstract), which needs them; they follow from the
 * forward's definition by the chain rule.  With P the masked softmax,
 * recomputed from the forward's LSE (P_ij = exp(scale q_i.k_j - LSE_i) for
 * attended keys, 0 otherwise), D_i = sum_c dO_ic O_ic and
 * dS_ij = P_ij (dO_i . v_j - D_i):
 *     dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
 * Tiles skipped by the forward's rule are skipped here too (they have P = 0).
 *
 *   q, k, v, out, dout : bfloat16 [B][H][N][d] device, contiguous, 16-byte
 *               aligned; out and lse are fm_attn_fwd's outputs for q, k, v
 *               and the same intervals and scale.
 *   lse       : float32 [B][H][N] device.
 *   col_start, col_end, B, H, N, d, scale : as fm_attn_fwd.
 *   dq, dk, dv : float32 [B][H][N][d] device, 16-byte aligned, fully written
 *               (rows no query attends get dk = dv = 0; rows that attend
 *               nothing get dq = 0).
 *   stream    : HIP stream the work is queued on.
 *
 * Asynchronous on `stream`; deterministic: a key block attended by many query
 * blocks is split into pieces (see FM_OPT_BWD_SPLIT_CHUNKS) whose partial dK,
 * dV sums are added into the output in a fixed piece order by a final
 * reduction, so repeated calls give identical bits (the pieces are found with
 * integer atomics, which fix only their slots, never a floating-point order).
 * Argument checks and errors as fm_attn_fwd.  Workspace: it shares
 * fm_attn_fwd's internal buffer per (device, stream), grown to about 4 B per
 * row and head plus 40 B per query block and, with one interval set for all
 * heads, the split pieces' partial sums, 32 * H * 128 * d * 8 bytes (128 MiB
 * at H = 32, d = 128); the buffer is kept until the process ends.  Inputs must
 * not alias the outputs.  On mid-sized problems the dQ part runs on a second
 * stream that the library keeps per (device, stream), forked from `stream`
 * after its first kernel and joined back into it before the call returns:
 * everything the call queues is still ordered on `stream` as a whole.
 */
FM_API int fm_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, const int32_t* col_start, const int32_t* col_end,
                       int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       float* dq, float* dk, float* dv, hipStream_t stream);

/* fm_attn_bwd for rows with n_ranges ranges ([B][n_ranges][N] intervals, as
 * fm_attn_fwd_multi). */
FM_API int fm_attn_bwd_multi(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                             float* dq, float* dk, float* dv, hipStream_t stream);

/* fm_attn_bwd for one interval set per head ([B][H][n_ranges][N] intervals, as
 * fm_attn_fwd_per_head, whose out and lse it takes). */
FM_API int fm_attn_bwd_per_head(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const int32_t* col_start, const int32_t* col_end,
                                int32_t n_ranges, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                float* dq, float* dk, float* dv, hipStream_t stream);

/* The query and key block sizes the attention kernel uses for head dimension d
 * (the shape at which tiles are skipped).  FM_ERR_UNSUPPORTED for other d. */
FM_API int fm_attn_tile_shape(int64_t d, int32_t* Br, int32_t* Bc);

/*
 * fm_tile_schedule -- inspection of the work ordering fm_attn_fwd uses
 * (FlashMask article §4.3 item 3: hand out work by each query block's
 * number of effective key blocks).
 *
 *   col_start, col_end : int32 [B][N] device.
 *   work_out  : int32 [B*ceil(N/Br)] device; non-skip key blocks of query
 *               block t of batch b at index b*ceil(N/Br) + t.
 *   order_out : int32 [B*ceil(N/Br)] device; those indices sorted by work,
 *               largest first, ties by increasing index.  Above 256 query
 *               blocks the sort key is floor(work / 32) (blocks of nearly
 *               equal work keep their index order).
 * Br, Bc are fm_attn_tile_shape(d).  Synchronous (null stream).
 */
FM_API int fm_tile_schedule(const int32_t* col_start, const int32_t* col_end,
                            int64_t B, int64_t N, int64_t d,
                            int32_t* work_out, int32_t* order_out);

/* Process-wide options (not synchronized with calls in flight on other threads). */
enum {
    FM_OPT_SCHEDULE = 1,      /* 0: longest-first order (default), 1: natural (b, t) order */
    FM_OPT_BWD_SPLIT_CHUNKS = 2, /* backward: a key block attended by more than max(this, twice the
                                   mean) query chunks of 64 rows is split into pieces of about that
                                   many chunks, whose partial dK/dV are summed in a fixed order
                                   (deterministic); default 32, 0: never split */
    FM_OPT_SINGLE_LAUNCH = 3,   /* forward, bf16 inputs: 1 (default) runs problems of at most 256
                                   workgroups (B * H * ceil(N/128)) as the attention kernel alone, each
                                   workgroup reducing its own query block's key range; 0 always
                                   queues the interval preprocessor and the work ordering first.
                                   Results are identical either way when FM_OPT_SPLIT_KEYS is 0. */
    FM_OPT_SPLIT_KEYS = 4,      /* forward, bf16 single launches (above): 1 (default) cuts each query
                                   block's long key ranges into pieces.  At d = 128, ranges of at
                                   least 32 key blocks go first to two groups of four wavefronts in
                                   each workgroup, combined through LDS; then, up to 8 pieces of at
                                   least 8 key blocks run in separate workgroups (at most 256 in all)
                                   whose partial softmax states the last one to finish combines.
                                   0: neither.  The results differ from the unsplit ones only by the
                                   order of fp32 additions.  fm_attn_fwd_noalloc uses the groups
                                   but never splits over workgroups. */
    FM_OPT_BWD_FUSED_PREP = 6,  /* backward: 1 (default) prepares both gradient kernels' tile records in
                                   one launch on small problems whose key blocks cannot split (at most
                                   FM_OPT_BWD_SPLIT_CHUNKS query chunks of 64 rows, at most 1024 chunks in
                                   all, one stream); 0: always the separate preprocessing launches.
                                   Results are identical either way. */
    FM_OPT_ROW_SLICES = 5       /* forward, bf16 single launches with FM_OPT_SPLIT_KEYS on: problems of
                                   at most this many slices of 32 query rows (B * H * ceil(N/32);
                                   default 512, 0: never) run one workgroup per slice, whose
                                   wavefronts share the slice's key blocks and combine their partial
                                   softmax states through LDS (no workspace; fm_attn_fwd_noalloc
                                   too).  Differs from the other launches only by the order of fp32
                                   additions. */
};
FM_API int fm_set_option(int option, int64_t value);

/*
 * Timing of the attention kernel alone, for measurement.  While enabled,
 * fm_attn_fwd launches the attention kernel with a HIP event pair that the
 * dispatch itself stamps at the kernel's start and end.  fm_profile_read
 * waits for the recorded events, returns the summed kernel time in
 * milliseconds and the number of launches, and clears the record.
 */
FM_API int fm_profile_enable(int enable);
FM_API int fm_profile_read(double* total_ms, int64_t* launches);

/* Text for a status code, and the HIP error code of the last failing HIP call
 * made by this thread inside the library (0 if none). */
FM_API const char* fm_status_string(int status);
FM_API int fm_last_hip_error(void);

#ifdef __cplusplus
}
#endif
#endif /* FLASHMASK_H */
