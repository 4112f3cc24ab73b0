// Internal declarations shared by the HIP sources of libflashmask (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>
#include <type_traits>

namespace fm {

// Tile shape of the attention kernel: query rows per workgroup, keys per step.
#ifndef FM_QUERY_TILE
#define FM_QUERY_TILE 128
#endif
#ifndef FM_KEY_TILE
#define FM_KEY_TILE 64
#endif
constexpr int kBr = FM_QUERY_TILE;
constexpr int kBc = FM_KEY_TILE;

// Per query block and per key range of its rows (one sequence of one batch),
// computed from the rows' intervals for that range:
//   x = first non-skip key block, y = last non-skip key block (y < x: none),
//   z = first FULL key block,     w = last FULL key block     (w < z: none).
// Under the min/max rule the non-skip blocks and the full blocks of one range
// each form one contiguous range of key blocks.  Rows may hold up to
// kMaxRanges ranges (their union is attended); the records of query block
// item are meta[item * n_iv + k], k < n_iv.
using TileMeta = int4;
constexpr int kMaxRanges = 4;

// Work items.  Each batch element holds n_sets interval sets (1: all heads
// share one set; H: one set per head), col_start/col_end [B][n_sets][n_iv][N].
// Query block t of set g of batch element b is item (g*B + b)*n_q + t, so the
// items of one set form a contiguous segment of B*n_q.
//
// Interval preprocessor: one wavefront per item.
//   meta[item * n_iv + k]; work[item] = non-skip key blocks of the union (may
//   be null); bad (may be null): set to 1 when a row breaks 0 <= s <= e <= N-1.
hipError_t launch_preprocess(const int32_t* col_start, const int32_t* col_end, int n_iv, int64_t B,
                             int64_t N, int Br, int Bc, TileMeta* meta, int32_t* work, int32_t* bad,
                             hipStream_t stream, int n_sets = 1);

// Expands meta of n_q query blocks (n_iv ranges each) into the uint8 class
// table [n_q][n_kv]: SKIP unless some range keeps the block, FULL when some
// range covers it for every row, else PARTIAL.
hipError_t launch_class_table(const TileMeta* meta, int n_iv, int64_t n_q, int64_t n_kv, uint8_t* table,
                              hipStream_t stream);

// Longest-first order (ties by index) within each segment of L consecutive
// items (L = 0: one segment of all M items; M must be a multiple of L):
// order[seg*L + rank] = item.  With shift > 0 the items are ranked by
// work >> shift, so that items of nearly equal work keep their index order
// (for the attention kernel: the query blocks of one document stay together,
// and the workgroups resident on an XCD share fewer documents' K/V).  Work
// values lie in [-1, max_work] (-1 ranks last).  A segment of at most
// kSortSmall items is sorted by one workgroup in LDS; a longer one takes a
// counting sort whose int32 scratch (schedule_scratch_ints; 0 when no segment
// is longer than kSortSmall) the caller provides.
constexpr int kSortSmall = 16384;       // items per segment sorted by one workgroup
constexpr int kSortSmallBits = 14;      // index bits of its sort keys (2^14 = kSortSmall)
constexpr int kSortChunk = 8192;        // items per chunk of the counting sort
constexpr int kSortChunkBits = 13;
int64_t schedule_scratch_ints(int64_t M, int64_t L, int shift, int max_work);
hipError_t launch_schedule(const int32_t* work, int64_t M, int32_t* order, hipStream_t stream, int64_t L,
                           int shift, int max_work, int32_t* scratch);

// Work bucket of the attention kernel's order above kScheduleExactMax query
// blocks: 32 key blocks.  Up to kScheduleExactMax query blocks (too few to fill
// the XCDs several times over) the order ranks by exact work.
constexpr int kScheduleBucketShift = 5;
constexpr int kScheduleExactMax = 256;
inline int schedule_shift(int64_t M) { return M <= kScheduleExactMax ? 0 : kScheduleBucketShift; }

// Preprocessor and scheduler in one launch of one workgroup, for at most
// kPrepSmallMax query blocks (B * n_q): same meta, work and order outputs.
// Above that the intervals are reduced by many workgroups (one wavefront per
// query block) and the order is a separate launch: one CU reading every row's
// intervals takes longer than the second launch costs.
constexpr int kPrepSmallMax = 64;
hipError_t launch_prep_small(const int32_t* col_start, const int32_t* col_end, int n_iv, int64_t B,
                             int64_t N, int Br, int Bc, TileMeta* meta, int32_t* work, int32_t* order,
                             hipStream_t stream, int n_sets = 1);

// Attention kernel.  order == nullptr runs query blocks in natural (b, t) order.
// start/stop (may be null) are stamped at the kernel's own start and end.
// fp8_scales == nullptr: q, k, v are bf16.  Otherwise they are e4m3,
// fp8_scales points to their three dequantization scales (host memory), and
// fp8_weights also rounds the weights to e4m3 for an FP8 PV product.
// Without records (meta == nullptr, bf16): split > 1 cuts each query block's
// key range into split pieces over as many workgroups (their states in part,
// their arrivals counted in counters), groups = 2 each workgroup's share over
// two groups of four wavefronts inside it.
hipError_t launch_attention(const void* q, const void* k, const void* v, const int32_t* col_start,
                            const int32_t* col_end, int n_iv, const TileMeta* meta, const int32_t* order,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale, void* out,
                            float* lse, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                            const float* fp8_scales = nullptr, int n_sets = 1, bool fp8_weights = false,
                            int split = 1, float* part = nullptr, unsigned* counters = nullptr, int groups = 1);

// Small problems: one workgroup per 32 query rows of one (b, h), whose
// wavefronts share the rows' key blocks and combine their states in LDS
// (bf16; no records, no workspace).
hipError_t launch_attention_rows(const void* q, const void* k, const void* v, const int32_t* col_start,
                                 const int32_t* col_end, int n_iv, int64_t B, int64_t H, int64_t N, int64_t d,
                                 float scale, void* out, float* lse, hipStream_t stream, hipEvent_t start,
                                 hipEvent_t stop, int n_sets = 1);

// The forward pass's launch sequence (fm_forward.hip).
struct FwdArgs {
    const void *q, *k, *v;
    const int32_t *col_start, *col_end;
    int32_t n_ranges;
    int64_t B, H, N, d;
    float scale;
    void* out;
    float* lse;
    hipStream_t stream;
    const float* fp8_scales;   // nullptr: bf16 inputs; else the three e4m3 dequantization scales
    bool per_head;             // one interval set per head
    bool fp8_weights;          // e4m3 weights and an FP8 PV product
};

// Workspace layout: meta[M][n_ranges] | work[M] | order[M] | scheduler scratch,
// M = n_sets * B * n_q, each part 256-byte aligned.
struct FwdPlan {
    int64_t n_q, n_kv, n_sets, M;
    size_t meta_bytes, int_bytes, sched_bytes;
    bool single;               // the attention kernel alone (no records, no order)
    bool rows;                 // single, as the 32-row slice kernel
    int split;                 // pieces per work item's key range (single launches only; 1: none)
    int groups;                // wavefront groups sharing each workgroup's range (single launches; 1: none)
    size_t part_bytes;         // the pieces' partial states
    size_t total() const { return single ? (rows ? 0 : part_bytes) : meta_bytes + 2 * int_bytes + sched_bytes; }
};

// Splitting the key ranges of small single launches: a power of two of pieces
// per work item, at most kMaxSplit, at most kSingleLaunchGrid workgroups in
// all, and at least kSplitMinBlocks key blocks per piece of the longest
// possible range (cross-workgroup combining costs a few block times, so short
// ranges are not split); the partial states take kFwdThreads lanes of d/2 + 4
// floats per piece.
constexpr int kMaxSplit = 8;
constexpr int kSplitMinBlocks = 8;
// Before that (d = 128), a workgroup's range is shared by two groups of four
// wavefronts combining through LDS, which costs far less, with at least
// kGroupMinBlocks key blocks per group of the longest range.
constexpr int kGroupMinBlocks = 16;
constexpr int kFwdThreads = 256;
// Arrival counters of split items: one per work item of a single launch,
// zero between calls.
constexpr int kSplitCounters = 256;
inline size_t split_part_bytes(int64_t items, int64_t split, int64_t d) {
    return (size_t)(items * split * kFwdThreads) * (size_t)(d / 2 + 4) * sizeof(float);
}
// split_keys: cut small single launches' key ranges (groups, and with
// across_workgroups also workgroups, which need the workspace and counters).
// row_slices_max: single launches of at most this many 32-row slices
// (B * H * ceil(N/32)) run the slice kernel (0: never).
FwdPlan fwd_plan(const FwdArgs& a, bool single_launch, bool split_keys, bool across_workgroups,
                 int64_t row_slices_max);

// Queues the preprocessor, the scheduler (unless natural order) and the
// attention kernel on a.stream, with ws (p.total() bytes of device memory) as
// their workspace.  Every byte of ws that a kernel reads was written earlier
// in the same sequence, so ws needs no clearing.  With p.single, a bf16 grid
// of at most kSingleLaunchGrid workgroups (all resident at once, so their
// order cannot matter) runs the attention kernel alone: each workgroup
// reduces its own query block's key range from the intervals it stages; with
// p.split > 1 each range is cut into p.split pieces whose partial states go
// to ws, and `counters` (kSplitCounters zeros, left zero again) counts their
// arrivals.
constexpr int64_t kSingleLaunchGrid = 256;
hipError_t fwd_launch(const FwdArgs& a, const FwdPlan& p, void* ws, unsigned* counters, bool natural,
                      hipEvent_t ev_start, hipEvent_t ev_stop);
// Fills n counters with zeros on stream (a kernel: no memset node in a graph).
hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream);

// Backward pass (gradients of Q, K, V).  Shapes: the key-block kernel runs
// kBwdKeys keys per workgroup against query chunks of kBwdRows rows; the
// query-block kernel uses the forward's (kBr, kBc).
constexpr int kBwdRows = 64;
constexpr int kBwdKeys = 128;

// D[bh][i] = sum_c dO[bh][i][c] * O[bh][i][c] (fp32) for B*H*N rows.
hipError_t launch_bwd_rowdot(const void* out, const void* dout, int64_t rows, int64_t d, float* dd,
                             hipStream_t stream);

// For each key-block item (set*B + b)*n_kb + J (blocks of kBwdKeys keys): the
// first and last query chunk (kBwdRows rows, records meta_c from
// launch_preprocess with that shape and the same n_sets) whose non-skip ranges
// hold J, and their count: kvr[item] = {t_lo, t_hi, count, 0}, work[item] = count.
hipError_t launch_kv_ranges(const TileMeta* meta_c, int n_iv, int64_t B, int64_t N, int4* kvr, int32_t* work,
                            hipStream_t stream, int n_sets = 1);

// Key-block pieces of the dK/dV kernel.  A key block attended by many more
// query chunks than the average is split into P pieces of consecutive chunks
// (at most kBwdExtraPieces extra pieces per call, only with one interval set):
// piece 0 writes dK/dV, pieces 1..P-1 write partial sums that the reduce kernel
// adds to them in piece order (deterministic).  With items = B * n_kb key
// blocks per set, the piece table has Lp = items + extra entries per set:
//   pieces[e] = {key-block item (-1: unused), first chunk, last chunk, p << 16 | P}
//   pslot[e]  = partial slot of piece p >= 1 (-1 otherwise)
//   pwork[e]  = estimated live chunks (-1 for unused entries: ranked last)
//   splits[0].x = number of split blocks; splits[1 + s] = {item, P, first slot, 0}
// min_chunks: pieces hold at least this many chunks (more when the average
// block is longer: twice the average).
constexpr int kBwdExtraPieces = 32;
inline int64_t bwd_piece_entries(int64_t items, int n_sets) { return n_sets == 1 ? items + kBwdExtraPieces : items; }
hipError_t launch_bwd_split(const int4* kvr, int64_t items, int n_sets, int min_chunks, int4* pieces,
                            int32_t* pslot, int32_t* pwork, int4* splits, hipStream_t stream);

// The two gradient kernels (see fm_attn_bwd.hip).  The dK/dV kernel runs the
// piece table's entries in `order` (longest first within each set);
// part: kBwdExtraPieces * H * kBwdKeys * d * 2 floats.
hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* dd, const int32_t* col_start, const int32_t* col_end, int n_iv,
                           const TileMeta* meta_c, const int4* pieces, const int32_t* pslot, const int32_t* order,
                           int64_t B, int64_t H, int64_t N, int64_t d, float scale, float* dk, float* dv,
                           float* part, hipStream_t stream, int n_sets = 1);
// Small problems whose key blocks cannot split: the dQ kernel's query-block
// records (natural order), the query chunks' records and the dK/dV kernel's
// one-piece table with the identity order, from one workgroup (at most
// kBwdFusedMaxChunks query chunks in all).
constexpr int kBwdFusedMaxChunks = 1024;
hipError_t launch_bwd_prep_fused(const int32_t* col_start, const int32_t* col_end, int n_iv, int64_t B, int64_t N,
                                 int n_sets, TileMeta* meta_q, TileMeta* meta_c, int4* pieces, int32_t* pslot,
                                 int32_t* order_k, hipStream_t stream);
// Adds the partial sums of split key blocks to dK, dV.
hipError_t launch_bwd_reduce(const int4* splits, const float* part, int64_t H, int64_t N, int64_t d, int64_t n_kb,
                             float* dk, float* dv, hipStream_t stream);
hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         const float* dd, const int32_t* col_start, const int32_t* col_end, int n_iv,
                         const TileMeta* meta, const int32_t* order, int64_t B, int64_t H, int64_t N, int64_t d,
                         float scale, float* dq, hipStream_t stream, int n_sets = 1);

// ---------------------------------------------------------------- wavefront helpers

// Butterfly exchange inside each 32-lane half with ds_swizzle (bit-mask mode:
// lane' = lane ^ XOR), then the two halves are combined with readlane.
template <int XOR>
__device__ __forceinline__ int swizzle_xor(int v) {
    static_assert(XOR > 0 && XOR < 32, "swizzle xor mask is 5 bits");
    return __builtin_amdgcn_ds_swizzle(v, (XOR << 10) | 0x1F);
}

__device__ __forceinline__ int wave_min(int v) {
    v = min(v, swizzle_xor<1>(v));
    v = min(v, swizzle_xor<2>(v));
    v = min(v, swizzle_xor<4>(v));
    v = min(v, swizzle_xor<8>(v));
    v = min(v, swizzle_xor<16>(v));
    return min(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}

__device__ __forceinline__ int wave_sum(int v) {
    v += swizzle_xor<1>(v);
    v += swizzle_xor<2>(v);
    v += swizzle_xor<4>(v);
    v += swizzle_xor<8>(v);
    v += swizzle_xor<16>(v);
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 32);
}

__device__ __forceinline__ int wave_max(int v) {
    v = max(v, swizzle_xor<1>(v));
    v = max(v, swizzle_xor<2>(v));
    v = max(v, swizzle_xor<4>(v));
    v = max(v, swizzle_xor<8>(v));
    v = max(v, swizzle_xor<16>(v));
    return max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}


// Bounds of a set of rows' intervals: the non-skip range needs the smallest
// start and largest end of the rows that attend some key, the full range the
// largest start and smallest end of all rows (a row with no key in [0, N)
// rules out FULL blocks).  `bad` flags a row that breaks 0 <= s <= e <= N-1.
struct RowBounds {
    int min_s = INT_MAX, max_e = INT_MIN;   // non-skip range
    int max_s = INT_MIN, min_e = INT_MAX;   // full range
    int bad = 0;

    __device__ __forceinline__ void add(int s, int e, int N) {
        bad |= (s < 0) | (e > N - 1) | (s > e);
        const int sc = max(s, 0);
        const int ec = min(e, N - 1);
        if (sc <= ec) {
            min_s = min(min_s, sc);
            max_e = max(max_e, ec);
            max_s = max(max_s, sc);
            min_e = min(min_e, ec);
        } else {
            max_s = INT_MAX;
            min_e = INT_MIN;
        }
    }

    // The tile record of a query block from the bounds of all of its rows.
    __device__ __forceinline__ TileMeta meta(int N, int Bc, int n_kv) const {
        TileMeta m;
        if (max_e < min_s) {          // no row attends any key
            m.x = 0;
            m.y = -1;
        } else {
            m.x = min_s / Bc;
            m.y = max_e / Bc;
        }
        if (max_s <= min_e) {
            m.z = (max_s + Bc - 1) / Bc;
            m.w = (min_e == N - 1) ? n_kv - 1 : (min_e + 1) / Bc - 1;
        } else {
            m.z = 0;
            m.w = -1;
        }
        return m;
    }
};

// Tile metadata of query block t of one sequence, reduced by one wavefront
// (all 64 lanes must call it).  Rows past N are neutral.  `invalid` (per
// lane) is set when one of the lane's rows breaks 0 <= s <= e <= N-1.
__device__ __forceinline__ TileMeta query_block_meta(const int32_t* __restrict__ s_row,
                                                     const int32_t* __restrict__ e_row, int t, int N,
                                                     int Br, int Bc, int n_kv, int lane, int* invalid) {
    RowBounds rb;
    const int r_end = min(t * Br + Br, N);
    for (int r = t * Br + lane; r < r_end; r += 64) rb.add(s_row[r], e_row[r], N);
    *invalid = rb.bad;
    rb.min_s = wave_min(rb.min_s);
    rb.max_e = wave_max(rb.max_e);
    rb.max_s = wave_max(rb.max_s);
    rb.min_e = wave_min(rb.min_e);
    return rb.meta(N, Bc, n_kv);
}

// The key blocks a query block visits are the union of the non-skip ranges
// [x, y] of its NIV records.  union_next gives the smallest block of that
// union after block j (j = -1: the first block), or INT_MAX when none is left.
// Every index is a compile-time constant after unrolling, so the records stay
// in registers.
template <int NIV>
__device__ __forceinline__ int union_next(const TileMeta (&m)[NIV], int j) {
    int best = INT_MAX;
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
        const int c = max(j + 1, m[k].x);
        if (c <= m[k].y) best = min(best, c);
    }
    return best;
}

// Number of key blocks in that union: runs of overlapping or adjacent ranges
// are walked from left to right.
template <int NIV>
__device__ __forceinline__ int union_blocks(const TileMeta (&m)[NIV]) {
    int total = 0;
    int j = union_next<NIV>(m, -1);
    while (j != INT_MAX) {
        int e = j;                     // end of the run that starts at j
        bool grew = true;
        while (grew) {
            grew = false;
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
                if (m[k].x <= m[k].y && m[k].x <= e + 1 && m[k].y > e) {
                    e = m[k].y;
                    grew = true;
                }
            }
        }
        total += e - j + 1;
        j = union_next<NIV>(m, e);
    }
    return total;
}

// Calls f(std::integral_constant<int, NIV>) for n_iv in 1..kMaxRanges.
template <typename F>
__host__ hipError_t dispatch_ranges(int n_iv, F&& f) {
    switch (n_iv) {
        case 1: return f(std::integral_constant<int, 1>{});
        case 2: return f(std::integral_constant<int, 2>{});
        case 3: return f(std::integral_constant<int, 3>{});
        case 4: return f(std::integral_constant<int, 4>{});
        default: return hipErrorInvalidValue;
    }
}

}  // namespace fm
