// Work ordering for the attention kernel (gfx950).
//
// FlashMask article ("FlashMask技术：大模型训练中的高效注意力掩码优化") §4.3
// item 3: hand out the work by each query block's number of effective
// (non-skipped) key blocks, and §4.2 (several query blocks per processor).
// Under document or sliding masks the per-block work is very uneven (a
// query block at the end of a long document needs many key blocks, one at
// the start of a short document needs one), so the blocks are issued
// longest first: the long ones start early and the short ones fill the
// tail.  The order is a stable sort by decreasing work; each item's rank is
// counted directly (items ranked ahead of x: larger work, or equal work and
// smaller index), which is deterministic and needs no atomics.  On large
// problems the attention order sorts by work in buckets of 32 key blocks, so
// that the query blocks of one document that need about the same work run
// together and share their K/V in the XCD's L2.  The order
// never changes a result: every query block's output depends only on its
// own fixed sequence of key blocks.

#include <climits>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kThreads = 256;

// Items are ranked within their segment of L; a workgroup walks the union of
// its threads' segments (uniform bounds for the barriers) and each thread
// counts only its own segment.
__global__ __launch_bounds__(kThreads) void schedule_kernel(const int32_t* __restrict__ work, int M, int L,
                                                            int shift, int32_t* __restrict__ order) {
    __shared__ int s_work[kThreads];
    const int x = blockIdx.x * kThreads + threadIdx.x;
    const int wx = x < M ? (work[x] >> shift) : INT_MIN;
    const int x_first = blockIdx.x * kThreads;
    const int x_last = min(M, x_first + kThreads) - 1;
    const int y_begin = (x_first / L) * L;
    const int y_end = min(M, (x_last / L + 1) * L);
    const int my_lo = (x / L) * L;
    const int my_hi = my_lo + L;
    int rank = 0;
    for (int base = y_begin; base < y_end; base += kThreads) {
        const int y = base + threadIdx.x;
        s_work[threadIdx.x] = y < y_end ? (work[y] >> shift) : INT_MIN;
        __syncthreads();
        const int lim = min(kThreads, y_end - base);
        for (int i = 0; i < lim; ++i) {
            const int wy = s_work[i];
            const int yy = base + i;
            rank += (yy >= my_lo) & (yy < my_hi) & ((wy > wx) | ((wy == wx) & (yy < x)));
        }
        __syncthreads();
    }
    if (x < M) order[my_lo + rank] = x;
}

constexpr int kPrepThreads = 1024;

// Small problems: one workgroup computes every query block's metadata and
// then ranks the blocks from LDS, saving a launch.  Each query block gets a
// group of G lanes (G = 1024 / M rounded down to a power of two, at most 64);
// a lane reads every G-th row (or 16-byte chunk of four rows) of the block
// with its loads unrolled, so that they are all in flight at once, and the
// group reduces by lane exchange.  The same groups then rank the items: each
// lane counts over one slice of the work array.
template <int NIV>
__global__ __launch_bounds__(kPrepThreads) void prep_small_kernel(
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_end, int N, int n_q, int n_kv,
    int Br, int Bc, int M, int G, bool vec4, int n_sets, int L, TileMeta* __restrict__ meta,
    int32_t* __restrict__ work, int32_t* __restrict__ order) {
    // work of each item, padded with INT_MIN up to G * SL <= M + 4 G <= 2 * kPrepSmallMax entries
    __shared__ __attribute__((aligned(16))) int s_work[2 * kPrepSmallMax];
    const int item = threadIdx.x / G;          // G divides 64: a group never straddles wavefronts
    const int g = threadIdx.x % G;
    if (item < M) {
        const int set = item / L;               // interval set (item = (set * B + b) * n_q + t)
        const int rem = item - set * L;
        const int b = rem / n_q;
        const int t = rem - b * n_q;
        const int r0 = t * Br;
        const int r_end = min(r0 + Br, N);
        TileMeta m[NIV];
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            const int32_t* s_row = col_start + (((int64_t)b * n_sets + set) * NIV + k) * N;
            const int32_t* e_row = col_end + (((int64_t)b * n_sets + set) * NIV + k) * N;
            RowBounds rb;
            if (vec4) {
                // rows in 16-byte chunks of four (N and both bases are multiples of 4 rows)
                const int4* s4 = reinterpret_cast<const int4*>(s_row);
                const int4* e4 = reinterpret_cast<const int4*>(e_row);
#pragma unroll 8
                for (int c = (r0 >> 2) + g; c < (r_end >> 2); c += G) {
                    const int4 sv = s4[c];
                    const int4 ev = e4[c];
                    rb.add(sv.x, ev.x, N);
                    rb.add(sv.y, ev.y, N);
                    rb.add(sv.z, ev.z, N);
                    rb.add(sv.w, ev.w, N);
                }
            } else {
#pragma unroll 8
                for (int r = r0 + g; r < r_end; r += G) rb.add(s_row[r], e_row[r], N);
            }
            for (int off = G >> 1; off > 0; off >>= 1) {
                rb.min_s = min(rb.min_s, __shfl_xor(rb.min_s, off));
                rb.max_e = max(rb.max_e, __shfl_xor(rb.max_e, off));
                rb.max_s = max(rb.max_s, __shfl_xor(rb.max_s, off));
                rb.min_e = min(rb.min_e, __shfl_xor(rb.min_e, off));
            }
            m[k] = rb.meta(N, Bc, n_kv);
        }
        if (g == 0) {
            const int w = union_blocks<NIV>(m);
#pragma unroll
            for (int k = 0; k < NIV; ++k) meta[(int64_t)item * NIV + k] = m[k];
            work[item] = w;
            s_work[item] = w;
        }
    }
    // Rank: the G lanes of item x each count the items ranked ahead of x in
    // one slice of SL entries of s_work (SL a multiple of 4, read 16 bytes at
    // a time); entries past M hold INT_MIN and never count.
    const int SL = (((M + G - 1) / G) + 3) & ~3;
    for (int y = M + threadIdx.x; y < G * SL; y += kPrepThreads) s_work[y] = INT_MIN;
    __syncthreads();
    if (item < M) {
        const int wx = s_work[item];
        const int lo = (item / L) * L;          // the item's segment [lo, lo + L)
        const int hi = lo + L;
        int rank = 0;
        const int4* w4 = reinterpret_cast<const int4*>(s_work + g * SL);
        for (int c = 0; c < SL / 4; ++c) {
            const int4 w = w4[c];
            const int y = g * SL + 4 * c;
            const int wv[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int q = 0; q < 4; ++q)
                rank += (y + q >= lo) & (y + q < hi) & ((wv[q] > wx) | ((wv[q] == wx) & (y + q < item)));
        }
        for (int off = G >> 1; off > 0; off >>= 1) rank += __shfl_xor(rank, off);
        if (g == 0) order[lo + rank] = item;
    }
}

}  // namespace

hipError_t launch_prep_small(const int32_t* col_start, const int32_t* col_end, int n_iv, int64_t B,
                             int64_t N, int Br, int Bc, TileMeta* meta, int32_t* work, int32_t* order,
                             hipStream_t stream, int n_sets) {
    const int64_t n_q = (N + Br - 1) / Br;
    const int64_t n_kv = (N + Bc - 1) / Bc;
    const int64_t L = B * n_q;                  // one segment per interval set
    const int64_t M = n_sets * L;
    if (M > kPrepSmallMax) return hipErrorInvalidValue;
    int G = 64;                                 // lanes per query block: a power of two, G * M <= 1024
    while (G * M > kPrepThreads) G >>= 1;
    // 128-bit interval loads when every query block starts on a 16-byte boundary
    const bool vec4 = N % 4 == 0 && Br % 4 == 0 && (reinterpret_cast<uintptr_t>(col_start) & 15) == 0 &&
                      (reinterpret_cast<uintptr_t>(col_end) & 15) == 0;
    return dispatch_ranges(n_iv, [&](auto niv) {
        hipLaunchKernelGGL(prep_small_kernel<decltype(niv)::value>, dim3(1), dim3(kPrepThreads), 0, stream,
                           col_start, col_end, (int)N, (int)n_q, (int)n_kv, Br, Bc, (int)M, G, vec4, n_sets,
                           (int)L, meta, work, order);
        return hipGetLastError();
    });
}

hipError_t launch_schedule(const int32_t* work, int64_t M, int32_t* order, hipStream_t stream, int64_t L,
                           int shift) {
    if (L <= 0) L = M;
    const int64_t blocks = (M + kThreads - 1) / kThreads;
    hipLaunchKernelGGL(schedule_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, work,
                       (int)M, (int)L, shift, order);
    return hipGetLastError();
}

}  // namespace fm
