// Work ordering for the attention kernel (gfx950).
//
// FlashMask article ("FlashMask技术：大模型训练中的高效注意力掩码优化") §4.3
// item 3: hand out the work by each query block's number of effective
// (non-skipped) key blocks, and §4.2 (several query blocks per processor).
// Under document or sliding masks the per-block work is very uneven (a
// query block at the end of a long document needs many key blocks, one at
// the start of a short document needs one), so the blocks are issued
// longest first: the long ones start early and the short ones fill the
// tail.  The order is a stable sort by decreasing work: items of equal work
// keep their index order.  On large problems the attention order sorts by
// work in buckets of 32 key blocks, so that the query blocks of one document
// that need about the same work run together and share their K/V in the
// XCD's L2.  The order never changes a result: every query block's output
// depends only on its own fixed sequence of key blocks.
//
// The sort is deterministic and has no floating point:
//   * a segment of at most kSortSmall items is sorted by one workgroup: each
//     item becomes the 32-bit key ((kmax - work') << bits) | index, unique
//     and ordered exactly as the result must be (work' = bucketed work + 1,
//     so that the -1 of unused backward entries sorts last), and a bitonic
//     network sorts the keys in LDS;
//   * a longer segment is a counting sort over work' (at most max_work + 2
//     values): chunks of kSortChunk items are sorted in LDS as above, which
//     gives each item its rank among the equal-work items of its chunk and
//     each chunk's count per work value; a second launch turns the counts
//     into each chunk's first position per work value (work values in
//     decreasing order, chunks in index order); a third places every item.
//     Work and memory are linear in the items plus chunks x work values.

#include <climits>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kSortThreads = 1024;

// Work value of an item: its bucketed work shifted up by one (so -1 becomes
// 0), clamped to [0, kw_max].  Every pass clamps alike, so the positions the
// counting sort hands out always form a permutation of the segment.
__device__ __forceinline__ int work_value(int w, int shift, int kw_max) {
    const int kw = (w >> shift) + 1;
    return kw < 0 ? 0 : (kw > kw_max ? kw_max : kw);
}

// Sort key of an item: the work value, decreasing, then the index inside the
// sorted run, increasing (kw_max <= kmax = 2^(32 - bits) - 1).
__device__ __forceinline__ uint32_t sort_key(int kw, int idx, int bits) {
    const uint32_t kmax = (1u << (32 - bits)) - 1u;
    return ((kmax - (uint32_t)kw) << bits) | (uint32_t)idx;
}

// Ascending bitonic sort of n = E * kSortThreads 32-bit keys (E a power of two,
// at most kMaxPerThread) held E per thread in registers, thread t holding
// elements t E .. t E + E - 1.  A compare-exchange of elements x and x ^ j
// keeps the smaller value in the lower element when (x & k) == 0 (ascending
// run), the larger otherwise.  Partners inside one thread (j < E) exchange in
// registers, partners inside one wavefront (j < 64 E) with lane shuffles, and
// only the stages whose partners lie in other wavefronts go through LDS
// (buffer s, n entries), two barriers each.
constexpr int kMaxPerThread = kSortSmall / kSortThreads;   // 16

template <int E>
__device__ __forceinline__ void bitonic_sort_regs(uint32_t (&v)[E], uint32_t* s) {
    static_assert(E >= 1 && E <= kMaxPerThread && (E & (E - 1)) == 0, "a power of two, at most kMaxPerThread");
    constexpr int n = E * kSortThreads;
    const int t = threadIdx.x;
    for (int k = 2; k <= n; k <<= 1) {
        for (int j = k >> 1; j > 0; j >>= 1) {
            if (j < E) {
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const int pr = r ^ j;
                    if (pr > r) {
                        const int x = t * E + r;
                        const bool up = (x & k) == 0;
                        const uint32_t a = v[r], b = v[pr];
                        v[r] = up ? min(a, b) : max(a, b);
                        v[pr] = up ? max(a, b) : min(a, b);
                    }
                }
            } else if (j < 64 * E) {
                const int lane_mask = j / E;
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const int x = t * E + r;
                    const uint32_t other = (uint32_t)__shfl_xor((int)v[r], lane_mask);
                    const bool keep_min = ((x & j) == 0) == ((x & k) == 0);
                    v[r] = keep_min ? min(v[r], other) : max(v[r], other);
                }
            } else {
#pragma unroll
                for (int r = 0; r < E; ++r) s[t * E + r] = v[r];
                __syncthreads();
#pragma unroll
                for (int r = 0; r < E; ++r) {
                    const int x = t * E + r;
                    const uint32_t other = s[x ^ j];
                    const bool keep_min = ((x & j) == 0) == ((x & k) == 0);
                    v[r] = keep_min ? min(v[r], other) : max(v[r], other);
                }
                __syncthreads();
            }
        }
    }
}

// Sorts the keys key(i) for i < count (entries up to n hold 0xFFFFFFFF) and
// leaves them sorted in s[0, n); n = E * kSortThreads.
template <int E, typename KeyOf>
__device__ __forceinline__ void sort_into_lds(uint32_t* s, int count, KeyOf key) {
    uint32_t v[E];
#pragma unroll
    for (int r = 0; r < E; ++r) {
        const int x = threadIdx.x * E + r;
        v[r] = x < count ? key(x) : 0xFFFFFFFFu;
    }
    bitonic_sort_regs<E>(v, s);
#pragma unroll
    for (int r = 0; r < E; ++r) s[threadIdx.x * E + r] = v[r];
    __syncthreads();
}

// Dispatch on the per-thread count for n = max(kSortThreads, next power of two >= count).
template <typename KeyOf>
__device__ __forceinline__ int sort_keys(uint32_t* s, int count, KeyOf key) {
    int e = 1;
    while (e * kSortThreads < count) e <<= 1;
    switch (e) {
        case 1: sort_into_lds<1>(s, count, key); break;
        case 2: sort_into_lds<2>(s, count, key); break;
        case 4: sort_into_lds<4>(s, count, key); break;
        case 8: sort_into_lds<8>(s, count, key); break;
        default: sort_into_lds<16>(s, count, key); break;
    }
    return e * kSortThreads;
}

// One segment of L <= kSortSmall items per workgroup: keys into registers,
// sort, write the order.  Padding entries hold 0xFFFFFFFF, which no item's
// key reaches (an item key with every bit set would need index
// 2^bits - 1 >= L).
__global__ __launch_bounds__(kSortThreads) void order_small_kernel(const int32_t* __restrict__ work, int L, int shift,
                                                                   int32_t* __restrict__ order) {
    __shared__ uint32_t s[kSortSmall];
    const int64_t lo = (int64_t)blockIdx.x * L;
    sort_keys(s, L, [&](int i) {
        return sort_key(work_value(work[lo + i], shift, (1 << (32 - kSortSmallBits)) - 1), i, kSortSmallBits);
    });
    const uint32_t mask = (1u << kSortSmallBits) - 1u;
    for (int p = threadIdx.x; p < L; p += kSortThreads) order[lo + p] = (int32_t)(lo + (s[p] & mask));
}

// Counting sort, pass 1: chunk t (chunk c of segment g) sorts its keys in LDS;
// item at sorted position p gets its rank among the equal-work items of the
// chunk (p minus the first position of its work value), and the last item of
// each run stores the run's length as the chunk's count for that work value.
// cnt[t][*] is cleared first by the same workgroup.
__global__ __launch_bounds__(kSortThreads) void order_count_kernel(const int32_t* __restrict__ work, int L,
                                                                   int n_chunks, int shift, int n_keys,
                                                                   int32_t* __restrict__ cnt,
                                                                   int32_t* __restrict__ lrank) {
    __shared__ uint32_t s[kSortChunk];
    const int t = blockIdx.x;
    const int g = t / n_chunks;
    const int c = t - g * n_chunks;
    const int64_t base = (int64_t)g * L + (int64_t)c * kSortChunk;
    const int n_c = min(kSortChunk, L - c * kSortChunk);
    int32_t* row = cnt + (int64_t)t * n_keys;
    for (int k = threadIdx.x; k < n_keys; k += kSortThreads) row[k] = 0;
    __syncthreads();                                       // the row is cleared before any count is stored
    static_assert(kSortChunk == 8 * kSortThreads, "eight keys per thread");
    sort_into_lds<8>(s, n_c, [&](int i) {
        return sort_key(work_value(work[base + i], shift, n_keys - 1), i, kSortChunkBits);
    });
    const uint32_t kmax = (1u << (32 - kSortChunkBits)) - 1u;
    const uint32_t mask = (1u << kSortChunkBits) - 1u;
    for (int p = threadIdx.x; p < n_c; p += kSortThreads) {
        const uint32_t hi = s[p] >> kSortChunkBits;
        int a = 0, b = p;                                  // first position whose key part is hi
        while (a < b) {
            const int m = (a + b) >> 1;
            if ((s[m] >> kSortChunkBits) < hi) a = m + 1; else b = m;
        }
        lrank[base + (s[p] & mask)] = p - a;
        const bool last = p + 1 == n_c || (s[p + 1] >> kSortChunkBits) != hi;
        const int kw = (int)(kmax - hi);                   // work value of the run (< n_keys)
        if (last) row[kw] = p - a + 1;
    }
}

// Counting sort, pass 2 (one workgroup per segment): for every work value w'
// (thread i takes the values at descending positions [i per, (i+1) per)),
// cnt[(g, c)][w'] becomes the number of items of value w' in the segment's
// earlier chunks, and start[g][w'] the number of items of larger value.
__global__ __launch_bounds__(kSortThreads) void order_offsets_kernel(int n_chunks, int n_keys,
                                                                     int32_t* __restrict__ cnt,
                                                                     int32_t* __restrict__ start) {
    __shared__ int s_sum[kSortThreads];
    const int g = blockIdx.x;
    const int per = (n_keys + kSortThreads - 1) / kSortThreads;
    const int q0 = threadIdx.x * per;
    const int q1 = min(n_keys, q0 + per);
    int32_t* st = start + (int64_t)g * n_keys;
    int mine = 0;
    for (int q = q0; q < q1; ++q) {
        const int kw = n_keys - 1 - q;
        int run = 0;
        for (int c = 0; c < n_chunks; ++c) {
            int32_t* e = cnt + ((int64_t)g * n_chunks + c) * n_keys + kw;
            const int v = *e;
            *e = run;
            run += v;
        }
        st[kw] = run;                                      // the value's total, for now
        mine += run;
    }
    s_sum[threadIdx.x] = mine;
    __syncthreads();
    // exclusive scan of the per-thread sums (Hillis-Steele, in place)
    for (int off = 1; off < kSortThreads; off <<= 1) {
        const int v = threadIdx.x >= off ? s_sum[threadIdx.x - off] : 0;
        __syncthreads();
        s_sum[threadIdx.x] += v;
        __syncthreads();
    }
    int acc = s_sum[threadIdx.x] - mine;
    for (int q = q0; q < q1; ++q) {
        const int kw = n_keys - 1 - q;
        const int tot = st[kw];
        st[kw] = acc;
        acc += tot;
    }
}

// Counting sort, pass 3: every item's place.
__global__ __launch_bounds__(256) void order_place_kernel(const int32_t* __restrict__ work, int64_t M, int L,
                                                          int n_chunks, int shift, int n_keys,
                                                          const int32_t* __restrict__ cnt,
                                                          const int32_t* __restrict__ start,
                                                          const int32_t* __restrict__ lrank,
                                                          int32_t* __restrict__ order) {
    const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (x >= M) return;
    const int64_t g = x / L;
    const int in_seg = (int)(x - g * L);
    const int c = in_seg / kSortChunk;
    const int kw = work_value(work[x], shift, n_keys - 1);
    const int pos = start[g * n_keys + kw] + cnt[(g * n_chunks + c) * n_keys + kw] + lrank[x];
    order[g * L + pos] = (int32_t)x;
}

constexpr int kPrepThreads = 1024;
// LDS slots of the one-launch prep's rank: G lanes per item (G <= 64) each
// take SL entries, SL = (ceil(M / G) + 3) rounded down to a multiple of 4,
// so G * SL <= G * ceil(M / G) + 3 G <= M + 4 G <= kPrepSmallMax + 256.
constexpr int kPrepWorkSlots = kPrepSmallMax + 4 * 64;

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
    // work of each item, padded with INT_MIN up to G * SL <= kPrepWorkSlots entries
    __shared__ __attribute__((aligned(16))) int s_work[kPrepWorkSlots];
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

int64_t schedule_scratch_ints(int64_t M, int64_t L, int shift, int max_work) {
    if (L <= 0) L = M;
    if (L <= kSortSmall) return 0;
    const int64_t S = M / L;
    const int64_t chunks = (L + kSortChunk - 1) / kSortChunk;
    const int64_t n_keys = (int64_t)(max_work >> shift) + 2;
    return S * chunks * n_keys + S * n_keys + M;
}

hipError_t launch_schedule(const int32_t* work, int64_t M, int32_t* order, hipStream_t stream, int64_t L,
                           int shift, int max_work, int32_t* scratch) {
    if (L <= 0) L = M;
    if (M <= 0 || M % L != 0 || max_work < 0) return hipErrorInvalidValue;
    const int64_t S = M / L;
    if (L <= kSortSmall) {
        hipLaunchKernelGGL(order_small_kernel, dim3((unsigned)S), dim3(kSortThreads), 0, stream, work, (int)L, shift,
                           order);
        return hipGetLastError();
    }
    // counting sort: keys are work' = (work >> shift) + 1 in [0, n_keys)
    const int64_t n_keys = (int64_t)(max_work >> shift) + 2;
    if (scratch == nullptr || n_keys > (int64_t(1) << (32 - kSortChunkBits))) return hipErrorInvalidValue;
    const int64_t chunks = (L + kSortChunk - 1) / kSortChunk;
    int32_t* cnt = scratch;
    int32_t* start = cnt + S * chunks * n_keys;
    int32_t* lrank = start + S * n_keys;
    hipLaunchKernelGGL(order_count_kernel, dim3((unsigned)(S * chunks)), dim3(kSortThreads), 0, stream, work,
                       (int)L, (int)chunks, shift, (int)n_keys, cnt, lrank);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(order_offsets_kernel, dim3((unsigned)S), dim3(kSortThreads), 0, stream, (int)chunks,
                       (int)n_keys, cnt, start);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(order_place_kernel, dim3((unsigned)((M + 255) / 256)), dim3(256), 0, stream, work, M, (int)L,
                       (int)chunks, shift, (int)n_keys, cnt, start, lrank, order);
    return hipGetLastError();
}

}  // namespace fm
