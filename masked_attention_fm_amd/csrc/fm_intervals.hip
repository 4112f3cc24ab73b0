// Interval preprocessor and tile-class table (gfx950).
//
// FlashMask article ("FlashMask技术：大模型训练中的高效注意力掩码优化") §2.2:
// each (query block, key block) pair is skipped, computed as a full block, or
// computed with the per-row mask.  Reading used here: a key block is skipped
// when it lies left of every row's start or right of every row's end, and is
// full when it lies inside every row's interval.  Both tests need only the
// minimum and maximum of the block's starts and ends, which one wavefront
// reduces per query block.  From those four numbers the non-skip key blocks
// and the full key blocks each form a single contiguous range.  Rows with
// several ranges (the article's §6.1 item 1, several disjoint column ranges
// per row; §5.2 item 4, attention sinks plus a window) keep one such record
// per range.

#include <climits>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kWavesPerBlock = 4;

// Rows with NIV ranges: the records of the ranges are reduced one after the
// other by the same wavefront; the work of the query block is the size of
// the union of their non-skip ranges.
template <int NIV>
__global__ __launch_bounds__(64 * kWavesPerBlock) void preprocess_kernel(
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_end, int N, int n_q,
    int n_kv, int Br, int Bc, int64_t items, int64_t seg, int n_sets, TileMeta* __restrict__ meta,
    int32_t* __restrict__ work, int32_t* __restrict__ bad) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (item >= items) return;  // whole wavefront leaves together
    const int64_t g = item / seg;              // interval set
    const int64_t rem = item - g * seg;
    const int64_t b = rem / n_q;
    const int t = (int)(rem - b * n_q);
    TileMeta m[NIV];
    int invalid = 0;
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
        const int64_t off = ((b * n_sets + g) * NIV + k) * N;
        int inv = 0;
        m[k] = query_block_meta(col_start + off, col_end + off, t, N, Br, Bc, n_kv, lane, &inv);
        invalid |= inv;
    }
    if (bad != nullptr && invalid) *bad = 1;   // vector store; every writer stores 1
    if (lane == 0) {
#pragma unroll
        for (int k = 0; k < NIV; ++k) meta[item * NIV + k] = m[k];
        if (work != nullptr) work[item] = union_blocks<NIV>(m);
    }
}

// SKIP unless some range keeps the key block; FULL when some range covers it
// for every row of the query block (the union then covers it too); PARTIAL
// otherwise.
template <int NIV>
__global__ __launch_bounds__(256) void class_table_kernel(const TileMeta* __restrict__ meta,
                                                          int64_t n_q, int64_t n_kv,
                                                          uint8_t* __restrict__ table) {
    const int64_t total = n_q * n_kv;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = idx / n_kv;
        const int j = (int)(idx - t * n_kv);
        bool live = false, full = false;
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            const TileMeta m = meta[t * NIV + k];
            const bool in = j >= m.x && j <= m.y;
            live |= in;
            full |= in && j >= m.z && j <= m.w;
        }
        table[idx] = full ? 1 : (live ? 2 : 0);    // FULL : PARTIAL : SKIP
    }
}

}  // namespace

hipError_t launch_preprocess(const int32_t* col_start, const int32_t* col_end, int n_iv, int64_t B,
                             int64_t N, int Br, int Bc, TileMeta* meta, int32_t* work, int32_t* bad,
                             hipStream_t stream, int n_sets) {
    const int64_t n_q = (N + Br - 1) / Br;
    const int64_t n_kv = (N + Bc - 1) / Bc;
    const int64_t seg = B * n_q;
    const int64_t items = n_sets * seg;
    const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    return dispatch_ranges(n_iv, [&](auto niv) {
        hipLaunchKernelGGL(preprocess_kernel<decltype(niv)::value>, dim3((unsigned)blocks),
                           dim3(64 * kWavesPerBlock), 0, stream, col_start, col_end, (int)N, (int)n_q,
                           (int)n_kv, Br, Bc, items, seg, n_sets, meta, work, bad);
        return hipGetLastError();
    });
}

hipError_t launch_class_table(const TileMeta* meta, int n_iv, int64_t n_q, int64_t n_kv, uint8_t* table,
                              hipStream_t stream) {
    const int64_t total = n_q * n_kv;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    return dispatch_ranges(n_iv, [&](auto niv) {
        hipLaunchKernelGGL(class_table_kernel<decltype(niv)::value>, dim3((unsigned)blocks), dim3(256), 0,
                           stream, meta, n_q, n_kv, table);
        return hipGetLastError();
    });
}

}  // namespace fm
