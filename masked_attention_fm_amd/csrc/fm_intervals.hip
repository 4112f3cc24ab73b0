// Interval preprocessor and tile-class table (gfx950).
//
// FlashMask article ("FlashMask技术：大模型训练中的高效注意力掩码优化") §2.2:
// each (query block, key block) pair is skipped, computed as a full block, or
// computed with the per-row mask.  Reading used here: a key block is skipped
// when it lies left of every row's start or right of every row's end, and is
// full when it lies inside every row's interval.  Both tests need only the
// minimum and maximum of the block's starts and ends, which one wavefront
// reduces per query block.  From those four numbers the non-skip key blocks
// and the full key blocks each form a single contiguous range.

#include <climits>

#include "fm_internal.h"

namespace fm {
namespace {

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(64 * kWavesPerBlock) void preprocess_kernel(
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_end, int N, int n_q,
    int n_kv, int Br, int Bc, int64_t items, TileMeta* __restrict__ meta,
    int32_t* __restrict__ work, int32_t* __restrict__ bad) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
    if (item >= items) return;  // whole wavefront leaves together
    const int64_t b = item / n_q;
    const int t = (int)(item - b * n_q);
    int invalid = 0;
    const TileMeta m = query_block_meta(col_start + b * N, col_end + b * N, t, N, Br, Bc, n_kv, lane,
                                        &invalid);
    if (bad != nullptr && invalid) *bad = 1;   // vector store; every writer stores 1
    if (lane == 0) {
        meta[item] = m;
        if (work != nullptr) work[item] = m.y >= m.x ? m.y - m.x + 1 : 0;
    }
}

__global__ __launch_bounds__(256) void class_table_kernel(const TileMeta* __restrict__ meta,
                                                          int64_t n_q, int64_t n_kv,
                                                          uint8_t* __restrict__ table) {
    const int64_t total = n_q * n_kv;
    for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = idx / n_kv;
        const int j = (int)(idx - t * n_kv);
        const TileMeta m = meta[t];
        uint8_t c = 0;                                   // SKIP
        if (j >= m.x && j <= m.y) c = (j >= m.z && j <= m.w) ? 1 : 2;   // FULL : PARTIAL
        table[idx] = c;
    }
}

}  // namespace

hipError_t launch_preprocess(const int32_t* col_start, const int32_t* col_end, int64_t B, int64_t N,
                             int Br, int Bc, TileMeta* meta, int32_t* work, int32_t* bad,
                             hipStream_t stream) {
    const int64_t n_q = (N + Br - 1) / Br;
    const int64_t n_kv = (N + Bc - 1) / Bc;
    const int64_t items = B * n_q;
    const int64_t blocks = (items + kWavesPerBlock - 1) / kWavesPerBlock;
    hipLaunchKernelGGL(preprocess_kernel, dim3((unsigned)blocks), dim3(64 * kWavesPerBlock), 0,
                       stream, col_start, col_end, (int)N, (int)n_q, (int)n_kv, Br, Bc, items, meta,
                       work, bad);
    return hipGetLastError();
}

hipError_t launch_class_table(const TileMeta* meta, int64_t n_q, int64_t n_kv, uint8_t* table,
                              hipStream_t stream) {
    const int64_t total = n_q * n_kv;
    int64_t blocks = (total + 255) / 256;
    if (blocks > (1 << 20)) blocks = 1 << 20;
    hipLaunchKernelGGL(class_table_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, meta, n_q,
                       n_kv, table);
    return hipGetLastError();
}

}  // namespace fm
