// Internal declarations shared by the HIP sources of libflashmask (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

// Tile shape of the attention kernel: 4 wavefronts x 32 query rows, 64 keys per step.
constexpr int kBr = 128;
constexpr int kBc = 64;

// Per query block (one sequence of one batch), computed from its rows' intervals:
//   x = first non-skip key block, y = last non-skip key block (y < x: none),
//   z = first FULL key block,     w = last FULL key block     (w < z: none).
// Under the min/max rule the non-skip blocks and the full blocks each form one
// contiguous range, so four integers describe the whole row of the class table.
using TileMeta = int4;

// Interval preprocessor: one wavefront per (b, query block).
//   meta[b*n_q + t], work[b*n_q + t] = non-skip key blocks (may be null),
//   bad (may be null): set to 1 when a row breaks 0 <= s <= e <= N-1.
hipError_t launch_preprocess(const int32_t* col_start, const int32_t* col_end, int64_t B, int64_t N,
                             int Br, int Bc, TileMeta* meta, int32_t* work, int32_t* bad,
                             hipStream_t stream);

// Expands meta of n_q query blocks into the uint8 class table [n_q][n_kv].
hipError_t launch_class_table(const TileMeta* meta, int64_t n_q, int64_t n_kv, uint8_t* table,
                              hipStream_t stream);

// Longest-first order of M work items (ties by index).
hipError_t launch_schedule(const int32_t* work, int64_t M, int32_t* order, hipStream_t stream);

// Attention kernel.  order == nullptr runs query blocks in natural (b, t) order.
// start/stop (may be null) are stamped at the kernel's own start and end.
hipError_t launch_attention(const void* q, const void* k, const void* v, const int32_t* col_start,
                            const int32_t* col_end, const TileMeta* meta, const int32_t* order,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale, void* out,
                            float* lse, hipStream_t stream, hipEvent_t start, hipEvent_t stop);

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

__device__ __forceinline__ int wave_max(int v) {
    v = max(v, swizzle_xor<1>(v));
    v = max(v, swizzle_xor<2>(v));
    v = max(v, swizzle_xor<4>(v));
    v = max(v, swizzle_xor<8>(v));
    v = max(v, swizzle_xor<16>(v));
    return max(__builtin_amdgcn_readlane(v, 0), __builtin_amdgcn_readlane(v, 32));
}

}  // namespace fm
