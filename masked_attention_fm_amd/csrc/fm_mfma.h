// Device helpers shared by the attention kernels of libflashmask (not installed):
// operand types of v_mfma_f32_32x32x16_bf16, the transposed-operand key order,
// half-wave exchange, buffer descriptors and the 4 x 8 transposing store.
//
// Lane layouts of v_mfma_f32_32x32x16_bf16 (C[32x32] += A[32x16] B[16x32]):
//   A[i][k]: lane i + 32 (k / 8), element k % 8;
//   B[k][j]: lane j + 32 (k / 8), element k % 8;
//   C[i][j]: lane j + 32 h, register v with i = 8 (v / 4) + 4 h + v % 4.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kEmptyStart = -(1 << 30);        // staged start of a range that holds no key
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Position of index j (within a 16-aligned group) in a transposed operand row
// of LDS.  A product whose B operand comes straight from a C-layout register
// tile consumes, in contraction step ks and half-wave h, indices
// 16ks + 8a + 4h + q (a = 0,1; q = 0..3) -- the indices that half-wave holds
// in its C registers.  Swapping bits 2 and 3 of j makes those eight indices
// contiguous, so the A operand is one 16-byte read.
__device__ __forceinline__ int vt_pos(int j) {
    return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

// Combine a value with the one held by the other 32-lane half (lane l ^ 32).
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Buffer descriptor over one (b, h) slice: 32-bit byte offsets from a scalar
// base, and the hardware returns zeros for any offset at or past num_records,
// so rows past N need no clamp or branch.
constexpr uint32_t kRawBufferFlags = 0x00020000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t slice_rsrc(const uint16_t* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, bytes, kRawBufferFlags);
}

// Four rows x eight bf16 columns (rows[r] = columns n0..n0+7 of row r) written
// transposed: columns n0 + c become rows of `dst` (pitch `pitch` elements),
// each receiving the four values at column offset p.  v_perm_b32 regroups the
// bf16 pairs: low halves give the even column, high halves the odd one.
__device__ __forceinline__ void store_transposed_4x8(const u32x4 (&rows)[4], uint16_t* dst, int pitch, int n0,
                                                     int p) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        const uint32_t a0 = rows[0][w], a1 = rows[1][w], a2 = rows[2][w], a3 = rows[3][w];
        const u32x2 even = {__builtin_amdgcn_perm(a1, a0, 0x05040100u), __builtin_amdgcn_perm(a3, a2, 0x05040100u)};
        const u32x2 odd = {__builtin_amdgcn_perm(a1, a0, 0x07060302u), __builtin_amdgcn_perm(a3, a2, 0x07060302u)};
        *reinterpret_cast<u32x2*>(dst + (n0 + 2 * w) * pitch + p) = even;
        *reinterpret_cast<u32x2*>(dst + (n0 + 2 * w + 1) * pitch + p) = odd;
    }
}

}  // namespace fm
