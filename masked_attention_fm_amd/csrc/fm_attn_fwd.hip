// Masked attention forward kernel for gfx950 (MI355X).
//
// Method: FlashMask article ("FlashMask技术：大模型训练中的高效注意力掩码优化")
//   §2.2  skip / full / partial decision per (query block, key block);
//   §4.1  intervals cached on chip (item 1), skip decided before any key or
//         value is loaded (item 2), inclusive interval compare fused into the
//         score of boundary blocks only (item 3);
// FlashAttention article ("FlashAttention优化：高效训练长上下文GPT的技术突破")
//   §2 items 1-3  blocks of keys streamed through on-chip memory, softmax
//         with the running maximum subtracted and earlier blocks rescaled,
//         both products fused in one kernel on the matrix units.
//
// Design (one workgroup = one query block of kBr = 128 rows of one (b, h)):
//   * 4 wavefronts, each owns 32 query rows.  Its Q rows stay in registers
//     for the whole key loop as the B operand of v_mfma_f32_32x32x16_bf16.
//   * The score block is computed transposed, S^T = K Q^T, so that in the
//     MFMA result layout lane l holds 16 keys of query row l % 32.  A row
//     maximum is then 15 register max operations and one exchange with the
//     other half-wave; the row sum needs no exchange until the end.
//   * The output is also accumulated transposed, O^T = V^T P^T, so that the
//     same lane holds the same query row in O: the rescale factor of a row
//     never leaves its lane.  P^T is taken straight from the S^T registers
//     (converted to bf16) as the B operand; the contraction index of the two
//     operands is permuted consistently so no data moves between lanes.
//   * K and V pass through a double-buffered LDS ring: while block j is
//     computed, block j+1 is loaded from HBM straight into the other buffer
//     (buffer loads with an LDS destination, no registers involved); one
//     barrier per key block.  K is read row-major as the A operand of the
//     score product (six reads ahead of the MFMAs), V transposed
//     (ds_read_b64_tr_b16) as the A operand of the PV product (FP8 inputs:
//     the same with bytes, see below).  These operand reads are issued as
//     inline assembly with explicit waits, so their pipelining does not
//     depend on the compiler's schedule.
//   * Softmax with lazy rescaling: a row's reference maximum may lag its
//     running maximum by up to 2^8 in weight, so the accumulator is rescaled
//     only when some row of the wavefront outgrows that margin.
//   * Key blocks outside the query block's non-skip range are never visited
//     (range from the interval preprocessor).  Inside the range each
//     wavefront tests its own 32 rows: it skips blocks none of its rows
//     attends and applies the interval compare only when the block is not
//     inside all of its rows' intervals.
//   * Rows may hold up to kMaxRanges ranges (FlashMask article §6.1 item 1,
//     several column ranges per row; §5.2 item 4, sinks plus a window).  The
//     kernel is instantiated per range count NIV: the visited key blocks are
//     the union of the ranges' non-skip blocks in increasing order, a block
//     is skipped or full for a wavefront by the per-range tests above, and
//     the compare keeps a key that lies in any of the row's ranges.  With
//     NIV = 1 this is the single-range kernel.
//   * A second instantiation (F8) takes e4m3 Q, K, V: the score product runs
//     on the FP8 matrix instruction; V is widened to bf16 as it is read for
//     the PV product, or, with e4m3 weights as well, that product runs on the
//     FP8 matrix instruction too (see the FP8 section below).
//   * With one interval set per head, head h reads set h; the work items of
//     each set are a contiguous, separately ranked segment of the order.

#include <hip/hip_ext.h>
#include <math.h>
#include <stddef.h>

#include <type_traits>

#include "fm_internal.h"
#include "fm_mfma.h"

namespace fm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = kBr / kWaves;     // 32

static_assert(kRowsPerWave == 32, "one 32x32 MFMA column block per wavefront");
static_assert(kBc % 32 == 0 && kBc % 16 == 0, "key block is a multiple of the MFMA shapes");

// acc + the sum of eight bf16 values, two per v_dot2 against (1, 1).
__device__ __forceinline__ float sum_bf16x8(bf16x8 p, bf16x2 ones, float acc) {
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 0, 1), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 2, 3), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 4, 5), ones, acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(p, p, 6, 7), ones, acc, false);
    return acc;
}

// ---- bf16 K and V blocks, loaded straight from global memory into LDS.
//
// A `buffer_load_dwordx4 ... lds` writes the 16 bytes of lane l to LDS
// address M0 + 16 l: one instruction fills a contiguous 1 KB segment, each
// lane fetching whichever 16 bytes of the block it is given.  Rows past N
// read as zero (the buffer range check), so their scores are masked and their
// values meet a weight of exactly 0.  No registers, VALU work or LDS store
// instructions are spent on staging.
//
// A segment holds kSegKeys = 1024 / (2 D) key rows (4 at d = 128, 8 at
// d = 64): key kappa of the block sits in segment kappa % kSegs, slot
// kappa / kSegs.  Segments are padded so that the operand reads below are
// free of bank conflicts:
//   * K, pitch 1024 + 16 B.  The score product reads 16 bytes of one key per
//     lane, eight consecutive keys per 8-lane phase: consecutive keys are in
//     consecutive segments, 16 bytes apart modulo 128.
//   * V, pitch 1024 + 64 B.  The PV product needs V^T, read with
//     ds_read_b64_tr_b16: within each 16-lane group, local lane i receives
//     element i % 4 of the 8-byte pieces addressed by lanes 4 e + i / 4,
//     e = 0..3 (verified by an in-bounds probe).  Lane 4 e + c addresses key
//     kappa0 + e, columns n0 + 4 c .. + 3, so lane i ends up with column
//     n0 + i of keys kappa0 .. kappa0 + 3.  The read serves 32 lanes per pass
//     (two groups: the two 16-column halves of the same four keys); the four
//     keys are in consecutive segments, 64 bytes apart modulo 256, and the
//     column halves 32 bytes apart: one 256-byte sweep per pass (a probe
//     measured no bank conflicts; a 32-byte pitch remainder gave two-way
//     conflicts).
template <int D>
struct Direct {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kSegKeys = 1024 / kRowBytes;
    static constexpr int kSegs = kBc / kSegKeys;
    static constexpr int kKPitch = 1024 + 16;
    static constexpr int kVPitch = 1024 + 64;
    static constexpr int kKBytes = kSegs * kKPitch;
    static constexpr int kVBytes = kSegs * kVPitch;
    static constexpr int kSegsPerWave = kSegs / kWaves;
    static_assert(kSegKeys * kSegs == kBc && kSegsPerWave * kWaves == kSegs, "segments split evenly");
    static_assert(kSegs % 8 == 0, "eight consecutive keys in distinct segments");
};

template <int D, int NIV>
struct alignas(16) Smem {
    alignas(16) uint8_t k[2][Direct<D>::kKBytes];
    alignas(16) uint8_t v[2][Direct<D>::kVBytes];
    int start[NIV][kBr];                          // clamped start of each range of each query row
                                                  // (kEmptyStart: the range holds no key)
    int width[NIV][kBr];                          // end - start (0 for empty ranges)
};

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// Byte offset, inside a block's slice of K or V, of this lane's 16 bytes in
// the first segment its wavefront fills (wave_u: the wavefront index).
template <int D>
__device__ __forceinline__ int direct_lane_offset(int lane, int wave_u) {
    using L = Direct<D>;
    const int slot = lane / (D / 8);
    const int chunk = lane % (D / 8);
    return (wave_u * L::kSegsPerWave + L::kSegs * slot) * L::kRowBytes + 16 * chunk;
}

// ---- V^T operand reads for the PV product (bf16 path).
//
// The transposing read is issued through inline assembly: the compiler
// treats the ds_read_tr builtin as a read of any LDS location and would wait
// for the next block's in-flight loads before every one of them, which
// serialises the prefetch with the compute.  The reads here target the
// current buffer only, which no in-flight load writes.  Their completion is
// waited for explicitly (LDS operations complete in issue order, so
// lgkmcnt(n) after n younger reads guarantees the older ones), and each wait
// passes the registers through itself so nothing can use them earlier.
// `after` is not used by the instruction: it only orders the read after the
// computation of that value.
template <int OFF>
__device__ __forceinline__ v4s lds_read_tr16(uint32_t addr, float after) {
    v4s r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF), "v"(after));
    return r;
}

// The 2 D / 32 reads of step KS (16 keys): part[2 nb + r] holds, for lane
// (column i, half h), keys 16 KS + 8 r + 4 h + 0..3 of column 32 nb + i.
template <int D, int KS, int I = 0>
__device__ __forceinline__ void issue_v_reads(v4s (&part)[2 * D / 32], uint32_t addr, float after = 0.f) {
    using L = Direct<D>;
    if constexpr (I < 2 * D / 32) {
        constexpr int nb = I / 2, r = I % 2;
        constexpr int key0 = 16 * KS + 8 * r;
        constexpr int off = (key0 % L::kSegs) * L::kVPitch + (key0 / L::kSegs) * L::kRowBytes + nb * 64;
        static_assert(off >= 0 && off < 65536, "ds offset field");
        part[I] = lds_read_tr16<off>(addr, after);
        issue_v_reads<D, KS, I + 1>(part, addr, after);
    }
}

// Wait until at most CNT LDS operations are outstanding; part is passed
// through the wait.
template <int CNT, int NP>
__device__ __forceinline__ void wait_lds_tied(v4s (&p)[NP]) {
    static_assert(CNT >= 0 && CNT <= 15, "lgkmcnt field");
    if constexpr (NP == 8)
        asm volatile("s_waitcnt lgkmcnt(%8)"
                     : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]), "+v"(p[4]), "+v"(p[5]), "+v"(p[6]),
                       "+v"(p[7])
                     : "i"(CNT));
    else if constexpr (NP == 4)
        asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]) : "i"(CNT));
    else
        static_assert(NP == 8 || NP == 4, "d = 64 or 128");
}

// K operand read of the score product: 16 bytes of one key row per lane
// (the compiler's schedule of these reads is not kept stable across changes
// elsewhere in the kernel, so they are issued explicitly, like the V reads).
template <int OFF>
__device__ __forceinline__ u32x4 lds_read_b128(uint32_t addr) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}
template <int CNT>
__device__ __forceinline__ void wait_lds_one(u32x4& r) {
    static_assert(CNT >= 0 && CNT <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(r) : "i"(CNT));
}

// S^T = K Q^T for one key block: MFMA i (i = 2 cs + jb) takes K rows of key
// half jb, head-dimension chunk cs.  The reads run kAheadK ahead of the MFMA
// that consumes them, through a ring of kAheadK registers.
constexpr int kAheadK = 6;
template <int D>
constexpr int k_read_offset(int i) {
    return (i % 2) * (32 / Direct<D>::kSegs) * Direct<D>::kRowBytes + (i / 2) * 32;
}
template <int D, int I = 0>
__device__ __forceinline__ void issue_k_reads(u32x4 (&ring)[kAheadK], uint32_t addr) {
    if constexpr (I < kAheadK) {
        ring[I] = lds_read_b128<k_read_offset<D>(I)>(addr);
        issue_k_reads<D, I + 1>(ring, addr);
    }
}
template <int D, int I = 0>
__device__ __forceinline__ void score_direct(floatx16 (&st)[kBc / 32], const bf16x8 (&q)[D / 16], uint32_t addr,
                                             u32x4 (&ring)[kAheadK]) {
    constexpr int kMfmas = (D / 16) * (kBc / 32);
    static_assert(kBc / 32 == 2 && kMfmas > kAheadK, "two key halves, more MFMAs than reads in flight");
    if constexpr (I < kMfmas) {
        constexpr int issued = I + kAheadK < kMfmas ? I + kAheadK : kMfmas;
        wait_lds_one<issued - (I + 1)>(ring[I % kAheadK]);
        st[I % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ring[I % kAheadK]), q[I / 2],
                                                            st[I % 2], 0, 0, 0);
        if constexpr (I + kAheadK < kMfmas)
            ring[I % kAheadK] = lds_read_b128<k_read_offset<D>(I + kAheadK)>(addr);
        score_direct<D, I + 1>(st, q, addr, ring);
    }
}

// O^T += V^T P^T over steps KS.. of one key block.  cur holds step KS's
// reads (issued earlier); the next step's reads are issued before waiting
// for them.
//
// The weights of step KS are formed here, from the scores: P = 2^(S c - m),
// summed in fp32 into rs (in the same key order as a loop over the block) and
// rounded to bf16 for the product, so that the exponentials of one step run
// while the previous step's MFMAs execute.
template <int D, int KS>
__device__ __forceinline__ void pv_direct(const floatx16 (&st)[kBc / 32], floatx16 (&oacc)[D / 32],
                                          uint32_t addr, float c, float m_use, float& rs, float& rs16,
                                          bf16x2 ones, v4s (&cur)[2 * D / 32]) {
    constexpr int NP = 2 * D / 32;
    if constexpr (KS < kBc / 16) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float p = __builtin_amdgcn_exp2f(fmaf(st[KS >> 1][8 * (KS & 1) + e], c, -m_use));
            rs += p;
            pb[e] = (__bf16)p;
        }
        rs16 = sum_bf16x8(pb, ones, rs16);
        v4s next[NP];
        if constexpr (KS + 1 < kBc / 16) {
            issue_v_reads<D, KS + 1>(next, addr);
            wait_lds_tied<NP>(cur);
        } else {
            wait_lds_tied<0>(cur);
        }
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(cur[2 * nb], cur[2 * nb + 1], 0, 1, 2, 3, 4, 5, 6, 7));
            oacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, oacc[nb], 0, 0, 0);
        }
        pv_direct<D, KS + 1>(st, oacc, addr, c, m_use, rs, rs16, ones, next);
    }
}

// Segment U of this wavefront's share.  The key row is selected through the
// lane offset: an instruction offset would move the LDS destination as well.
template <int D, int NIV, int U>
__device__ __forceinline__ void load_segment(Smem<D, NIV>& sm, int buf, __amdgpu_buffer_rsrc_t krs,
                                             __amdgpu_buffer_rsrc_t vrs, int off, int wave_u) {
    using L = Direct<D>;
    if constexpr (U < L::kSegsPerWave) {
        const int seg = wave_u * L::kSegsPerWave + U;
        const int row_off = off + U * L::kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)&sm.k[buf][seg * L::kKPitch], 16, row_off, 0, 0,
                                                 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)&sm.v[buf][seg * L::kVPitch], 16, row_off, 0, 0,
                                                 0);
        load_segment<D, NIV, U + 1>(sm, buf, krs, vrs, off, wave_u);
    }
}

// Key block starting at key kv0 into buffer buf (voff = direct_lane_offset).
template <int D, int NIV>
__device__ __forceinline__ void load_block_direct(Smem<D, NIV>& sm, int buf, __amdgpu_buffer_rsrc_t krs,
                                                  __amdgpu_buffer_rsrc_t vrs, int voff, int kv0, int wave_u) {
    load_segment<D, NIV, 0>(sm, buf, krs, vrs, voff + kv0 * Direct<D>::kRowBytes, wave_u);
}

// ---------------------------------------------------------------- FP8 inputs
//
// Q, K and V stored as OCP e4m3 (one byte) with per-tensor dequantization
// scales.  The score product runs on v_mfma_scale_f32_32x32x64_f8f6f4 with
// unit block scales: a 32 x 32 x 64 product whose A and B operands hold 32
// bytes per lane, and whose A row / B column is the lane mod 32 and whose
// contraction index depends only on (lane / 32, byte) in the same way for A
// and B (checked by an in-bounds probe), so any consistent order of the head
// dimension is correct: lane half h of a 64-wide step holds columns
// 64 cs + 32 h + (0..31).  K and V reach LDS as bytes (straight from global
// memory, below).  In the FP8-scores mode V is widened to bf16 as it is read
// for the PV product (exact: the three mantissa bits of e4m3 fit in bf16), so
// the PV product, the weights and the output keep the bf16 path's arithmetic.
constexpr int kUnitScales = 0x7F7F7F7F;        // E8M0 block scale 2^0 in every byte

typedef int v8i __attribute__((ext_vector_type(8)));

// Two e4m3 bytes of `w` (the low or the high half) as a packed bf16 pair.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w) {
    const bf16x2 r = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH);
    return __builtin_bit_cast(uint32_t, r);
}

// ---- e4m3 weights (PREC 2): the PV product on the FP8 unit as well.
//
// The weights P (in (0, 1], the row maximum subtracted) are scaled by 2^8, an
// exact power of two that keeps every weight above 2^-14 out of the e4m3
// subnormals, and rounded to e4m3 (round to nearest even, the hardware
// conversion).  A 64-key block is one 32 x 32 x 64 contraction step; lane half
// h of a row holds, as bytes e = 16 jb + v, the weights of keys
// 32 jb + 8 (v / 4) + 4 h + v % 4 -- exactly the keys its S^T registers hold.
// The A operand (V^T) of lane half h must hold the same keys in the same
// byte order; it is read transposed from V's rows (below).

// K and V of e4m3 weights mode loaded straight into LDS (as in the bf16 path):
// 1 KB segments of kSegKeys = 1024 / D byte rows (8 at d = 128, 16 at d = 64),
// key kappa in segment kappa % kSegs, slot kappa / kSegs.
//   * K, pitch 1024 + 16 B, read row-major: 32 bytes of one key per lane (two
//     16-byte reads); consecutive keys land 16 bytes apart modulo 256.
//   * V, pitch 1024 + 32 B, read transposed with ds_read_b64_tr_b8: within
//     each 16-lane group, lane i receives byte i % 8 of the 8-byte pieces
//     addressed by lanes 2 e + i / 8, e = 0..7 (verified by an in-bounds
//     probe).  Lane 2 e + c addresses the key of byte e of the weights'
//     order, columns n0 + 8 c .., so lane i ends up with column n0 + i of
//     those eight keys; a lane's 32 bytes are four such reads.  The eight keys
//     of a read are 32 bytes apart modulo 256 per segment step and 128 per
//     slot step: one 256-byte sweep per 32-lane pass.
template <int D>
struct Direct8 {
    static constexpr int kRowBytes = D;
    static constexpr int kSegKeys = 1024 / kRowBytes;
    static constexpr int kSegs = kBc / kSegKeys;
    static constexpr int kKPitch = 1024 + 16;
    static constexpr int kVPitch = 1024 + 32;
    static constexpr int kKBytes = kSegs * kKPitch;
    static constexpr int kVBytes = kSegs * kVPitch;
    static constexpr int kSegsPerWave = kSegs / kWaves;
    static_assert(kSegKeys * kSegs == kBc && kSegsPerWave * kWaves == kSegs, "segments split evenly");
};

template <int D, int NIV>
struct alignas(16) Smem8w {
    alignas(16) uint8_t k8[2][Direct8<D>::kKBytes];
    alignas(16) uint8_t v8[2][Direct8<D>::kVBytes];
    int start[NIV][kBr];
    int width[NIV][kBr];
};

// This lane's byte offset inside a key block's e4m3 slice, for the first
// segment its wavefront fills.
template <int D>
__device__ __forceinline__ int direct8_lane_offset(int lane, int wave_u) {
    using L = Direct8<D>;
    const int slot = lane / (L::kRowBytes / 16);
    const int chunk = lane % (L::kRowBytes / 16);
    return (wave_u * L::kSegsPerWave + L::kSegs * slot) * L::kRowBytes + 16 * chunk;
}

template <int D, int NIV, int U = 0>
__device__ __forceinline__ void load_block8_direct(Smem8w<D, NIV>& sm, int buf, __amdgpu_buffer_rsrc_t krs,
                                                   __amdgpu_buffer_rsrc_t vrs, int voff, int kv0, int wave_u) {
    using L = Direct8<D>;
    if constexpr (U < L::kSegsPerWave) {
        const int seg = wave_u * L::kSegsPerWave + U;
        const int row_off = voff + kv0 * L::kRowBytes + U * L::kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)&sm.k8[buf][seg * L::kKPitch], 16, row_off, 0, 0,
                                                 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)&sm.v8[buf][seg * L::kVPitch], 16, row_off, 0, 0,
                                                 0);
        load_block8_direct<D, NIV, U + 1>(sm, buf, krs, vrs, voff, kv0, wave_u);
    }
}

typedef int v2i __attribute__((ext_vector_type(2)));

template <int OFF>
__device__ __forceinline__ v2i lds_read_tr8(uint32_t addr, float after) {
    v2i r;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF), "v"(after));
    return r;
}

// The four reads of output columns 32 NB + (0..31): part[t] holds bytes
// 8 t .. 8 t + 7 of the lane's A operand, keys 32 (t / 2) + 16 (t % 2) +
// 8 (u / 4) + 4 h + u % 4 for byte u.
template <int D, int NB, int T = 0>
__device__ __forceinline__ void issue_v8_reads(v2i (&part)[4], uint32_t addr, float after) {
    using L = Direct8<D>;
    if constexpr (T < 4) {
        constexpr int base = 32 * (T / 2) + 16 * (T % 2);
        constexpr int off = (base / L::kSegs) * L::kRowBytes + 32 * NB;
        static_assert(off >= 0 && off < 65536 && base % L::kSegs == 0, "ds offset field");
        part[T] = lds_read_tr8<off>(addr, after);
        issue_v8_reads<D, NB, T + 1>(part, addr, after);
    }
}

template <int CNT>
__device__ __forceinline__ void wait_lds_tied8(v2i (&p)[4]) {
    static_assert(CNT >= 0 && CNT <= 15, "lgkmcnt field");
    asm volatile("s_waitcnt lgkmcnt(%4)" : "+v"(p[0]), "+v"(p[1]), "+v"(p[2]), "+v"(p[3]) : "i"(CNT));
}

// O^T += V^T P^T on the FP8 units, column blocks NB.. (cur: block NB's reads).
template <int D, int NB>
__device__ __forceinline__ void pv8_direct(const v8i& pb8, floatx16 (&oacc)[D / 32], uint32_t addr, v2i (&cur)[4]) {
    if constexpr (NB < D / 32) {
        v2i next[4];
        if constexpr (NB + 1 < D / 32) {
            issue_v8_reads<D, NB + 1>(next, addr, 0.f);
            wait_lds_tied8<4>(cur);
        } else {
            wait_lds_tied8<0>(cur);
        }
        const v8i a = {cur[0][0], cur[0][1], cur[1][0], cur[1][1], cur[2][0], cur[2][1], cur[3][0], cur[3][1]};
        oacc[NB] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pb8, oacc[NB], 0, 0, 0, kUnitScales, 0,
                                                                   kUnitScales);
        pv8_direct<D, NB + 1>(pb8, oacc, addr, next);
    }
}

// FP8 scores, bf16 weights: O^T += V^T P^T on bf16 MFMAs, column blocks NB..,
// V widened from the same transposing byte reads (read t is step ks = t:
// keys 16 ks + 8 (e / 4) + 4 h + e % 4 for element e, the order of pbs[ks]).
template <int D, int NB>
__device__ __forceinline__ void pv8_bf16_direct(const bf16x8 (&pbs)[kBc / 16], floatx16 (&oacc)[D / 32],
                                                uint32_t addr, v2i (&cur)[4]) {
    if constexpr (NB < D / 32) {
        v2i next[4];
        if constexpr (NB + 1 < D / 32) {
            issue_v8_reads<D, NB + 1>(next, addr, 0.f);
            wait_lds_tied8<4>(cur);
        } else {
            wait_lds_tied8<0>(cur);
        }
#pragma unroll
        for (int ks = 0; ks < kBc / 16; ++ks) {
            const uint32_t w0 = (uint32_t)cur[ks][0], w1 = (uint32_t)cur[ks][1];
            const u32x4 wide = {e4m3x2_to_bf16x2<false>(w0), e4m3x2_to_bf16x2<true>(w0),
                                e4m3x2_to_bf16x2<false>(w1), e4m3x2_to_bf16x2<true>(w1)};
            oacc[NB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wide), pbs[ks], oacc[NB],
                                                               0, 0, 0);
        }
        pv8_bf16_direct<D, NB + 1>(pbs, oacc, addr, next);
    }
}

// The score product for e4m3 inputs: MFMA i (i = 2 cs + jb, 32 x 32 x 64) takes 32
// bytes of K per lane half, two 16-byte reads.  All reads of the block are
// issued first (two per MFMA, 2 D / 32 in all), then each MFMA waits for its
// own two.
template <int D>
constexpr int k8_read_offset(int r) {
    return ((r / 2) % 2) * (32 / Direct8<D>::kSegs) * Direct8<D>::kRowBytes + (r / 4) * 64 + (r % 2) * 16;
}
template <int D, int R = 0>
__device__ __forceinline__ void issue_k8_reads(u32x4 (&rd)[2 * (D / 64) * (kBc / 32)], uint32_t addr) {
    if constexpr (R < 2 * (D / 64) * (kBc / 32)) {
        rd[R] = lds_read_b128<k8_read_offset<D>(R)>(addr);
        issue_k8_reads<D, R + 1>(rd, addr);
    }
}
template <int D, int I = 0>
__device__ __forceinline__ void score8_direct(floatx16 (&st)[kBc / 32], const v8i (&q)[D / 64],
                                              u32x4 (&rd)[2 * (D / 64) * (kBc / 32)]) {
    constexpr int kMfmas = (D / 64) * (kBc / 32);
    static_assert(kBc / 32 == 2 && 2 * kMfmas <= 16, "two key halves; reads fit the lgkm counter");
    if constexpr (I < kMfmas) {
        wait_lds_one<2 * kMfmas - 2 * (I + 1)>(rd[2 * I + 1]);   // in order: 2 I done too
        asm volatile("" : "+v"(rd[2 * I]));
        const v8i a = __builtin_bit_cast(v8i, __builtin_shufflevector(rd[2 * I], rd[2 * I + 1], 0, 1, 2, 3, 4, 5, 6, 7));
        st[I % 2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, q[I / 2], st[I % 2], 0, 0, 0, kUnitScales, 0,
                                                                    kUnitScales);
        __builtin_amdgcn_sched_barrier(0);   // keep MFMA i ahead of the wait for MFMA i + 1
        score8_direct<D, I + 1>(st, q, rd);
    }
}

// Types of one instantiation: PREC 0 bf16 inputs; 1 e4m3 inputs (V widened to
// bf16, bf16 weights); 2 e4m3 inputs and e4m3 weights; 3 bf16 inputs of a
// single launch, whose key ranges may be split over several workgroups.
template <int D, int NIV, int PREC>
struct FwdTypes {
    using In = uint16_t;
    using Shared = Smem<D, NIV>;
    using QReg = bf16x8;
    static constexpr int kQRegs = D / 16;
};
template <int D, int NIV>
struct FwdTypes8 {
    using In = uint8_t;
    using Shared = Smem8w<D, NIV>;
    using QReg = v8i;
    static constexpr int kQRegs = D / 64;
};
template <int D, int NIV>
struct FwdTypes<D, NIV, 1> : FwdTypes8<D, NIV> {};
// bf16 inputs launched alone (no records), key ranges possibly split.
template <int D, int NIV>
struct FwdTypes<D, NIV, 3> : FwdTypes<D, NIV, 0> {};
// The same with a query block's key blocks shared by two groups of four
// wavefronts in one workgroup (PREC 4).
template <int D, int NIV>
struct FwdTypes<D, NIV, 4> : FwdTypes<D, NIV, 0> {};
template <int PREC>
constexpr int kGroups = PREC == 4 ? 2 : 1;

// One group's shared memory: its K/V buffers and staged intervals during the
// key loop, its running state (d/2 accumulators, the reference maximum and
// both sums per lane, as float4 chunks) afterwards.
template <int D, int NIV>
union alignas(16) GroupShared {
    Smem<D, NIV> s;
    float4 state[(D / 8 + 1) * kThreads];
};
template <class S>
__device__ __forceinline__ S& group_smem(S& s) {
    return s;
}
template <int D, int NIV>
__device__ __forceinline__ Smem<D, NIV>& group_smem(GroupShared<D, NIV>& g) {
    return g.s;
}
template <int D, int NIV>
struct FwdTypes<D, NIV, 2> : FwdTypes8<D, NIV> {};

// NIV: ranges per query row (the row attends their union).  col_start and
// col_end are [B][NIV][N]; meta holds NIV records per query block.  F8: Q, K,
// V are e4m3 (c then includes their dequantization scales, and v_scale
// multiplies the output); PREC 2 also rounds the weights to e4m3.
// Two workgroups per CU in bf16; the e4m3 kernels' smaller K/V buffers and
// register sets leave room for three, which the register limit keeps.
template <int D, int NIV, int PREC>
__global__ __launch_bounds__(kThreads * kGroups<PREC>)
__attribute__((amdgpu_waves_per_eu(PREC == 1 || PREC == 2 ? 3 : 2)))
void attn_fwd_kernel(
    const typename FwdTypes<D, NIV, PREC>::In* __restrict__ Q,
    const typename FwdTypes<D, NIV, PREC>::In* __restrict__ K,
    const typename FwdTypes<D, NIV, PREC>::In* __restrict__ V, const int32_t* __restrict__ col_start,
    const int32_t* __restrict__ col_end, const TileMeta* __restrict__ meta, const int32_t* __restrict__ order,
    int H, int N, int n_q, float c, float v_scale, int xcd_heads, int per_head, uint16_t* __restrict__ O,
    float* __restrict__ LSE, int split_arg, float* __restrict__ part, unsigned* __restrict__ counters) {
    using T = FwdTypes<D, NIV, PREC>;
    constexpr bool F8 = PREC == 1 || PREC == 2;   // e4m3 inputs
    constexpr bool W8 = PREC == 2;                // e4m3 weights
    // Only the single-launch instances (PREC 3, 4) split key ranges; in the
    // others split is the constant 1 and its code folds away.
    constexpr int GRP = kGroups<PREC>;
    const int split = PREC >= 3 ? split_arg : 1;
    constexpr float kW8Shift = W8 ? 8.f : 0.f;   // log2 of the weights' scale
    constexpr int kElt = (int)sizeof(typename T::In);   // bytes per Q/K/V element
    // With GRP groups, group g (threads 256 g ..) works as a workgroup of its
    // own on the shared memory smg[g].
    using Shared = std::conditional_t<(GRP > 1), GroupShared<D, NIV>, typename T::Shared>;
    __shared__ Shared smg[GRP];
    const int group = GRP == 1 ? 0 : (int)(threadIdx.x / kThreads);
    typename T::Shared& sm = group_smem(smg[group]);

    const int tid = GRP == 1 ? (int)threadIdx.x : (int)(threadIdx.x % kThreads);
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;      // which 32-lane half of the wavefront
    const int r32 = lane & 31;       // query row of this lane inside the wavefront's 32

    // Work item.  Workgroups are dispatched round-robin over the 8 XCDs, so
    // XCD x receives launch slots x, x+8, ...  With xcd_heads set (H a
    // multiple of 8 and enough query blocks per head to fill an XCD), XCD x
    // runs all query blocks of head x, longest first, then those of head x+8,
    // and so on: the workgroups resident on one XCD stream one head's K/V
    // nearly in lockstep and share it through that XCD's L2.  Otherwise the
    // heads of one query block are adjacent in launch order.
    // With the key ranges split (split > 1: small bf16 problems launched
    // alone), workgroup blockIdx.x takes piece `piece` of the key blocks of
    // work item `item`; the last of an item's pieces to finish combines them.
    const unsigned n_items = split == 1 ? gridDim.x : gridDim.x / (unsigned)split;
    const int piece = split == 1 ? 0 : (int)(blockIdx.x / n_items);
    const unsigned item = blockIdx.x - (unsigned)piece * n_items;
    int h, q_item;
    if (xcd_heads) {
        const int s = item >> 3;
        const int M = n_items / H;              // query blocks per head
        h = (item & 7) + 8 * (s / M);
        q_item = s % M;
    } else {
        h = item % H;
        q_item = item / H;
    }
    // With one interval set per head, head h reads set h: its items are the
    // segment [h L, h L + L) of the preprocessor's records and of the order.
    const int L = n_items / H;                   // query blocks per head (B n_q)
    const int set = per_head ? h : 0;
    const int n_sets = per_head ? H : 1;
    const int bt = order != nullptr ? order[set * L + q_item] : set * L + q_item;
    const int local = bt - set * L;
    const int b = local / n_q;
    const int t = local - b * n_q;
    // The query block's key-block records (only the non-skip range x..y of
    // each range is used here), from the preprocessor; without one (meta ==
    // nullptr, small problems launched alone) they are reduced below from the
    // block's own staged intervals.
    TileMeta tm[NIV];
    if (meta != nullptr) {
#pragma unroll
        for (int k = 0; k < NIV; ++k) tm[k] = meta[(int64_t)bt * NIV + k];
    }

    const int64_t bh = (int64_t)b * H + h;
    const typename T::In* Qbh = Q + bh * N * D;
    const __amdgpu_buffer_rsrc_t krs =
        slice_rsrc(reinterpret_cast<const uint16_t*>(K + bh * N * D), N * D * kElt);
    const __amdgpu_buffer_rsrc_t vrs =
        slice_rsrc(reinterpret_cast<const uint16_t*>(V + bh * N * D), N * D * kElt);
    const int row0 = t * kBr;

    // Stage the block's intervals on chip, clamped to the key range [0, N).
    if (tid < kBr) {
        const int r = row0 + tid;
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            int s = kEmptyStart, w = 0;
            if (r < N) {
                const int64_t at = (((int64_t)b * n_sets + set) * NIV + k) * N + r;
                const int sc = max(col_start[at], 0);
                const int ec = min(col_end[at], N - 1);
                if (sc <= ec) {
                    s = sc;
                    w = ec - sc;
                }
            }
            sm.start[k][tid] = s;
            sm.width[k][tid] = w;
        }
    }

    if constexpr (!F8) {
      if (meta == nullptr) {
        // Every wavefront reduces the smallest start and largest end over all
        // kBr rows of the block (two rows per lane), the preprocessor's rule,
        // before any Q row occupies registers.  (bf16 inputs only: the host
        // never launches the e4m3 kernels without records.)
        __syncthreads();
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            int lo = INT_MAX, hi = INT_MIN;
#pragma unroll
            for (int r = lane; r < kBr; r += 64) {
                const int st = sm.start[k][r];
                if (st != kEmptyStart) {
                    lo = min(lo, st);
                    hi = max(hi, st + sm.width[k][r]);
                }
            }
            lo = wave_min(lo);
            hi = wave_max(hi);
            tm[k] = hi >= lo ? make_int4(lo / kBc, hi / kBc, 0, -1) : make_int4(0, -1, 0, -1);
        }
      }
    }

    // Q rows of this lane as MFMA B operands: Q[row][16 cs + 8 half .. +7]
    // (F8: Q[row][64 cs + 32 half .. +31]).
    const int qrow = row0 + wave * kRowsPerWave + r32;
    typename T::QReg qreg[T::kQRegs];
#pragma unroll
    for (int cs = 0; cs < T::kQRegs; ++cs) {
        if constexpr (F8) {
            if (qrow < N) {
                const uint8_t* src = Qbh + (int64_t)qrow * D + cs * 64 + half * 32;
                const u32x4 lo = *reinterpret_cast<const u32x4*>(src);
                const u32x4 hi = *reinterpret_cast<const u32x4*>(src + 16);
                qreg[cs] = __builtin_bit_cast(v8i, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
            } else {
                qreg[cs] = v8i{};
            }
        } else {
            if (qrow < N)
                qreg[cs] = *reinterpret_cast<const bf16x8*>(Qbh + (int64_t)qrow * D + cs * 16 + half * 8);
            else
                qreg[cs] = bf16x8{};
        }
    }

    // bf16 blocks (loaded straight into LDS): this lane's load offset and its
    // operand read offsets in the segment layout.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int dvoff = F8 ? 0 : direct_lane_offset<D>(lane, wave_u);
    const int k_lane = F8 ? 0 : (r32 % Direct<D>::kSegs) * Direct<D>::kKPitch +
                                    (r32 / Direct<D>::kSegs) * Direct<D>::kRowBytes + 16 * half;
    const int v_lane = F8 ? 0 : (4 * (lane >> 5) + ((lane & 15) >> 2)) * Direct<D>::kVPitch +
                                    32 * ((lane >> 4) & 1) + 8 * (lane & 3);
    // e4m3 inputs: load offset, K read offset, V transposing-read offset
    const int dvoff8 = F8 ? direct8_lane_offset<D>(lane, wave_u) : 0;
    const int k8_lane = F8 ? (r32 % Direct8<D>::kSegs) * Direct8<D>::kKPitch +
                                 (r32 / Direct8<D>::kSegs) * Direct8<D>::kRowBytes + 32 * half
                           : 0;
    const int lp8 = 8 * ((lane & 15) >> 3) + 4 * (lane >> 5) + ((lane & 15) >> 1) % 4;
    const int v8_lane = F8 ? (lp8 % Direct8<D>::kSegs) * Direct8<D>::kVPitch +
                                 (lp8 / Direct8<D>::kSegs) * Direct8<D>::kRowBytes + 16 * ((lane >> 4) & 1) +
                                 8 * (lane & 1)
                           : 0;

    floatx16 oacc[D / 32];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) oacc[nb] = floatx16{};
    float m_run = -INFINITY;   // running row maximum, in log2 units (score * scale * log2 e)
    float l_run = 0.f;         // this lane's share of the running row sum (fp32 weights) -> LSE
    float l16_run = 0.f;       // the same sum over the bf16-rounded weights the PV product uses -> O
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    __syncthreads();
    // Per range: this lane's row interval, and the bounds of the wavefront's
    // rows (the half-waves hold the same rows).
    int my_s[NIV], my_w[NIV];
    int w_min_s[NIV], w_max_e[NIV], w_max_s[NIV], w_min_e[NIV];
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
        my_s[k] = sm.start[k][wave * kRowsPerWave + r32];
        my_w[k] = sm.width[k][wave * kRowsPerWave + r32];
        const bool any = my_s[k] != kEmptyStart;
        w_min_s[k] = wave_min(any ? my_s[k] : INT_MAX);
        w_max_e[k] = wave_max(any ? my_s[k] + my_w[k] : INT_MIN);
        w_max_s[k] = wave_max(any ? my_s[k] : (qrow < N ? INT_MAX : INT_MIN));
        w_min_e[k] = wave_min(any ? my_s[k] + my_w[k] : (qrow < N ? INT_MIN : INT_MAX));
    }

    // Key blocks in increasing order over the union of the ranges' non-skip
    // blocks (one contiguous run for a single range).  A piece of a split
    // item takes the union's blocks [lo, hi) by position, lo = piece * n /
    // pieces; the pieces are the workgroups' (split) times their groups'.
    // Every group of a workgroup takes the same number of steps (a group
    // past its last block idles through the rest), so that all of them meet
    // the same barriers.
    const int pieces = split * GRP;
    int j = union_next<NIV>(tm, -1);
    int left = INT_MAX;                           // blocks this group still computes
    int steps = 0;                                // GRP > 1: steps every group takes
    if (pieces > 1) {
        int n = 0;
        for (int x = j; x != INT_MAX; x = union_next<NIV>(tm, x)) ++n;
        const int my_piece = piece * GRP + group;
        const int lo = my_piece * n / pieces, hi = (my_piece + 1) * n / pieces;
        for (int s = 0; s < lo; ++s) j = union_next<NIV>(tm, j);
        left = hi - lo;
        if (left == 0) j = INT_MAX;
        steps = (n + pieces - 1) / pieces;
    }
    if (GRP > 1 ? steps > 0 : j != INT_MAX) {
        if (GRP == 1 || j != INT_MAX) {
            if constexpr (F8)
                load_block8_direct<D>(sm, 0, krs, vrs, dvoff8, j * kBc, wave_u);
            else
                load_block_direct<D>(sm, 0, krs, vrs, dvoff, j * kBc, wave_u);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();

        for (int buf = 0, it = 0;; buf ^= 1, ++it) {
            const bool active = GRP == 1 || j != INT_MAX;
            const int j_next = active ? union_next<NIV>(tm, j) : INT_MAX;
            const bool has_next = j_next != INT_MAX && (pieces == 1 || --left > 0);
            if (has_next) {
                if constexpr (F8)
                    load_block8_direct<D>(sm, buf ^ 1, krs, vrs, dvoff8, j_next * kBc, wave_u);
                else
                    load_block_direct<D>(sm, buf ^ 1, krs, vrs, dvoff, j_next * kBc, wave_u);
            }

            const int klo = (active ? j : 0) * kBc;
            const int khi = min(klo + kBc, N) - 1;
            // The wavefront skips the block when each range of each of its
            // rows misses it, and computes it without the compare when one
            // range covers it for all of its rows.
            bool wave_skip = true, wave_full = false;
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
                wave_skip &= khi < w_min_s[k] || klo > w_max_e[k];
                wave_full |= klo >= w_max_s[k] && khi <= w_min_e[k];
            }
            wave_skip |= !active;                // a group past its last block
            if (!wave_skip) {
                // ---- S^T = K Q^T: lane holds S[q = r32][key = 32 jb + 8 (v/4) + 4 half + v%4]
                floatx16 st[kBc / 32];
#pragma unroll
                for (int jb = 0; jb < kBc / 32; ++jb) st[jb] = floatx16{};
                if constexpr (F8) {
                    u32x4 rd[2 * (D / 64) * (kBc / 32)];
                    issue_k8_reads<D>(rd, lds_address(&sm.k8[buf][0]) + k8_lane);
                    score8_direct<D>(st, qreg, rd);
                } else {
                    u32x4 ring[kAheadK];
                    const uint32_t kaddr = lds_address(&sm.k[buf][0]) + k_lane;
                    issue_k_reads<D>(ring, kaddr);
                    score_direct<D>(st, qreg, kaddr, ring);
                }

                // ---- interval compare, only where some row of the wavefront
                // does not attend the whole key block (boundary blocks).
                const bool full = (klo + kBc <= N) && wave_full;
                if (!full) {
                    int base[NIV];
#pragma unroll
                    for (int k = 0; k < NIV; ++k) base[k] = klo + 4 * half - my_s[k];
#pragma unroll
                    for (int jb = 0; jb < kBc / 32; ++jb) {
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const int off = jb * 32 + 8 * (v >> 2) + (v & 3);
                            bool ok = false;
#pragma unroll
                            for (int k = 0; k < NIV; ++k) ok |= (uint32_t)(base[k] + off) <= (uint32_t)my_w[k];
                            st[jb][v] = ok ? st[jb][v] : -INFINITY;
                        }
                    }
                }

                // ---- online softmax (exp2 with scale * log2 e folded in)
                float mx = st[0][0];
#pragma unroll
                for (int jb = 0; jb < kBc / 32; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[jb][v]);
                // Lazy rescaling: the reference m_run of a row may lag its true
                // running maximum by up to kSlack (log2 units), so weights reach
                // 2^kSlack at most (fine for bf16 and the fp32 sums), and the
                // accumulator is rescaled only when some row of the wavefront
                // exceeds its reference by more than that -- in practice after the
                // first block of a row, instead of on most blocks.  A rescale then
                // moves every row that grew to its exact maximum.  The e4m3 weights
                // keep the exact maximum (kSlack 0): 2^8 P must stay below 448.
                constexpr float kSlack = W8 ? 0.f : 8.f;
                const float m_blk = halves_max(mx) * c;
                if (__builtin_amdgcn_ballot_w64(m_blk > m_run + kSlack) != 0) {
                    const bool grow = m_blk > m_run;
                    const float m_new = grow ? m_blk : m_run;
                    const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                    l_run *= alpha;
                    l16_run *= alpha;
#pragma unroll
                    for (int nb = 0; nb < D / 32; ++nb) oacc[nb] *= alpha;
                    m_run = m_new;
                }
                // e4m3 weights are formed as 2^8 P: the exponent offset is folded in here
                const float m_use = (m_run == -INFINITY ? 0.f : m_run) - kW8Shift;
                // V^T reads of the PV product's first step, issued once the
                // score product's operand reads are done, so that their
                // latency overlaps the exponentials.
                [[maybe_unused]] v4s vpart[2 * D / 32];
                [[maybe_unused]] uint32_t vaddr = 0;
                if constexpr (!F8) {
                    vaddr = lds_address(&sm.v[buf][0]) + v_lane;
                    issue_v_reads<D, 0>(vpart, vaddr, m_use);
                }
                [[maybe_unused]] v2i v8part[4];
                [[maybe_unused]] uint32_t v8addr = 0;
                if constexpr (F8) {
                    v8addr = lds_address(&sm.v8[buf][0]) + v8_lane;
                    issue_v8_reads<D, 0>(v8part, v8addr, m_use);
                }
                float rs = 0.f;
                if constexpr (F8) {
#pragma unroll
                    for (int jb = 0; jb < kBc / 32; ++jb)
#pragma unroll
                        for (int v = 0; v < 16; ++v) {
                            const float p = __builtin_amdgcn_exp2f(fmaf(st[jb][v], c, -m_use));
                            st[jb][v] = p;
                            rs += p;
                        }
                }

                // ---- O^T += V^T P^T.  O is later divided by the sum of the same
                // bf16-rounded weights, so the rounding of P perturbs the weights
                // of a proper weighted mean instead of biasing its scale.
                float rs16 = 0.f;
                if constexpr (W8) {
                    // the weights (already 2^8 P) as e4m3, bytes e = 16 jb + v; the
                    // normaliser is the sum of the rounded weights, read back
                    uint32_t pw[8];
#pragma unroll
                    for (int w = 0; w < 8; ++w) {
                        const int jb = w >> 2, v0 = 4 * (w & 3);
                        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(st[jb][v0], st[jb][v0 + 1], 0, false);
                        packed = __builtin_amdgcn_cvt_pk_fp8_f32(st[jb][v0 + 2], st[jb][v0 + 3], packed, true);
                        pw[w] = (uint32_t)packed;
                        const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)pw[w], false);
                        const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)pw[w], true);
                        rs16 += (lo[0] + lo[1]) + (hi[0] + hi[1]);
                    }
                    const v8i pb8 = {(int)pw[0], (int)pw[1], (int)pw[2], (int)pw[3],
                                     (int)pw[4], (int)pw[5], (int)pw[6], (int)pw[7]};
                    pv8_direct<D, 0>(pb8, oacc, v8addr, v8part);
                } else if constexpr (F8) {
                    bf16x8 pbs[kBc / 16];
#pragma unroll
                    for (int ks = 0; ks < kBc / 16; ++ks) {
#pragma unroll
                        for (int e = 0; e < 8; ++e) pbs[ks][e] = (__bf16)st[ks >> 1][8 * (ks & 1) + e];
                        rs16 = sum_bf16x8(pbs[ks], ones, rs16);
                    }
                    pv8_bf16_direct<D, 0>(pbs, oacc, v8addr, v8part);
                } else {
                    // A operand lane (i, half h), element e: V^T[column i][key
                    // 16 ks + 8 (e / 4) + 4 h + e % 4], the key order of the P^T
                    // registers: two transposing reads of four keys each.
                    pv_direct<D, 0>(st, oacc, vaddr, c, m_use, rs, rs16, ones, vpart);
                }
                l_run += rs;
                l16_run += rs16;
            }

            if (has_next) __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads have landed
            __syncthreads();
            if (GRP == 1 ? !has_next : it + 1 >= steps) break;
            j = has_next ? j_next : INT_MAX;
        }
    }

    // ---- groups: groups 1.. leave their running state in their own shared
    // memory and finish; group 0 combines it with its own against the largest
    // reference (the combination of the split pieces below, in LDS).
    if constexpr (GRP > 1) {
        constexpr int kAcc = D / 32 * 16;
        constexpr int kChunks = kAcc / 4 + 1;
        if (group > 0) {
            float4* const st = smg[group].state;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    st[(nb * 4 + g) * kThreads + tid] =
                        make_float4(oacc[nb][4 * g], oacc[nb][4 * g + 1], oacc[nb][4 * g + 2], oacc[nb][4 * g + 3]);
            st[(kChunks - 1) * kThreads + tid] = make_float4(m_run, l_run, l16_run, 0.f);
        }
        __syncthreads();
        if (group > 0) return;
        float m = m_run;
        for (int gp = 1; gp < GRP; ++gp) m = fmaxf(m, smg[gp].state[(kChunks - 1) * kThreads + tid].x);
        const float w0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m);
        l_run *= w0;
        l16_run *= w0;
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) oacc[nb] *= w0;
#pragma unroll 1
        for (int gp = 1; gp < GRP; ++gp) {
            const float4 s4 = smg[gp].state[(kChunks - 1) * kThreads + tid];
            const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s4.x - m);
            l_run = fmaf(w, s4.y, l_run);
            l16_run = fmaf(w, s4.z, l16_run);
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const float4 x = smg[gp].state[(nb * 4 + g) * kThreads + tid];
                    oacc[nb][4 * g] = fmaf(w, x.x, oacc[nb][4 * g]);
                    oacc[nb][4 * g + 1] = fmaf(w, x.y, oacc[nb][4 * g + 1]);
                    oacc[nb][4 * g + 2] = fmaf(w, x.z, oacc[nb][4 * g + 2]);
                    oacc[nb][4 * g + 3] = fmaf(w, x.w, oacc[nb][4 * g + 3]);
                }
        }
        m_run = m;
    }

    // ---- split key ranges: every piece stores its running state (the
    // unnormalised accumulators, the reference maximum and both sums, per
    // lane); the last piece of the item to arrive reads them all back and
    // combines them against the largest reference,
    //     O_acc = sum_p 2^(m_p - m) O_acc,p,  l = sum_p 2^(m_p - m) l_p,
    // which is the state one workgroup would have reached over all the
    // blocks (up to the order of the fp32 additions).  The arrival count is
    // reset by that last piece, so it is zero again for the next call.
    if constexpr (!F8) {
        if (split > 1) {
            constexpr int kAcc = D / 32 * 16;                 // accumulator floats per lane
            constexpr int kChunks = kAcc / 4 + 1;             // float4 chunks per lane (last: m, l, l16)
            float4* const mine = reinterpret_cast<float4*>(part) + ((int64_t)item * split + piece) * kChunks * kThreads;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    mine[(nb * 4 + g) * kThreads + tid] =
                        make_float4(oacc[nb][4 * g], oacc[nb][4 * g + 1], oacc[nb][4 * g + 2], oacc[nb][4 * g + 3]);
            mine[(kChunks - 1) * kThreads + tid] = make_float4(m_run, l_run, l16_run, 0.f);
            __threadfence();                                  // the state is visible before the arrival counts
            __syncthreads();
            int* const arrived = &sm.start[0][0];             // the intervals are in registers by now
            if (tid == 0) *arrived = (int)atomicAdd(&counters[item], 1u);
            __syncthreads();
            if (*arrived != split - 1) return;                // another piece finishes the item
            __threadfence();                                  // every piece's state is visible
            if (tid == 0) counters[item] = 0u;
            const float4* const all = reinterpret_cast<const float4*>(part) + (int64_t)item * split * kChunks * kThreads;
            // Two passes: the largest reference, then the weighted sums (the
            // pieces' loads are independent of one another, so they overlap).
            float m = -INFINITY;
            for (int pc = 0; pc < split; ++pc) m = fmaxf(m, all[(pc * kChunks + kChunks - 1) * kThreads + tid].x);
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb) oacc[nb] = floatx16{};
            l_run = 0.f;
            l16_run = 0.f;
            for (int pc = 0; pc < split; ++pc) {
                const float4 st = all[(pc * kChunks + kChunks - 1) * kThreads + tid];
                const float w = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(st.x - m);
                l_run = fmaf(w, st.y, l_run);
                l16_run = fmaf(w, st.z, l16_run);
#pragma unroll
                for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const float4 x = all[(pc * kChunks + nb * 4 + g) * kThreads + tid];
                        oacc[nb][4 * g] = fmaf(w, x.x, oacc[nb][4 * g]);
                        oacc[nb][4 * g + 1] = fmaf(w, x.y, oacc[nb][4 * g + 1]);
                        oacc[nb][4 * g + 2] = fmaf(w, x.z, oacc[nb][4 * g + 2]);
                        oacc[nb][4 * g + 3] = fmaf(w, x.w, oacc[nb][4 * g + 3]);
                    }
            }
            m_run = m;
        }
    }

    // ---- epilogue: O = O_acc / l16 (bf16, nearest even), LSE = ln(sum) in natural log.
    // O goes out through LDS so that every store writes whole rows: each
    // wavefront stages its rows in its own part of the K/V buffers, idle now
    // (after the last block's barrier no wavefront reads them, and no load
    // into them is in flight), then writes 16 contiguous bytes per lane.
    // Where those buffers cannot hold all 128 rows at once (e4m3 inputs), the
    // rows go in two passes of 16 per wavefront; LDS operations of one
    // wavefront take effect in issue order, so a pass may overwrite what the
    // previous one read.
    const float l = halves_sum(l_run);
    const float l16 = halves_sum(l16_run);
    float inv = l16 > 0.f ? 1.f / l16 : 0.f;
    if constexpr (F8) inv *= v_scale;
    constexpr int kOPitch = 2 * D + 16;           // bytes per staged row (16-byte aligned, rows 4 banks apart)
    constexpr int kStageRoom = (int)offsetof(typename T::Shared, start);
    constexpr int kOTile = kWaves * kRowsPerWave * kOPitch;
    constexpr int kOPasses = kOTile <= kStageRoom ? 1 : 2;
    static_assert(kOTile <= kOPasses * kStageRoom, "the K/V buffers hold the staged output");
    constexpr int kPassRows = kRowsPerWave / kOPasses;
    constexpr int kLanesPerRow = 2 * D / 16;      // 16 bytes per lane
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    static_assert(kPassRows % kRowsPerStore == 0, "whole stores per pass");
    uint8_t* const ost = reinterpret_cast<uint8_t*>(&sm) + wave * kPassRows * kOPitch;
    uint8_t* const obh = reinterpret_cast<uint8_t*>(O + bh * N * D);
    // rounded to bf16 up front: half the registers of the accumulators
    bf16x4 o4[D / 32][4];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int q = 0; q < 4; ++q) o4[nb][g][q] = (__bf16)(oacc[nb][4 * g + q] * inv);
#pragma unroll
    for (int pass = 0; pass < kOPasses; ++pass) {
        if (r32 / kPassRows == pass) {
            uint8_t* const orow = ost + (r32 - pass * kPassRows) * kOPitch;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<bf16x4*>(orow + 2 * (nb * 32 + 8 * g + 4 * half)) = o4[nb][g];
        }
#pragma unroll
        for (int i = 0; i < kPassRows / kRowsPerStore; ++i) {
            const int r = i * kRowsPerStore + lane / kLanesPerRow;
            const int cb = 16 * (lane % kLanesPerRow);
            const u32x4 v = *reinterpret_cast<const u32x4*>(ost + r * kOPitch + cb);
            const int grow = row0 + wave * kRowsPerWave + pass * kPassRows + r;
            if (grow < N) *reinterpret_cast<u32x4*>(obh + (int64_t)grow * (2 * D) + cb) = v;
        }
    }
    // (one fused multiply-add, written out: left to the compiler, the
    // contraction differs between instances and so would the last bit)
    if (qrow < N && half == 0) LSE[bh * N + qrow] = l > 0.f ? fmaf(m_run - kW8Shift, kLn2, logf(l)) : -INFINITY;
}

// ---------------------------------------------------------------- small problems
//
// With a few dozen query blocks, the kernel above leaves most CUs idle while
// each workgroup walks its key blocks one after another, one wavefront per
// SIMD, with nothing beside it to hide the latency of each block's chain of
// products and exponentials.  For such problems a workgroup takes one slice
// of 32 query rows of one (b, h), and its kRowWaves wavefronts share the
// slice's key blocks: wavefront w walks the w-th contiguous share of them
// (in increasing order) through its own LDS buffer, with the same block body
// as above.  The wavefronts then leave their running states in their
// buffers and combine them against the largest reference maximum, as the
// wavefront groups above do, each combining its own columns of the output.
// No records and no workspace: every wavefront reduces the slice's key range
// from the intervals it loads itself.
template <int D>
constexpr int kRowWaves = D == 64 ? 8 : 4;

template <int D>
struct alignas(16) RowsWaveBuf {
    alignas(16) uint8_t k[Direct<D>::kKBytes];
    alignas(16) uint8_t v[Direct<D>::kVBytes];
};

// Every segment of one key block, loaded by one wavefront (off: the lane's
// offset for segment 0, direct_lane_offset with wave 0, plus the block's).
template <int D, int SEG = 0>
__device__ __forceinline__ void load_block_wave(RowsWaveBuf<D>& wb, __amdgpu_buffer_rsrc_t krs,
                                                __amdgpu_buffer_rsrc_t vrs, int off) {
    using L = Direct<D>;
    if constexpr (SEG < L::kSegs) {
        const int row_off = off + SEG * L::kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_ptr_t)&wb.k[SEG * L::kKPitch], 16, row_off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_ptr_t)&wb.v[SEG * L::kVPitch], 16, row_off, 0, 0, 0);
        load_block_wave<D, SEG + 1>(wb, krs, vrs, off);
    }
}

template <int D, int NIV>
__global__ __launch_bounds__(64 * kRowWaves<D>)
void attn_fwd_rows_kernel(const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K,
                          const uint16_t* __restrict__ V, const int32_t* __restrict__ col_start,
                          const int32_t* __restrict__ col_end, int H, int N, int n_slices, float c, int per_head,
                          uint16_t* __restrict__ O, float* __restrict__ LSE) {
    constexpr int W = kRowWaves<D>;
    constexpr int kChunks = D / 8 + 1;            // float4 chunks of a lane's state (last: m, l, l16)
    static_assert(sizeof(float4) * kChunks * 64 <= sizeof(RowsWaveBuf<D>), "a state fits its buffer");
    __shared__ RowsWaveBuf<D> wbuf[W];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int half = lane >> 5;
    const int r32 = lane & 31;
    // workgroup (b n_slices + t) H + h: slice t of batch element b, head h
    const int h = blockIdx.x % H;
    const int bt = blockIdx.x / H;
    const int b = bt / n_slices;
    const int t = bt - b * n_slices;
    const int set = per_head ? h : 0;
    const int n_sets = per_head ? H : 1;
    const int64_t bh = (int64_t)b * H + h;
    const int qrow = t * kRowsPerWave + r32;

    // Q rows of this lane as MFMA B operands: Q[row][16 cs + 8 half .. +7]
    bf16x8 qreg[D / 16];
#pragma unroll
    for (int cs = 0; cs < D / 16; ++cs)
        qreg[cs] = qrow < N ? *reinterpret_cast<const bf16x8*>(Q + (bh * N + qrow) * D + cs * 16 + half * 8)
                            : bf16x8{};

    // This lane's row intervals, clamped to [0, N), and the slice's bounds
    // per range (both halves hold the same rows).
    int my_s[NIV], my_w[NIV];
    int w_min_s[NIV], w_max_e[NIV], w_max_s[NIV], w_min_e[NIV];
    TileMeta tm[NIV];
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
        int s = kEmptyStart, w = 0;
        if (qrow < N) {
            const int64_t at = (((int64_t)b * n_sets + set) * NIV + k) * N + qrow;
            const int sc = max(col_start[at], 0);
            const int ec = min(col_end[at], N - 1);
            if (sc <= ec) {
                s = sc;
                w = ec - sc;
            }
        }
        my_s[k] = s;
        my_w[k] = w;
        const bool any = s != kEmptyStart;
        w_min_s[k] = wave_min(any ? s : INT_MAX);
        w_max_e[k] = wave_max(any ? s + w : INT_MIN);
        w_max_s[k] = wave_max(any ? s : (qrow < N ? INT_MAX : INT_MIN));
        w_min_e[k] = wave_min(any ? s + w : (qrow < N ? INT_MIN : INT_MAX));
        tm[k] = w_max_e[k] >= w_min_s[k] ? make_int4(w_min_s[k] / kBc, w_max_e[k] / kBc, 0, -1)
                                         : make_int4(0, -1, 0, -1);
    }

    // This wavefront's share of the union of the non-skip key blocks.
    const int n = union_blocks<NIV>(tm);
    const int lo = wave * n / W;
    int left = (wave + 1) * n / W - lo;
    int j = union_next<NIV>(tm, -1);
    for (int s = 0; s < lo; ++s) j = union_next<NIV>(tm, j);

    RowsWaveBuf<D>& wb = wbuf[wave];
    const __amdgpu_buffer_rsrc_t krs = slice_rsrc(K + bh * N * D, N * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(V + bh * N * D, N * D * 2);
    const int loff = direct_lane_offset<D>(lane, 0);
    if (left > 0) load_block_wave<D>(wb, krs, vrs, loff + j * kBc * Direct<D>::kRowBytes);

    const int k_lane = (r32 % Direct<D>::kSegs) * Direct<D>::kKPitch + (r32 / Direct<D>::kSegs) * Direct<D>::kRowBytes +
                       16 * half;
    const int v_lane = (4 * (lane >> 5) + ((lane & 15) >> 2)) * Direct<D>::kVPitch + 32 * ((lane >> 4) & 1) +
                       8 * (lane & 3);
    floatx16 oacc[D / 32];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) oacc[nb] = floatx16{};
    float m_run = -INFINITY;   // running row maximum, in log2 units
    float l_run = 0.f;         // this lane's share of the row sum of the fp32 weights -> LSE
    float l16_run = 0.f;       // the same over the bf16-rounded weights -> O
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    for (; left > 0; --left) {
        __builtin_amdgcn_s_waitcnt(0);             // block j is in this wavefront's buffer
        asm volatile("" ::: "memory");
        const int klo = j * kBc;
        const int khi = min(klo + kBc, N) - 1;
        bool wave_skip = true, wave_full = false;
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            wave_skip &= khi < w_min_s[k] || klo > w_max_e[k];
            wave_full |= klo >= w_max_s[k] && khi <= w_min_e[k];
        }
        if (!wave_skip) {
            floatx16 st[kBc / 32];
#pragma unroll
            for (int jb = 0; jb < kBc / 32; ++jb) st[jb] = floatx16{};
            u32x4 ring[kAheadK];
            const uint32_t kaddr = lds_address(&wb.k[0]) + k_lane;
            issue_k_reads<D>(ring, kaddr);
            score_direct<D>(st, qreg, kaddr, ring);
            if (!((klo + kBc <= N) && wave_full)) {
                int base[NIV];
#pragma unroll
                for (int k = 0; k < NIV; ++k) base[k] = klo + 4 * half - my_s[k];
#pragma unroll
                for (int jb = 0; jb < kBc / 32; ++jb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        const int off = jb * 32 + 8 * (v >> 2) + (v & 3);
                        bool ok = false;
#pragma unroll
                        for (int k = 0; k < NIV; ++k) ok |= (uint32_t)(base[k] + off) <= (uint32_t)my_w[k];
                        st[jb][v] = ok ? st[jb][v] : -INFINITY;
                    }
            }
            float mx = st[0][0];
#pragma unroll
            for (int jb = 0; jb < kBc / 32; ++jb)
#pragma unroll
                for (int v = 0; v < 16; ++v) mx = fmaxf(mx, st[jb][v]);
            // lazy rescaling, as above: the reference may trail the running
            // maximum by up to 8 in log2 units
            const float m_blk = halves_max(mx) * c;
            if (__builtin_amdgcn_ballot_w64(m_blk > m_run + 8.f) != 0) {
                const bool grow = m_blk > m_run;
                const float m_new = grow ? m_blk : m_run;
                const float alpha = grow ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;
                l_run *= alpha;
                l16_run *= alpha;
#pragma unroll
                for (int nb = 0; nb < D / 32; ++nb) oacc[nb] *= alpha;
                m_run = m_new;
            }
            const float m_use = m_run == -INFINITY ? 0.f : m_run;
            v4s vpart[2 * D / 32];
            const uint32_t vaddr = lds_address(&wb.v[0]) + v_lane;
            issue_v_reads<D, 0>(vpart, vaddr, m_use);
            float rs = 0.f, rs16 = 0.f;
            pv_direct<D, 0>(st, oacc, vaddr, c, m_use, rs, rs16, ones, vpart);
            l_run += rs;
            l16_run += rs16;
        }
        j = union_next<NIV>(tm, j);
        if (left > 1) {
            // every read of the buffer has completed (the products waited for them)
            asm volatile("" ::: "memory");
            load_block_wave<D>(wb, krs, vrs, loff + j * kBc * Direct<D>::kRowBytes);
        }
    }

    // Every wavefront's state into its own buffer (no load into it is in flight).
    float4* const mine = reinterpret_cast<float4*>(&wb);
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            mine[(nb * 4 + g) * 64 + lane] =
                make_float4(oacc[nb][4 * g], oacc[nb][4 * g + 1], oacc[nb][4 * g + 2], oacc[nb][4 * g + 3]);
    mine[(kChunks - 1) * 64 + lane] = make_float4(m_run, l_run, l16_run, 0.f);
    __syncthreads();

    // Combination against the largest reference: O_acc = sum_w 2^(m_w - m) O_acc,w
    // and the same for both sums, in wavefront order.
    float m = -INFINITY;
#pragma unroll
    for (int w = 0; w < W; ++w)
        m = fmaxf(m, reinterpret_cast<const float4*>(&wbuf[w])[(kChunks - 1) * 64 + lane].x);
    float wgt[W];
    float l = 0.f, l16 = 0.f;
#pragma unroll
    for (int w = 0; w < W; ++w) {
        const float4 s4 = reinterpret_cast<const float4*>(&wbuf[w])[(kChunks - 1) * 64 + lane];
        wgt[w] = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s4.x - m);
        l = fmaf(wgt[w], s4.y, l);
        l16 = fmaf(wgt[w], s4.z, l16);
    }
    l = halves_sum(l);
    l16 = halves_sum(l16);
    const float inv = l16 > 0.f ? 1.f / l16 : 0.f;
    // Wavefront `wave` writes chunks wave, wave + W, ...: chunk nb 4 + g holds
    // columns 32 nb + 8 g + 4 half .. +3 of row qrow (the MFMA result layout).
    uint16_t* const orow = O + (bh * N + qrow) * D;
#pragma unroll
    for (int ch = wave; ch < D / 8; ch += W) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float4 x = reinterpret_cast<const float4*>(&wbuf[w])[ch * 64 + lane];
            acc.x = fmaf(wgt[w], x.x, acc.x);
            acc.y = fmaf(wgt[w], x.y, acc.y);
            acc.z = fmaf(wgt[w], x.z, acc.z);
            acc.w = fmaf(wgt[w], x.w, acc.w);
        }
        const bf16x4 o4 = {(__bf16)(acc.x * inv), (__bf16)(acc.y * inv), (__bf16)(acc.z * inv),
                           (__bf16)(acc.w * inv)};
        const int col = 32 * (ch / 4) + 8 * (ch % 4) + 4 * half;
        if (qrow < N) *reinterpret_cast<bf16x4*>(orow + col) = o4;
    }
    if (wave == 0 && qrow < N && half == 0) LSE[bh * N + qrow] = l > 0.f ? fmaf(m, kLn2, logf(l)) : -INFINITY;
}

}  // namespace

hipError_t launch_attention(const void* q, const void* k, const void* v, const int32_t* col_start,
                            const int32_t* col_end, int n_iv, const TileMeta* meta, const int32_t* order,
                            int64_t B, int64_t H, int64_t N, int64_t d, float scale, void* out,
                            float* lse, hipStream_t stream, hipEvent_t start, hipEvent_t stop,
                            const float* fp8_scales, int n_sets, bool fp8_weights, int split, float* part,
                            unsigned* counters, int groups) {
    const int64_t n_q = (N + kBr - 1) / kBr;
    const bool f8 = fp8_scales != nullptr;
    // Split key ranges only for bf16 launches without records.
    if (split < 1 || (split & (split - 1)) != 0 ||
        (split > 1 && (f8 || meta != nullptr || part == nullptr || counters == nullptr)) ||
        (groups != 1 && groups != 2) || (groups > 1 && (f8 || meta != nullptr)))
        return hipErrorInvalidValue;
    const int64_t grid = B * H * n_q * split;
    const float c = (f8 ? scale * fp8_scales[0] * fp8_scales[1] : scale) * kLog2e;
    const float v_scale = f8 ? fp8_scales[2] : 1.f;
    auto* Op = static_cast<uint16_t*>(out);
    // XCD-local head order needs whole heads per XCD and at least one XCD's
    // worth of resident workgroups (32 CUs x 2) per head.
    const int xcd_heads = (H % 8 == 0 && B * n_q >= 128) ? 1 : 0;
    return dispatch_ranges(n_iv, [&](auto niv) {
        constexpr int NIV = decltype(niv)::value;
        // With an event pair, the dispatch packet itself stamps the kernel's
        // start and end, so the pair measures the kernel alone.
        if (f8) {
            const auto* Qp = static_cast<const uint8_t*>(q);
            const auto* Kp = static_cast<const uint8_t*>(k);
            const auto* Vp = static_cast<const uint8_t*>(v);
            auto kernel = fp8_weights ? (d == 128 ? attn_fwd_kernel<128, NIV, 2> : attn_fwd_kernel<64, NIV, 2>)
                                      : (d == 128 ? attn_fwd_kernel<128, NIV, 1> : attn_fwd_kernel<64, NIV, 1>);
            hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, start, stop, 0, Qp, Kp,
                                  Vp, col_start, col_end, meta, order, (int)H, (int)N, (int)n_q, c, v_scale,
                                  xcd_heads, n_sets > 1 ? 1 : 0, Op, lse, 1, nullptr, nullptr);
        } else {
            const auto* Qp = static_cast<const uint16_t*>(q);
            const auto* Kp = static_cast<const uint16_t*>(k);
            const auto* Vp = static_cast<const uint16_t*>(v);
            auto kernel = meta != nullptr ? (d == 128 ? attn_fwd_kernel<128, NIV, 0> : attn_fwd_kernel<64, NIV, 0>)
                          : groups == 2   ? (d == 128 ? attn_fwd_kernel<128, NIV, 4> : attn_fwd_kernel<64, NIV, 4>)
                                          : (d == 128 ? attn_fwd_kernel<128, NIV, 3> : attn_fwd_kernel<64, NIV, 3>);
            hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads * groups), 0, stream, start, stop, 0,
                                  Qp, Kp,
                                  Vp, col_start, col_end, meta, order, (int)H, (int)N, (int)n_q, c, v_scale,
                                  xcd_heads, n_sets > 1 ? 1 : 0, Op, lse, split, part, counters);
        }
        return hipGetLastError();
    });
}

hipError_t launch_attention_rows(const void* q, const void* k, const void* v, const int32_t* col_start,
                                 const int32_t* col_end, int n_iv, int64_t B, int64_t H, int64_t N, int64_t d,
                                 float scale, void* out, float* lse, hipStream_t stream, hipEvent_t start,
                                 hipEvent_t stop, int n_sets) {
    if (d != 64 && d != 128) return hipErrorInvalidValue;
    const int64_t n_slices = (N + kRowsPerWave - 1) / kRowsPerWave;
    const int64_t grid = B * H * n_slices;
    const float c = scale * kLog2e;
    const auto* Qp = static_cast<const uint16_t*>(q);
    const auto* Kp = static_cast<const uint16_t*>(k);
    const auto* Vp = static_cast<const uint16_t*>(v);
    auto* Op = static_cast<uint16_t*>(out);
    return dispatch_ranges(n_iv, [&](auto niv) {
        constexpr int NIV = decltype(niv)::value;
        auto kernel = d == 128 ? attn_fwd_rows_kernel<128, NIV> : attn_fwd_rows_kernel<64, NIV>;
        const int threads = 64 * (d == 128 ? kRowWaves<128> : kRowWaves<64>);
        hipExtLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(threads), 0, stream, start, stop, 0, Qp, Kp, Vp,
                              col_start, col_end, (int)H, (int)N, (int)n_slices, c, n_sets > 1 ? 1 : 0, Op, lse);
        return hipGetLastError();
    });
}

}  // namespace fm
