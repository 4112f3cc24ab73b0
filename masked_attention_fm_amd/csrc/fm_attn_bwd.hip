// Gradients of masked attention for gfx950 (MI355X): dQ, dK, dV from the
// forward's LSE.
//
// The pages give the forward pass only; they use the method in training
// (FlashMask abstract), which needs these gradients.  With P the masked
// softmax recomputed from the saved LSE (P = exp(scale q.k - LSE), 0 outside
// the row's ranges), D = rowsum(dO * O) and dS = P (dO V^T - D):
//   dV = P^T dO,   dK = scale dS^T Q,   dQ = scale dS K.
// The tile skipping of the forward carries over unchanged (FlashMask article
// §2.2, §4.1 items 2-3): a pair of blocks skipped there has P = 0 here and
// contributes nothing, so it is never loaded; a FULL pair needs no compare.
//
// Two kernels, no atomics, deterministic:
//   * bwd_dkdv_kernel: one workgroup per (b, h, block of kBwdKeys = 128 keys),
//     four pairs of wavefronts, a pair per 32 keys, walking the query chunks
//     (kBwdRows = 64 rows) whose non-skip ranges hold the key block.  One
//     wavefront of a pair holds the keys' K rows (MFMA B operands) and dV^T:
//     S = Q K^T, the masked P (to LDS), dV^T += dO^T P.  The other holds V and
//     dK^T, one chunk behind: dS = P (dP - D) with P from LDS, dK^T += Q^T dS,
//     and dP = dO V^T of the current chunk.  Q and dO are read from LDS, row
//     by row or with transposing reads; they are loaded straight into LDS.
//     Two wavefronts per SIMD.  A lane ends up holding one key's dK or dV row.
//   * bwd_dq_kernel: one workgroup per (b, h, query block of kBr = 128 rows),
//     the forward's structure: S^T = K Q^T and dP^T = V dO^T with Q and dO in
//     registers, then dQ^T += K^T dS^T, walking the union of the non-skip key
//     blocks.  K and V are loaded straight into LDS; K^T is read with
//     transposing LDS reads.  Two workgroups per CU.  A lane ends up holding
//     one query's dQ row.
// Both buffer their operands through LDS with one barrier per step.  A key
// block attended by far more query chunks than the others is split into
// pieces over equal shares of its chunks (bwd_split_kernel); later pieces
// write fp32 partial sums that bwd_reduce_kernel adds in piece order.

#include <hip/hip_runtime.h>
#include <type_traits>
#include <math.h>

#include "fm_internal.h"
#include "fm_mfma.h"

namespace fm {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;

static_assert(kBwdKeys == 32 * kWaves, "one 32-key MFMA column block per wavefront");
static_assert(kBr == 32 * kWaves, "one 32-row MFMA column block per wavefront");
static_assert(kBwdRows % 16 == 0 && kBc % 16 == 0, "chunks are whole MFMA contraction steps");

// ---------------------------------------------------------------- D = rowsum(dO * O)

template <int D>
__global__ __launch_bounds__(256) void bwd_rowdot_kernel(const uint16_t* __restrict__ O,
                                                         const uint16_t* __restrict__ dO, int64_t rows,
                                                         float* __restrict__ dd) {
    constexpr int kLanes = D / 8;              // lanes per row, 8 columns each
    const int64_t row = ((int64_t)blockIdx.x * 256 + threadIdx.x) / kLanes;
    const int c8 = threadIdx.x % kLanes;
    float acc = 0.f;
    if (row < rows) {
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(O + row * D + c8 * 8);
        const bf16x8 g = *reinterpret_cast<const bf16x8*>(dO + row * D + c8 * 8);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    }
#pragma unroll
    for (int off = kLanes / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
    if (row < rows && c8 == 0) dd[row] = acc;
}

// ---------------------------------------------------------------- query chunks per key block

// One wavefront per key-block item (set*B + b)*n_kb + J: lanes scan the query
// chunks t = lane, lane + 64, ... of the same set and batch element, whose
// records are rows (set*B + b)*n_qc + t.
template <int NIV>
__global__ __launch_bounds__(256) void kv_ranges_kernel(const TileMeta* __restrict__ meta_c, int n_qc, int n_kb,
                                                        int64_t items, int4* __restrict__ kvr,
                                                        int32_t* __restrict__ work) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (item >= items) return;                 // whole wavefront leaves together
    const int64_t sb = item / n_kb;            // set * B + b
    const int J = (int)(item - sb * n_kb);
    int lo = INT_MAX, hi = INT_MIN, count = 0;
    for (int t = lane; t < n_qc; t += 64) {
        bool live = false;
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            const TileMeta m = meta_c[(sb * n_qc + t) * NIV + k];
            live |= m.x <= J && J <= m.y;
        }
        if (live) {
            lo = min(lo, t);
            hi = max(hi, t);
            ++count;
        }
    }
    lo = wave_min(lo);
    hi = wave_max(hi);
    count = wave_sum(count);
    if (lane == 0) {
        kvr[item] = make_int4(count > 0 ? lo : 0, count > 0 ? hi : -1, count, 0);
        work[item] = count;
    }
}

// ---------------------------------------------------------------- key-block pieces

constexpr int kSplitThreads = 1024;

// Sum over the workgroup; every thread calls it and gets the total.
__device__ __forceinline__ int split_block_sum(int v, int* red) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < kSplitThreads / 64; ++i) t += red[i];
    __syncthreads();
    return t;
}

// One workgroup.  Piece size S: at least min_chunks, at least twice the mean
// live-chunk count of the non-empty blocks, doubled until the extra pieces fit
// kBwdExtraPieces.  A block with c > S live chunks becomes P = ceil(c / S)
// pieces over equal shares of its chunk-index range.  Which extra entries and
// partial slots a block receives depends on arrival order, but not the
// numbers: each block's partial sums are added in piece order.
__global__ __launch_bounds__(kSplitThreads) void bwd_split_kernel(const int4* __restrict__ kvr, int items,
                                                                  int n_sets, int min_chunks,
                                                                  int4* __restrict__ pieces,
                                                                  int32_t* __restrict__ pslot,
                                                                  int32_t* __restrict__ pwork,
                                                                  int4* __restrict__ splits) {
    __shared__ int red[kSplitThreads / 64];
    __shared__ int n_extra, n_split;
    const int tid = threadIdx.x;
    if (n_sets != 1) {                          // several interval sets: one piece per block
        for (int e = tid; e < items * n_sets; e += kSplitThreads) {
            const int4 r = kvr[e];
            pieces[e] = make_int4(e, r.x, r.y, 1);
            pslot[e] = -1;
            pwork[e] = r.z;
        }
        if (tid == 0) splits[0] = make_int4(0, 0, 0, 0);
        return;
    }
    int tot = 0, nz = 0;
    for (int j = tid; j < items; j += kSplitThreads) {
        const int c = kvr[j].z;
        tot += c;
        nz += c > 0;
    }
    tot = split_block_sum(tot, red);
    nz = split_block_sum(nz, red);
    int S = max(min_chunks, 1);
    if (nz > 0) S = max(S, (2 * tot + nz - 1) / nz);
    for (;;) {                                  // uniform: every thread sees the same sums
        int extra = 0;
        for (int j = tid; j < items; j += kSplitThreads) {
            const int c = kvr[j].z;
            extra += c > S ? (c + S - 1) / S - 1 : 0;
        }
        extra = split_block_sum(extra, red);
        if (extra <= kBwdExtraPieces) break;
        S *= 2;
    }
    if (tid == 0) {
        n_extra = 0;
        n_split = 0;
    }
    __syncthreads();
    for (int j = tid; j < items; j += kSplitThreads) {
        const int4 r = kvr[j];
        const int c = r.z;
        const int P = c > S ? (c + S - 1) / S : 1;
        int base = 0;
        if (P > 1) {
            base = atomicAdd(&n_extra, P - 1);
            splits[1 + atomicAdd(&n_split, 1)] = make_int4(j, P, base, 0);
        }
        const int len = r.y - r.x + 1;          // 0 for a block no chunk attends
        const int w = (c + P - 1) / P;
        for (int p = 0; p < P; ++p) {
            const int lo = r.x + (int)((int64_t)len * p / P);
            const int hi = r.x + (int)((int64_t)len * (p + 1) / P) - 1;
            const int e = p == 0 ? j : items + base + p - 1;
            pieces[e] = make_int4(j, lo, hi, (p << 16) | P);
            pslot[e] = p == 0 ? -1 : base + p - 1;
            pwork[e] = w;
        }
    }
    __syncthreads();
    for (int e = n_extra + tid; e < kBwdExtraPieces; e += kSplitThreads) {
        pieces[items + e] = make_int4(-1, 0, -1, 0);
        pslot[items + e] = -1;
        pwork[items + e] = -1;
    }
    if (tid == 0) splits[0] = make_int4(n_split, 0, 0, 0);
}

// dK, dV of each split block (one interval set) += its pieces 1..P-1, in order.
template <int D>
__global__ __launch_bounds__(256) void bwd_reduce_kernel(const int4* __restrict__ splits,
                                                         const float* __restrict__ part, int H, int N, int n_kb,
                                                         float* __restrict__ dK, float* __restrict__ dV) {
    const int pairs = splits[0].x * H;
    for (int x = blockIdx.x; x < pairs; x += gridDim.x) {
        const int4 sp = splits[1 + x / H];     // {item, P, first slot}
        const int h = x % H;
        const int b = sp.x / n_kb;
        const int k0 = (sp.x - b * n_kb) * kBwdKeys;
        const int64_t bh = (int64_t)b * H + h;
        const int nk = min(kBwdKeys, N - k0);
        for (int i = threadIdx.x; i < nk * (D / 4); i += 256) {
            const int kl = i / (D / 4);
            const int c4 = i % (D / 4);
            float4* dk = reinterpret_cast<float4*>(dK + (bh * N + k0 + kl) * D) + c4;
            float4* dv = reinterpret_cast<float4*>(dV + (bh * N + k0 + kl) * D) + c4;
            float4 ak = *dk, av = *dv;
            for (int p = 1; p < sp.y; ++p) {
                const float* pb = part + ((int64_t)(sp.z + p - 1) * H + h) * (kBwdKeys * D * 2);
                const float4 pk = reinterpret_cast<const float4*>(pb + kl * D)[c4];
                const float4 pv = reinterpret_cast<const float4*>(pb + kBwdKeys * D + kl * D)[c4];
                ak.x += pk.x;
                ak.y += pk.y;
                ak.z += pk.z;
                ak.w += pk.w;
                av.x += pv.x;
                av.y += pv.y;
                av.z += pv.z;
                av.w += pv.w;
            }
            *dk = ak;
            *dv = av;
        }
    }
}

// Launch slot -> (head, work item): the forward's XCD-local head order.
__device__ __forceinline__ void slot_to_item(int xcd_heads, int H, int& h, int& item) {
    if (xcd_heads) {
        const int s = blockIdx.x >> 3;
        const int M = gridDim.x / H;
        h = (blockIdx.x & 7) + 8 * (s / M);
        item = s % M;
    } else {
        h = blockIdx.x % H;
        item = blockIdx.x / H;
    }
}

// Staged interval of one row of one range, clamped to [0, N): start, width.
__device__ __forceinline__ int2 clamp_interval(int s_raw, int e_raw, int N) {
    const int sc = max(s_raw, 0);
    const int ec = min(e_raw, N - 1);
    return sc <= ec ? make_int2(sc, ec - sc) : make_int2(kEmptyStart, 0);
}

// Bounds of one wavefront's rows for one range (rows past N are neutral; a
// row with no key in the range rules out FULL): {min_s, max_e, max_s, min_e}.
__device__ __forceinline__ int4 wave_row_bounds(int s, int w, bool in_seq) {
    const bool any = s != kEmptyStart;
    return make_int4(wave_min(any ? s : INT_MAX), wave_max(any ? s + w : INT_MIN),
                     wave_max(any ? s : (in_seq ? INT_MAX : INT_MIN)),
                     wave_min(any ? s + w : (in_seq ? INT_MIN : INT_MAX)));
}

// Blocks of 64 rows (keys for dQ, query rows for dK/dV) loaded straight from
// global memory into LDS (buffer loads with an LDS destination: one
// instruction writes lane l's 16 bytes to M0 + 16 l, a 1 KB segment per
// wavefront).  A segment holds kSegKeys rows (4 at d = 128, 8 at d = 64);
// segments are padded to 1024 + 16 bytes.  Rows past N read as zero (the
// buffer range check).
//   * A block read row-major only (V in dP^T = V dO^T) keeps row rho in
//     segment rho % kSegs, slot rho / kSegs, so the eight consecutive rows of a
//     ds_read_b128 phase land 16 bytes apart modulo 128.
//   * A block read row-major and transposed (K for dQ; Q and dO for dK/dV;
//     ds_read_b64_tr_b16: within each 16-lane group, lane i receives element
//     i % 4 of the 8-byte pieces addressed by lanes 4 e + i / 4) has its
//     segment index swizzled at d = 128, rho % 16 = 4 a + b -> segment 4 b + a,
//     so that both patterns are free of bank conflicts: sixteen consecutive
//     rows still occupy sixteen segments, and the four consecutive rows of a
//     transposing read sit four segments (64 bytes modulo 256) apart, the two
//     column halves of a 32-lane pass 32 bytes apart.
template <int D>
struct SegLayout {
    static constexpr int kRowBytes = 2 * D;
    static constexpr int kSegKeys = 1024 / kRowBytes;
    static constexpr int kSegs = kBc / kSegKeys;
    static constexpr int kPitch = 1024 + 16;
    static constexpr int kBytes = kSegs * kPitch;
    static constexpr int kSegsPerWave = kSegs / kWaves;
    static_assert(kSegKeys * kSegs == kBc && kSegsPerWave * kWaves == kSegs, "segments split evenly");
};

// segment of a swizzled block holding row rho (x = rho % kSegs)
template <int D>
__device__ __forceinline__ int k_segment(int x) {
    if constexpr (D == 128)
        return 4 * (x & 3) + (x >> 2);
    else
        return x;
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint32_t lds_address(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((lds_ptr_t)p));
}

// This lane's byte offset, inside a 64-row block, of its 16 bytes in the
// first segment its wavefront fills.
template <int D, bool SWZ>
__device__ __forceinline__ int seg_lane_offset(int lane, int wave_u) {
    using L = SegLayout<D>;
    const int slot = lane / (D / 8), chunk = lane % (D / 8);
    const int first = (SWZ && D == 128) ? wave_u : wave_u * L::kSegsPerWave;
    return (first + L::kSegs * slot) * L::kRowBytes + 16 * chunk;
}

// This wavefront's segments of the 64-row block starting at row0 into dst
// (the segment of index wave_u kSegsPerWave + U per instruction; the row is
// selected through the lane offset, since an instruction offset would move
// the LDS destination as well).
template <int D, bool SWZ, int U = 0, typename Ptr>
__device__ __forceinline__ void dma_rows(Ptr dst, __amdgpu_buffer_rsrc_t rs, int lane_off, int row0, int wave_u) {
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS address-space cast exists in the device pass only
    using L = SegLayout<D>;
    if constexpr (U < L::kSegsPerWave) {
        const int seg = wave_u * L::kSegsPerWave + U;
        constexpr int kUStep = (SWZ && D == 128) ? 4 * L::kRowBytes : L::kRowBytes;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)(dst + seg * L::kPitch), 16,
                                                 row0 * L::kRowBytes + lane_off + U * kUStep, 0, 0, 0);
        dma_rows<D, SWZ, U + 1, Ptr>(dst, rs, lane_off, row0, wave_u);
    }
#endif
}

// ---- transposing K reads for the dQ product, issued through inline assembly
// (the builtin would make the compiler wait for the next block's in-flight
// loads before each read).  LDS operations complete in issue order, so
// lgkmcnt(n) after n younger reads guarantees the older ones; each wait
// passes the registers through itself so nothing can use them earlier.
template <int OFF>
__device__ __forceinline__ v4s lds_read_tr16(uint32_t addr) {
    v4s r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
    return r;
}

// Step KS (16 keys): part[2 nb + r] holds, for lane (column i, half h), keys
// 16 KS + 8 r + 4 h + 0..3 of column 32 nb + i.
template <int D, int KS, int I = 0>
__device__ __forceinline__ void issue_kt_reads(v4s (&part)[2 * D / 32], uint32_t addr) {
    using L = SegLayout<D>;
    if constexpr (I < 2 * D / 32) {
        constexpr int nb = I / 2, r = I % 2;
        constexpr int off = D == 128 ? 2 * r * L::kPitch + KS * L::kRowBytes + nb * 64
                                     : (2 * KS + r) * L::kRowBytes + nb * 64;
        static_assert(off >= 0 && off < 65536, "ds offset field");
        part[I] = lds_read_tr16<off>(addr);
        issue_kt_reads<D, KS, I + 1>(part, addr);
    }
}

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

// dQ^T += K^T dS^T over steps KS.. of one key block (cur: step KS's reads).
template <int D, int KS>
__device__ __forceinline__ void dq_product(const floatx16 (&dst)[kBc / 32], floatx16 (&dqacc)[D / 32],
                                           uint32_t addr, v4s (&cur)[2 * D / 32]) {
    constexpr int NP = 2 * D / 32;
    if constexpr (KS < kBc / 16) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[e] = (__bf16)dst[KS >> 1][8 * (KS & 1) + e];
        v4s next[NP];
        if constexpr (KS + 1 < kBc / 16) {
            issue_kt_reads<D, KS + 1>(next, addr);
            wait_lds_tied<NP>(cur);
        } else {
            wait_lds_tied<0>(cur);
        }
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(cur[2 * nb], cur[2 * nb + 1], 0, 1, 2, 3, 4, 5, 6, 7));
            dqacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, sb, dqacc[nb], 0, 0, 0);
        }
        dq_product<D, KS + 1>(dst, dqacc, addr, next);
    }
}

// Row-major operand reads (ds_read_b128) are issued as inline assembly and
// run kAheadS ahead of their MFMAs through a ring of registers (left to
// itself the compiler hoists all of them, and the registers they hold push
// the accumulators out of the vector register file).
constexpr int kAheadS = 7;
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
// S^T = K Q^T and dP^T = V dO^T of the dQ kernel for one key block: read r
// = 4 cs + 2 jb + {0: K, 1: V} holds head-dimension chunk cs of key half jb
// and feeds MFMA r; issued kAheadS ahead like the dK/dV kernel's reads.
template <int D, int R>
__device__ __forceinline__ u32x4 dq_sdp_read(uint32_t kaddr, uint32_t vaddr) {
    using SL = SegLayout<D>;
    constexpr int off = ((R / 2) % (kBc / 32)) * (32 / SL::kSegs) * SL::kRowBytes + (R / (kBc / 16)) * 32;
    return lds_read_b128<off>(R % 2 == 0 ? kaddr : vaddr);
}
template <int D, int I = 0>
__device__ __forceinline__ void dq_sdp_issue(u32x4 (&ring)[kAheadS], uint32_t kaddr, uint32_t vaddr) {
    if constexpr (I < kAheadS) {
        ring[I] = dq_sdp_read<D, I>(kaddr, vaddr);
        dq_sdp_issue<D, I + 1>(ring, kaddr, vaddr);
    }
}
template <int D, int I = 0>
__device__ __forceinline__ void dq_sdp_products(floatx16 (&st)[kBc / 32], floatx16 (&dpt)[kBc / 32],
                                                const bf16x8 (&qreg)[D / 16], const bf16x8 (&greg)[D / 16],
                                                uint32_t kaddr, uint32_t vaddr, u32x4 (&ring)[kAheadS]) {
    constexpr int kN = 2 * (D / 16) * (kBc / 32);
    static_assert(kN > kAheadS, "more MFMAs than reads in flight");
    if constexpr (I < kN) {
        constexpr int cs = I / (kBc / 16), jb = (I / 2) % (kBc / 32);
        constexpr int issued = I + kAheadS < kN ? I + kAheadS : kN;
        wait_lds_one<issued - (I + 1)>(ring[I % kAheadS]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, ring[I % kAheadS]);
        if constexpr (I % 2 == 0)
            st[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[cs], st[jb], 0, 0, 0);
        else
            dpt[jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, greg[cs], dpt[jb], 0, 0, 0);
        if constexpr (I + kAheadS < kN) ring[I % kAheadS] = dq_sdp_read<D, I + kAheadS>(kaddr, vaddr);
        dq_sdp_products<D, I + 1>(st, dpt, qreg, greg, kaddr, vaddr, ring);
    }
}

// ---------------------------------------------------------------- dK, dV

static_assert(kBwdRows == kBc, "query chunks use the 64-row segment layout");

// Per-row values of a chunk staged through registers (Q and dO go straight
// into LDS), as loaded: they are scaled and clamped only when stored, at the
// end of the step, so that no wait for them (which would also wait for the
// chunk's LDS loads issued before them) falls inside the step.
template <int D, int NIV>
struct DkvStage {
    float lse, dd;
    int cs[NIV], ce[NIV];
};

// The per-row values of the chunk starting at row0 into registers (thread
// tid < kBwdRows takes row row0 + tid).
template <int D, int NIV>
__device__ __forceinline__ void dkv_load_rows(DkvStage<D, NIV>& st, const float* __restrict__ lse_bh,
                                              const float* __restrict__ dd_bh, const int32_t* __restrict__ cs_b,
                                              const int32_t* __restrict__ ce_b, int row0, int N, int tid) {
    if (tid < kBwdRows) {
        const int row = row0 + tid;
        st.lse = 0.f;
        st.dd = 0.f;
#pragma unroll
        for (int k = 0; k < NIV; ++k) st.cs[k] = st.ce[k] = 0;
        if (row < N) {
            st.lse = lse_bh[row];
            st.dd = dd_bh[row];
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
                st.cs[k] = cs_b[(int64_t)k * N + row];
                st.ce[k] = ce_b[(int64_t)k * N + row];
            }
        }
    }
}

template <int D, int NIV, class SM>
__device__ __forceinline__ void dkv_store(const DkvStage<D, NIV>& st, SM& sm, int buf, int row0, int N, int tid) {
    if (tid < kBwdRows) {
        const bool in = row0 + tid < N;
        sm.lse2[buf][tid] = in ? st.lse * kLog2e : INFINITY;   // P = 0 for rows past N
        sm.dd[buf][tid] = in ? st.dd : 0.f;
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            const int2 iv = in ? clamp_interval(st.cs[k], st.ce[k], N) : make_int2(kEmptyStart, 0);
            sm.start[buf][k][tid] = iv.x;
            sm.width[buf][k][tid] = iv.y;
        }
    }
}

// Records of chunk c (one per range) for key block J: live if some range's
// non-skip blocks [x, y] hold J, full if some range covers J for every row of
// the chunk (its blocks [z, w]).
template <int NIV>
__device__ __forceinline__ void chunk_state(const TileMeta (&m)[NIV], int J, bool& live, bool& full) {
    live = full = false;
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
        live |= m[k].x <= J && J <= m[k].y;
        full |= m[k].z <= J && J <= m[k].w;
    }
}

// First live chunk >= c (INT_MAX if none up to last), searched synchronously;
// full: its full flag.
template <int NIV>
__device__ __forceinline__ int next_live_chunk(const TileMeta* __restrict__ meta_c, int64_t meta_row, int J, int c,
                                               int last, bool& full) {
    full = false;
    for (; c <= last; ++c) {
        TileMeta m[NIV];
#pragma unroll
        for (int k = 0; k < NIV; ++k) m[k] = meta_c[(meta_row + c) * NIV + k];
        bool live, f;
        chunk_state<NIV>(m, J, live, f);
        if (live) {
            full = f;
            return c;
        }
    }
    return INT_MAX;
}

// The records of one candidate chunk, loaded a step ahead: issued at the top
// of a step and tested at its end, where the wait for that step's own loads
// already is, so that finding the chunk after next costs no exposed load.
template <int NIV>
struct ChunkProbe {
    TileMeta m[NIV];
    int cand;
};
template <int NIV>
__device__ __forceinline__ void probe_issue(ChunkProbe<NIV>& pr, const TileMeta* __restrict__ meta_c,
                                            int64_t meta_row, int cand, int last) {
    pr.cand = cand;
    if (cand <= last) {
#pragma unroll
        for (int k = 0; k < NIV; ++k) pr.m[k] = meta_c[(meta_row + cand) * NIV + k];
    }
}
template <int NIV>
__device__ __forceinline__ int probe_resolve(const ChunkProbe<NIV>& pr, const TileMeta* __restrict__ meta_c,
                                             int64_t meta_row, int J, int last, bool& full) {
    full = false;
    if (pr.cand > last) return INT_MAX;
    bool live, f;
    chunk_state<NIV>(pr.m, J, live, f);
    if (live) {
        full = f;
        return pr.cand;
    }
    return next_live_chunk<NIV>(meta_c, meta_row, J, pr.cand + 1, last, full);
}

// Start and width of the same four queries in every range (range k at
// k kBwdRows entries), waited for at once.
template <int NIV, int OFF, int K = 0>
__device__ __forceinline__ void range_rows_read(u32x4 (&sr)[NIV], u32x4 (&wr)[NIV], uint32_t sbase,
                                                uint32_t wbase) {
    if constexpr (K < NIV) {
        sr[K] = lds_read_b128<OFF + K * kBwdRows * 4>(sbase);
        wr[K] = lds_read_b128<OFF + K * kBwdRows * 4>(wbase);
        range_rows_read<NIV, OFF, K + 1>(sr, wr, sbase, wbase);
    } else {
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            wait_lds_one<0>(sr[k]);
            wait_lds_one<0>(wr[k]);
        }
    }
}

// ---- dK/dV.  Keeping K, V and both accumulators of 32 keys in one wavefront
// fills the register file (one wavefront per SIMD), and its exponentials and
// dS then run with no MFMA beside them.  Here a pair of wavefronts shares 32
// keys, one chunk apart.  In step s the P wavefront (K and dV^T in registers)
// computes S = Q K^T of chunk s, the masked P (written to LDS), and
// dV^T += dO^T P; the dS wavefront (V and dK^T) takes P of chunk s-1 from LDS,
// forms dS = P (dP - D) with the dP it kept from step s-1, accumulates
// dK^T += Q^T dS over chunk s-1, and computes dP = dO V^T of chunk s.  Each
// wavefront fits in half the registers, so two run per SIMD, and each role's
// vector work (the exponentials; dS) has the other role's products beside it,
// with one barrier per step.  Q is kept for three chunks (s-1 for dK, s, s+1
// loading), dO and P for two.  Both products of a role come out in the same
// tile layout (rows of the chunk by the pair's keys), so a lane of the dS
// wavefront reads back exactly the P values the same lane of the P wavefront
// wrote.  Each of dK and dV sums the same products in the same order as one
// wavefront doing both would.

// S = Q K^T (or dP = dO V^T) of both 32-query halves of a chunk: read I holds
// head-dimension chunk I / 2 of query 32 (I % 2) + r32 of the lane and feeds
// MFMA I; the halves alternate so that consecutive products are independent.
template <int D, int I>
__device__ __forceinline__ u32x4 rows_read(uint32_t addr) {
    using SL = SegLayout<D>;
    constexpr int off = (I % 2) * (32 / SL::kSegs) * SL::kRowBytes + (I / 2) * 32;
    return lds_read_b128<off>(addr);
}
template <int D, int I = 0>
__device__ __forceinline__ void rows_issue(u32x4 (&ring)[kAheadS], uint32_t addr) {
    if constexpr (I < kAheadS) {
        ring[I] = rows_read<D, I>(addr);
        rows_issue<D, I + 1>(ring, addr);
    }
}
template <int D, int I = 0>
__device__ __forceinline__ void rows_products(floatx16 (&acc)[2], const bf16x8 (&b)[D / 16], uint32_t addr,
                                              u32x4 (&ring)[kAheadS]) {
    constexpr int kN = 2 * (D / 16);
    static_assert(kN > kAheadS, "more MFMAs than reads in flight");
    if constexpr (I < kN) {
        constexpr int issued = I + kAheadS < kN ? I + kAheadS : kN;
        wait_lds_one<issued - (I + 1)>(ring[I % kAheadS]);
        const bf16x8 a = __builtin_bit_cast(bf16x8, ring[I % kAheadS]);
        acc[I % 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b[I / 2], acc[I % 2], 0, 0, 0);
        if constexpr (I + kAheadS < kN) ring[I % kAheadS] = rows_read<D, I + kAheadS>(addr);
        rows_products<D, I + 1>(acc, b, addr, ring);
    }
}

// acc^T += X^T W over steps KS .. KEND-1 (16 queries each) of a chunk, X^T
// read with transposing LDS reads (cur: step KS's), W the weights as MFMA B
// operands (w[KS]: queries 16 KS .. of the lane's key).
template <int D, int KS, int KEND>
__device__ __forceinline__ void kt_products(const bf16x8 (&w)[kBwdRows / 16], floatx16 (&acc)[D / 32],
                                            uint32_t addr, v4s (&cur)[2 * D / 32]) {
    constexpr int NP = 2 * D / 32;
    if constexpr (KS < KEND) {
        v4s next[NP];
        if constexpr (KS + 1 < KEND) {
            issue_kt_reads<D, KS + 1>(next, addr);
            wait_lds_tied<NP>(cur);
        } else {
            wait_lds_tied<0>(cur);
        }
#pragma unroll
        for (int nb = 0; nb < D / 32; ++nb) {
            const bf16x8 a = __builtin_bit_cast(
                bf16x8, __builtin_shufflevector(cur[2 * nb], cur[2 * nb + 1], 0, 1, 2, 3, 4, 5, 6, 7));
            acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, w[KS], acc[nb], 0, 0, 0);
        }
        kt_products<D, KS + 1, KEND>(w, acc, addr, next);
    }
}

// The dS wavefront's P (exchange slots I = 4 qb + g, 1 KB apart) and D
// (queries 32 qb + 8 g + 4 half .. +3) reads, and the waits for them in issue
// order (LDS reads complete in order; lgkmcnt counts up to 15).
template <int I = 0>
__device__ __forceinline__ void pair_weight_reads(u32x4 (&pr)[8], u32x4 (&dr)[8], uint32_t xaddr, uint32_t daddr) {
    if constexpr (I < 8) {
        pr[I] = lds_read_b128<I * 1024>(xaddr);
        dr[I] = lds_read_b128<((I / 4) * 32 + 8 * (I % 4)) * 4>(daddr);
        pair_weight_reads<I + 1>(pr, dr, xaddr, daddr);
    }
}
template <int I = 0>
__device__ __forceinline__ void pair_weight_waits(u32x4 (&pr)[8], u32x4 (&dr)[8]) {
    if constexpr (I < 8) {
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(pr[I]), "+v"(dr[I]) : "i"(2 * (7 - I)));
        pair_weight_waits<I + 1>(pr, dr);
    }
}

// LSE of queries 32 QB + 8 g + 4 half .. +3, g = 0..3 (lbase: this lane's
// element 4 half of the row array), as inline assembly.
template <int QB, int G = 0>
__device__ __forceinline__ void lse_issue(u32x4 (&lr)[4], uint32_t lbase) {
    if constexpr (G < 4) {
        lr[G] = lds_read_b128<(QB * 32 + 8 * G) * 4>(lbase);
        lse_issue<QB, G + 1>(lr, lbase);
    }
}
__device__ __forceinline__ void wait_lds4(u32x4 (&r)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
}
template <int OFF>
__device__ __forceinline__ void lds_write_b128(uint32_t addr, float4 v) {
    static_assert(OFF >= 0 && OFF < 65536, "ds offset field");
    const u32x4 bits = __builtin_bit_cast(u32x4, v);
    asm volatile("ds_write_b128 %0, %1 offset:%2" : : "v"(addr), "v"(bits), "i"(OFF) : "memory");
}

// One 1 KB slab into LDS: lane l's 16 bytes from byte src of the tensor to
// dst + 16 l.
template <typename Ptr>
__device__ __forceinline__ void dma_kv_slab(__amdgpu_buffer_rsrc_t rs, Ptr dst, int src) {
#if defined(__HIP_DEVICE_COMPILE__)   // the LDS address-space cast exists in the device pass only
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 16, src, 0, 0, 0);
#endif
}

template <int D, int NIV>
struct alignas(16) DkvSmem {
    alignas(16) uint8_t q[3][SegLayout<D>::kBytes];     // Q of chunks s-1, s, s+1 (index chunk % 3)
    alignas(16) uint8_t go[2][SegLayout<D>::kBytes];    // dO of chunks s, s+1 (index chunk % 2)
    alignas(16) float lse2[3][kBwdRows];
    alignas(16) float dd[3][kBwdRows];
    alignas(16) int start[3][NIV][kBwdRows];
    alignas(16) int width[3][NIV][kBwdRows];
    alignas(16) float4 xch[2][kWaves][2][4][64];       // P of step s in [s % 2]: [pair][half][four queries][lane]
};

template <int D, int NIV>
__global__ __launch_bounds__(2 * kThreads, 1) void bwd_dkdv_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dd,
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_end,
    const TileMeta* __restrict__ meta_c, const int4* __restrict__ pieces, const int32_t* __restrict__ pslot,
    const int32_t* __restrict__ order, int H, int N, int n_qc, int n_kb, int Lk, float c, float scale,
    int xcd_heads, int per_head, float* __restrict__ dK, float* __restrict__ dV, float* __restrict__ part) {
    __shared__ DkvSmem<D, NIV> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int kw = wave & (kWaves - 1);          // the pair's 32-key column block
    const bool dsw = wave >= kWaves;             // dS wavefront (it also loads the chunks)
    const int half = lane >> 5;
    const int r32 = lane & 31;

    int h, slot;
    slot_to_item(xcd_heads, H, h, slot);
    const int Lp = gridDim.x / H;
    const int set = per_head ? h : 0;
    const int n_sets = per_head ? H : 1;
    const int pe = order[set * Lp + slot];
    const int4 piece = pieces[pe];              // {item, first chunk, last chunk, p << 16 | P}
    if (piece.x < 0) return;                    // unused entry: the whole workgroup leaves
    const int bj = piece.x;
    const int local = bj - set * Lk;
    const int b = local / n_kb;
    const int J = local - b * n_kb;

    const int64_t bh = (int64_t)b * H + h;
    const int key = J * kBwdKeys + kw * 32 + r32;
    const int kw0 = J * kBwdKeys + kw * 32;

    // The key block's K and V rows go into the P exchange buffer (idle until
    // the first step) in whole-kilobyte pieces, the P wavefronts loading K and
    // the dS wavefronts V; below, each lane reads its key's row from there
    // (K for the P wavefront, V for the dS wavefront) as MFMA B operands,
    // [key][16 cs + 8 half .. +7].  Loaded straight into registers, each
    // instruction would fetch 32-byte pieces of 32 rows.  Rows are stored
    // whole, their 16-byte chunks permuted (chunk c of row R in slot
    // c ^ (R mod chunks per row)) so that the 32 rows of one read meet no bank
    // conflict; rows past N arrive as zeros (the buffer range check).
    constexpr int kKvRow = 2 * D;                         // bytes per row
    constexpr int kKvChunks = kKvRow / 16;
    constexpr int kKvSlabs = 2 * kBwdKeys * kKvRow / 1024;  // K then V, 1 KB per load instruction
    constexpr int kKvSlabsPerWave = kKvSlabs / (2 * kWaves);
    static_assert(2 * kBwdKeys * kKvRow <= (int)sizeof(sm.xch), "K and V of a key block fit the exchange buffer");
    static_assert(kKvSlabs % (2 * kWaves) == 0 && kKvChunks <= 64, "whole slabs per wavefront");
    uint8_t* const kvst = reinterpret_cast<uint8_t*>(&sm.xch[0][0][0][0][0]);
    {
        const int wv = __builtin_amdgcn_readfirstlane(wave);
        const __amdgpu_buffer_rsrc_t trs = slice_rsrc((wv >= kWaves ? V : K) + bh * N * D, N * D * 2);
#pragma unroll
        for (int u = 0; u < kKvSlabsPerWave; ++u) {
            const int m = wv * kKvSlabsPerWave + u;               // slab: rows of K (m < kKvSlabs / 2), then V
            const int R = (m % (kKvSlabs / 2)) * (1024 / kKvRow) + lane / kKvChunks;
            const int c = (lane % kKvChunks) ^ (R % kKvChunks);
            dma_kv_slab(trs, kvst + m * 1024, (J * kBwdKeys + R) * kKvRow + 16 * c);
        }
    }
    bf16x8 kv[D / 16];
    floatx16 acc[D / 32];                        // dV^T (P wavefront) or dK^T (dS wavefront)
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) acc[nb] = floatx16{};

    const __amdgpu_buffer_rsrc_t qrs = slice_rsrc(Q + bh * N * D, N * D * 2);
    const __amdgpu_buffer_rsrc_t grs = slice_rsrc(dO + bh * N * D, N * D * 2);
    const float* lse_bh = LSE + bh * N;
    const float* dd_bh = Dd + bh * N;
    const int32_t* cs_b = col_start + ((int64_t)b * n_sets + set) * NIV * N;
    const int32_t* ce_b = col_end + ((int64_t)b * n_sets + set) * NIV * N;
    const int64_t meta_row = ((int64_t)set * (Lk / n_kb) + b) * n_qc;

    using SL = SegLayout<D>;
    const int wave_u = __builtin_amdgcn_readfirstlane(kw);
    const int loff = seg_lane_offset<D, true>(lane, wave_u);
    const int q_lane = k_segment<D>(r32 % SL::kSegs) * SL::kPitch + (r32 / SL::kSegs) * SL::kRowBytes + 16 * half;
    const int a4 = (lane & 15) >> 2;
    const int t_lane = (D == 128 ? 4 * a4 + half : 4 * half + a4) * SL::kPitch + 32 * ((lane >> 4) & 1) +
                       8 * (lane & 3);
    const int ltid = dsw ? kBwdRows : tid;             // the P wavefronts stage the per-row values

    bool full_t, full_next;
    int t = next_live_chunk<NIV>(meta_c, meta_row, J, piece.y, piece.z, full_t);
    if (t != INT_MAX) {
        int t_next = next_live_chunk<NIV>(meta_c, meta_row, J, t + 1, piece.z, full_next);
        // The P wavefronts load Q and the per-row values, the dS wavefronts dO.
        DkvStage<D, NIV> stage;
        if (!dsw) {
            dma_rows<D, true>(&sm.q[0][0], qrs, loff, t * kBwdRows, wave_u);
            dkv_load_rows<D, NIV>(stage, lse_bh, dd_bh, cs_b, ce_b, t * kBwdRows, N, ltid);
            dkv_store<D, NIV>(stage, sm, 0, t * kBwdRows, N, ltid);
        } else {
            dma_rows<D, true>(&sm.go[0][0], grs, loff, t * kBwdRows, wave_u);
        }
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        {
            const uint8_t* rowp = kvst + (dsw ? kBwdKeys * kKvRow : 0) + (kw * 32 + r32) * kKvRow;
            const int rsw = (kw * 32 + r32) % kKvChunks;
#pragma unroll
            for (int cs = 0; cs < D / 16; ++cs)
                kv[cs] = *reinterpret_cast<const bf16x8*>(rowp + 16 * ((2 * cs + half) ^ rsw));
        }
        __syncthreads();   // every K/V row is in registers before the first P is written there
        // The dS wavefront's pending chunk (the previous step's): its dP tiles,
        // whether it was skipped.
        floatx16 dpp[2] = {};
        bool pend = false, pend_skip = true;
        for (int s = 0;; ++s) {
            const bool has_cur = t != INT_MAX;
            const bool has_next = has_cur && t_next != INT_MAX;
            const int q3 = s % 3, qp3 = (s + 2) % 3, qn3 = (s + 1) % 3;   // chunk s, s-1, s+1 buffers
            const int g2 = s & 1;

            // Does some row of chunk t attend the wavefront's keys, and does
            // one range cover them for every row (both roles decide alike)?
            const int klo = kw0;
            bool wave_skip = !has_cur || klo >= N, wave_full = true;
            if (has_cur && !full_t) {
                const int row0 = t * kBwdRows;
                const int khi = min(kw0 + 31, N - 1);
                bool skip = true, full = false;
#pragma unroll
                for (int k = 0; k < NIV; ++k) {
                    const int4 rb = wave_row_bounds(sm.start[q3][k][lane], sm.width[q3][k][lane], row0 + lane < N);
                    skip &= khi < rb.x || klo > rb.y;
                    full |= klo >= rb.z && khi <= rb.w;
                }
                wave_skip |= skip;
                wave_full = full;
            }

            ChunkProbe<NIV> probe;
            if (has_next) {
                if (!dsw) {
                    dma_rows<D, true>(&sm.q[qn3][0], qrs, loff, t_next * kBwdRows, wave_u);
                    dkv_load_rows<D, NIV>(stage, lse_bh, dd_bh, cs_b, ce_b, t_next * kBwdRows, N, ltid);
                } else {
                    dma_rows<D, true>(&sm.go[g2 ^ 1][0], grs, loff, t_next * kBwdRows, wave_u);
                }
                probe_issue<NIV>(probe, meta_c, meta_row, t_next + 1, piece.z);
            }

            if (!dsw) {
                if (!wave_skip) {
                    // ---- S of chunk s: lane holds [query 32 qb + 8 (v/4) + 4 half + v%4][key] in x[qb][v]
                    floatx16 x[2] = {};
                    {
                        const uint32_t rows = lds_address(&sm.q[q3][0]) + q_lane;
                        u32x4 ring[kAheadS];
                        rows_issue<D>(ring, rows);
                        rows_products<D>(x, kv, rows, ring);
                    }
                    // ---- P = exp(scale s - LSE) inside the ranges, to LDS and as operands.
                    // LSE, the intervals and the exchange slots are read and written
                    // as inline assembly: ordinary LDS accesses here would make the
                    // compiler first wait for this wavefront's loads of chunk s+1.
                    const uint32_t lbase = lds_address(&sm.lse2[q3][4 * half]);
                    const uint32_t sbase = lds_address(&sm.start[q3][0][4 * half]);
                    const uint32_t wbase = lds_address(&sm.width[q3][0][4 * half]);
                    const uint32_t xbase = lds_address(&sm.xch[g2][kw][0][0][lane]);
                    auto weights = [&](auto qbc, auto fullc) {
                        constexpr int qb = decltype(qbc)::value;
                        constexpr bool kFull = decltype(fullc)::value;
                        u32x4 lr[4];
                        lse_issue<qb>(lr, lbase);
                        wait_lds4(lr);
                        auto group = [&](auto gc) {
                            constexpr int g = decltype(gc)::value;
                            const float4 l4 = __builtin_bit_cast(float4, lr[g]);
                            const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                            bool ok[4] = {true, true, true, true};
                            if constexpr (!kFull) {
#pragma unroll
                                for (int q = 0; q < 4; ++q) ok[q] = false;
                                u32x4 sr[NIV], wr[NIV];
                                range_rows_read<NIV, (qb * 32 + 8 * g) * 4>(sr, wr, sbase, wbase);
#pragma unroll
                                for (int k = 0; k < NIV; ++k) {
                                    const int4 s4 = __builtin_bit_cast(int4, sr[k]);
                                    const int4 w4 = __builtin_bit_cast(int4, wr[k]);
                                    ok[0] |= (uint32_t)(key - s4.x) <= (uint32_t)w4.x;
                                    ok[1] |= (uint32_t)(key - s4.y) <= (uint32_t)w4.y;
                                    ok[2] |= (uint32_t)(key - s4.z) <= (uint32_t)w4.z;
                                    ok[3] |= (uint32_t)(key - s4.w) <= (uint32_t)w4.w;
                                }
                            }
#pragma unroll
                            for (int q = 0; q < 4; ++q) {
                                const int v = 4 * g + q;
                                const float p = __builtin_amdgcn_exp2f(fmaf(x[qb][v], c, -lv[q]));
                                x[qb][v] = kFull || ok[q] ? p : 0.f;
                            }
                            lds_write_b128<(qb * 4 + g) * 1024>(
                                xbase, make_float4(x[qb][4 * g], x[qb][4 * g + 1], x[qb][4 * g + 2], x[qb][4 * g + 3]));
                        };
                        group(std::integral_constant<int, 0>{});
                        group(std::integral_constant<int, 1>{});
                        group(std::integral_constant<int, 2>{});
                        group(std::integral_constant<int, 3>{});
                    };
                    if (wave_full) {
                        weights(std::integral_constant<int, 0>{}, std::true_type{});
                        weights(std::integral_constant<int, 1>{}, std::true_type{});
                    } else {
                        weights(std::integral_constant<int, 0>{}, std::false_type{});
                        weights(std::integral_constant<int, 1>{}, std::false_type{});
                    }
                    bf16x8 w[kBwdRows / 16];
#pragma unroll
                    for (int ks = 0; ks < kBwdRows / 16; ++ks)
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[ks][e] = (__bf16)x[ks >> 1][8 * (ks & 1) + e];
                    // ---- dV^T += dO^T P over chunk s
                    const uint32_t taddr = lds_address(&sm.go[g2][0]) + t_lane;
                    v4s cur[2 * D / 32];
                    issue_kt_reads<D, 0>(cur, taddr);
                    kt_products<D, 0, kBwdRows / 16>(w, acc, taddr, cur);
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // P is in LDS before the barrier
                }
            } else {
                if (pend && !pend_skip) {
                    // ---- dS = P (dP - D) of chunk s-1, P and D read as inline
                    // assembly (the compiler would first wait for this
                    // wavefront's loads of chunk s+1, which write other LDS)
                    u32x4 pr[8], dr[8];
                    pair_weight_reads(pr, dr, lds_address(&sm.xch[g2 ^ 1][kw][0][0][lane]),
                                      lds_address(&sm.dd[qp3][4 * half]));
                    pair_weight_waits(pr, dr);
#pragma unroll
                    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
                        for (int g = 0; g < 4; ++g) {
                            const float4 p4 = __builtin_bit_cast(float4, pr[4 * qb + g]);
                            const float4 d4 = __builtin_bit_cast(float4, dr[4 * qb + g]);
                            dpp[qb][4 * g] = p4.x * (dpp[qb][4 * g] - d4.x);
                            dpp[qb][4 * g + 1] = p4.y * (dpp[qb][4 * g + 1] - d4.y);
                            dpp[qb][4 * g + 2] = p4.z * (dpp[qb][4 * g + 2] - d4.z);
                            dpp[qb][4 * g + 3] = p4.w * (dpp[qb][4 * g + 3] - d4.w);
                        }
                    }
                    bf16x8 w[kBwdRows / 16];
#pragma unroll
                    for (int ks = 0; ks < kBwdRows / 16; ++ks)
#pragma unroll
                        for (int e = 0; e < 8; ++e) w[ks][e] = (__bf16)dpp[ks >> 1][8 * (ks & 1) + e];
                    // ---- dK^T += Q^T dS over chunk s-1
                    const uint32_t taddr = lds_address(&sm.q[qp3][0]) + t_lane;
                    v4s cur[2 * D / 32];
                    issue_kt_reads<D, 0>(cur, taddr);
                    kt_products<D, 0, kBwdRows / 16>(w, acc, taddr, cur);
                }
                if (!wave_skip) {
                    // ---- dP of chunk s, kept for the next step
                    dpp[0] = floatx16{};
                    dpp[1] = floatx16{};
                    const uint32_t rows = lds_address(&sm.go[g2][0]) + q_lane;
                    u32x4 ring[kAheadS];
                    rows_issue<D>(ring, rows);
                    rows_products<D>(dpp, kv, rows, ring);
                }
                pend = has_cur;
                pend_skip = wave_skip;
            }

            int t_after = INT_MAX;
            bool full_after = false;
            if (has_next) {
                if (!dsw) dkv_store<D, NIV>(stage, sm, qn3, t_next * kBwdRows, N, ltid);
                __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads have landed
                t_after = probe_resolve<NIV>(probe, meta_c, meta_row, J, piece.z, full_after);
            }
            __syncthreads();
            if (!has_cur) break;                 // that step finished the dS wavefront's last chunk
            t = t_next;
            full_t = full_next;
            t_next = t_after;
            full_next = full_after;
        }
    }

    // ---- epilogue: lane holds dV (P wavefront) or dK (dS wavefront) of its key
    // at d = 32 nb + 8 g + 4 half + (0..3); a later piece of a split block
    // writes its partial sums.  The rows go out through LDS, idle after the
    // last step's barrier (each wavefront stages its own 32 rows), so that
    // every store writes whole rows: straight from the MFMA layout one store
    // instruction would write 32-byte pieces of 32 rows.
    // (A piece with no live chunk skipped the steps: its K/V loads are waited
    // for here, so that none lands in the staged rows.)
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    constexpr int kOPitch = 4 * D + 16;                  // bytes per staged row (rows 4 banks apart)
    constexpr int kLanesPerRow = 4 * D / 16;             // 16 bytes per lane
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    static_assert(2 * kWaves * 32 * kOPitch <= (int)sizeof(DkvSmem<D, NIV>), "the staged rows fit in LDS");
    uint8_t* const ost = reinterpret_cast<uint8_t*>(&sm) + wave * 32 * kOPitch;
    const float f = dsw ? scale : 1.f;
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
        for (int g = 0; g < 4; ++g)
            *reinterpret_cast<float4*>(ost + r32 * kOPitch + 4 * (nb * 32 + 8 * g + 4 * half)) =
                make_float4(f * acc[nb][4 * g], f * acc[nb][4 * g + 1], f * acc[nb][4 * g + 2], f * acc[nb][4 * g + 3]);
    float* rows = (dsw ? dK : dV) + (bh * N + kw0) * D;  // the row of key kw0
    if ((piece.w >> 16) != 0) {
        float* pb = part + ((int64_t)pslot[pe] * H + h) * (kBwdKeys * D * 2);
        rows = pb + (kw0 - J * kBwdKeys) * D + (dsw ? 0 : kBwdKeys * D);
    }
#pragma unroll
    for (int i = 0; i < 32 / kRowsPerStore; ++i) {
        const int r = i * kRowsPerStore + lane / kLanesPerRow;
        const int cb = 16 * (lane % kLanesPerRow);
        const float4 v = *reinterpret_cast<const float4*>(ost + r * kOPitch + cb);
        if (kw0 + r < N) *reinterpret_cast<float4*>(reinterpret_cast<uint8_t*>(rows + r * D) + cb) = v;
    }
}

// ---------------------------------------------------------------- dQ

template <int D, int NIV>
struct alignas(16) DqSmem {
    alignas(16) uint8_t k[2][SegLayout<D>::kBytes];
    alignas(16) uint8_t v[2][SegLayout<D>::kBytes];
    int start[NIV][kBr];
    int width[NIV][kBr];
};

template <int D, int NIV>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(
    const uint16_t* __restrict__ Q, const uint16_t* __restrict__ K, const uint16_t* __restrict__ V,
    const uint16_t* __restrict__ dO, const float* __restrict__ LSE, const float* __restrict__ Dd,
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_end, const TileMeta* __restrict__ meta,
    const int32_t* __restrict__ order, int H, int N, int n_q, float c, float scale, int xcd_heads, int per_head,
    float* __restrict__ dQ) {
    __shared__ DqSmem<D, NIV> sm;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int half = lane >> 5;
    const int r32 = lane & 31;

    int h, slot;
    slot_to_item(xcd_heads, H, h, slot);
    const int L = gridDim.x / H;                 // query blocks per head (B n_q)
    const int set = per_head ? h : 0;
    const int n_sets = per_head ? H : 1;
    const int bt = order != nullptr ? order[set * L + slot] : set * L + slot;
    const int local = bt - set * L;
    const int b = local / n_q;
    const int t = local - b * n_q;
    TileMeta tm[NIV];
#pragma unroll
    for (int k = 0; k < NIV; ++k) tm[k] = meta[(int64_t)bt * NIV + k];

    const int64_t bh = (int64_t)b * H + h;
    const int row0 = t * kBr;
    const int qrow = row0 + wave * 32 + r32;

    if (tid < kBr) {
        const int r = row0 + tid;
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            int2 iv = make_int2(kEmptyStart, 0);
            if (r < N) {
                const int64_t at = (((int64_t)b * n_sets + set) * NIV + k) * N + r;
                iv = clamp_interval(col_start[at], col_end[at], N);
            }
            sm.start[k][tid] = iv.x;
            sm.width[k][tid] = iv.y;
        }
    }

    // Q and dO rows of this lane's query as MFMA B operands.
    bf16x8 qreg[D / 16], greg[D / 16];
#pragma unroll
    for (int cs = 0; cs < D / 16; ++cs) {
        if (qrow < N) {
            qreg[cs] = *reinterpret_cast<const bf16x8*>(Q + (bh * N + qrow) * D + cs * 16 + half * 8);
            greg[cs] = *reinterpret_cast<const bf16x8*>(dO + (bh * N + qrow) * D + cs * 16 + half * 8);
        } else {
            qreg[cs] = bf16x8{};
            greg[cs] = bf16x8{};
        }
    }
    const float lse2 = qrow < N ? LSE[bh * N + qrow] * kLog2e : INFINITY;   // P = 0 past N
    const float drow = qrow < N ? Dd[bh * N + qrow] : 0.f;

    floatx16 dqacc[D / 32];
#pragma unroll
    for (int nb = 0; nb < D / 32; ++nb) dqacc[nb] = floatx16{};

    __syncthreads();
    int my_s[NIV], my_w[NIV];
    int4 wb[NIV];
#pragma unroll
    for (int k = 0; k < NIV; ++k) {
        my_s[k] = sm.start[k][wave * 32 + r32];
        my_w[k] = sm.width[k][wave * 32 + r32];
        wb[k] = wave_row_bounds(my_s[k], my_w[k], qrow < N);
    }

    const __amdgpu_buffer_rsrc_t krs = slice_rsrc(K + bh * N * D, N * D * 2);
    const __amdgpu_buffer_rsrc_t vrs = slice_rsrc(V + bh * N * D, N * D * 2);

    // Lane offsets of the loads and of the operand reads (see SegLayout).
    using DL = SegLayout<D>;
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    const int kvoff = seg_lane_offset<D, true>(lane, wave_u);
    const int vvoff = seg_lane_offset<D, false>(lane, wave_u);
    const int k_lane = k_segment<D>(r32 % DL::kSegs) * DL::kPitch + (r32 / DL::kSegs) * DL::kRowBytes + 16 * half;
    const int v_lane = (r32 % DL::kSegs) * DL::kPitch + (r32 / DL::kSegs) * DL::kRowBytes + 16 * half;
    const int a4 = (lane & 15) >> 2;
    const int kt_lane = (D == 128 ? 4 * a4 + half : 4 * half + a4) * DL::kPitch + 32 * ((lane >> 4) & 1) +
                        8 * (lane & 3);

    int j = union_next<NIV>(tm, -1);
    if (j != INT_MAX) {
        dma_rows<D, true>(&sm.k[0][0], krs, kvoff, j * kBc, wave_u);
        dma_rows<D, false>(&sm.v[0][0], vrs, vvoff, j * kBc, wave_u);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        for (int buf = 0;; buf ^= 1) {
            const int j_next = union_next<NIV>(tm, j);
            const bool has_next = j_next != INT_MAX;
            if (has_next) {
                dma_rows<D, true>(&sm.k[buf ^ 1][0], krs, kvoff, j_next * kBc, wave_u);
                dma_rows<D, false>(&sm.v[buf ^ 1][0], vrs, vvoff, j_next * kBc, wave_u);
            }

            const int klo = j * kBc;
            const int khi = min(klo + kBc, N) - 1;
            bool wave_skip = true, wave_full = false;
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
                wave_skip &= khi < wb[k].x || klo > wb[k].y;
                wave_full |= klo >= wb[k].z && khi <= wb[k].w;
            }
            wave_full &= klo + kBc <= N;         // keys past N are always masked
            if (!wave_skip) {
                // ---- S^T = K Q^T, dP^T = V dO^T: lane holds [key 32 jb + 8 (v/4) + 4 half + v%4][query]
                floatx16 st[kBc / 32], dpt[kBc / 32];
#pragma unroll
                for (int jb = 0; jb < kBc / 32; ++jb) {
                    st[jb] = floatx16{};
                    dpt[jb] = floatx16{};
                }
                {
                    const uint32_t krow = lds_address(&sm.k[buf][0]) + k_lane;
                    const uint32_t vrow = lds_address(&sm.v[buf][0]) + v_lane;
                    u32x4 ring[kAheadS];
                    dq_sdp_issue<D>(ring, krow, vrow);
                    dq_sdp_products<D>(st, dpt, qreg, greg, krow, vrow, ring);
                }
                // ---- dS^T = P^T (dP^T - D) with P = exp(scale s - LSE) inside the ranges
                int base[NIV];
#pragma unroll
                for (int k = 0; k < NIV; ++k) base[k] = klo + 4 * half - my_s[k];
#pragma unroll
                for (int jb = 0; jb < kBc / 32; ++jb) {
#pragma unroll
                    for (int v = 0; v < 16; ++v) {
                        bool ok = true;
                        if (!wave_full) {
                            const int off = jb * 32 + 8 * (v >> 2) + (v & 3);
                            ok = false;
#pragma unroll
                            for (int k = 0; k < NIV; ++k) ok |= (uint32_t)(base[k] + off) <= (uint32_t)my_w[k];
                        }
                        const float p = __builtin_amdgcn_exp2f(fmaf(st[jb][v], c, -lse2));
                        const float pm = ok ? p : 0.f;
                        dpt[jb][v] = pm * (dpt[jb][v] - drow);
                    }
                }
                // ---- dQ^T += K^T dS^T: A operand lane (column i, half h), element e:
                // K^T[i][key 16 ks + 8 (e / 4) + 4 h + e % 4], the key order of dS^T
                // in the registers; two transposing reads of four keys each.
                const uint32_t kaddr = lds_address(&sm.k[buf][0]) + kt_lane;
                v4s kpart[2 * D / 32];
                issue_kt_reads<D, 0>(kpart, kaddr);
                dq_product<D, 0>(dpt, dqacc, kaddr, kpart);
            }
            if (has_next) __builtin_amdgcn_s_waitcnt(0);   // this wavefront's loads have landed
            __syncthreads();
            if (!has_next) break;
            j = j_next;
        }
    }

    // ---- epilogue: lane holds dQ of its query at d = 32 nb + 8 g + 4 half + (0..3).
    // The rows go out through LDS so that every store writes whole rows (as in
    // the dK/dV kernel), each wavefront staging its own rows; where the
    // buffers cannot hold all 128 rows at once (d = 64) they go in two passes
    // of 16 rows per wavefront (LDS operations of one wavefront take effect in
    // issue order, so a pass may overwrite what the previous one read).  The
    // barrier keeps the staging clear of another wavefront's reads of the
    // staged intervals on a query block with no key blocks.
    __syncthreads();
    constexpr int kOPitch = 4 * D + 16;                  // bytes per staged row (rows 4 banks apart)
    constexpr int kOPasses = kWaves * 32 * kOPitch <= (int)sizeof(DqSmem<D, NIV>) ? 1 : 2;
    static_assert(kWaves * 32 * kOPitch <= kOPasses * (int)sizeof(DqSmem<D, NIV>), "the staged rows fit in LDS");
    constexpr int kPassRows = 32 / kOPasses;
    constexpr int kLanesPerRow = 4 * D / 16;             // 16 bytes per lane
    constexpr int kRowsPerStore = 64 / kLanesPerRow;
    static_assert(kPassRows % kRowsPerStore == 0, "whole stores per pass");
    uint8_t* const ost = reinterpret_cast<uint8_t*>(&sm) + wave * kPassRows * kOPitch;
    float* const rows = dQ + (bh * N + row0 + wave * 32) * D;   // the wavefront's first row
#pragma unroll
    for (int pass = 0; pass < kOPasses; ++pass) {
        if (r32 / kPassRows == pass) {
            uint8_t* const orow = ost + (r32 - pass * kPassRows) * kOPitch;
#pragma unroll
            for (int nb = 0; nb < D / 32; ++nb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<float4*>(orow + 4 * (nb * 32 + 8 * g + 4 * half)) =
                        make_float4(scale * dqacc[nb][4 * g], scale * dqacc[nb][4 * g + 1],
                                    scale * dqacc[nb][4 * g + 2], scale * dqacc[nb][4 * g + 3]);
        }
#pragma unroll
        for (int i = 0; i < kPassRows / kRowsPerStore; ++i) {
            const int r = i * kRowsPerStore + lane / kLanesPerRow;
            const int cb = 16 * (lane % kLanesPerRow);
            const float4 v = *reinterpret_cast<const float4*>(ost + r * kOPitch + cb);
            const int rr = pass * kPassRows + r;
            if (row0 + wave * 32 + rr < N)
                *reinterpret_cast<float4*>(reinterpret_cast<uint8_t*>(rows + rr * D) + cb) = v;
        }
    }
}

// ---------------------------------------------------------------- small problems: one preparation launch
//
// When no key block can be split (no block sees more query chunks than the
// smallest piece holds) and the problem is small, the records of both
// gradient kernels come from one workgroup instead of five launches: the
// query blocks' records of the dQ kernel (run in natural order), the query
// chunks' records, each key block's first and last live chunk, and the
// one-piece table with the identity order of the dK/dV kernel.  They are the
// numbers the separate launches produce (the preprocessor's rule, the chunk
// scan of kv_ranges_kernel, bwd_split_kernel with nothing to split); only
// the order of the gradient kernels' workgroups differs, which changes no
// result.  The chunk records are kept in LDS for the chunk scan.
constexpr int kPrepFusedThreads = 1024;
template <int NIV>
__global__ __launch_bounds__(kPrepFusedThreads) void bwd_prep_fused_kernel(
    const int32_t* __restrict__ col_start, const int32_t* __restrict__ col_end, int N, int B, int n_sets,
    TileMeta* __restrict__ meta_q, TileMeta* __restrict__ meta_c, int4* __restrict__ pieces,
    int32_t* __restrict__ pslot, int32_t* __restrict__ order_k, int Lp) {
    __shared__ TileMeta chunk_meta[kBwdFusedMaxChunks * NIV];
    constexpr int kWv = kPrepFusedThreads / 64;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int n_q = (N + kBr - 1) / kBr, n_kv = (N + kBc - 1) / kBc;
    const int n_qc = (N + kBwdRows - 1) / kBwdRows, n_kb = (N + kBwdKeys - 1) / kBwdKeys;
    const int Mq = n_sets * B * n_q, Mc = n_sets * B * n_qc, Mk = n_sets * B * n_kb;
    // records: query blocks (kBr rows, kBc keys) then query chunks (kBwdRows
    // rows, kBwdKeys keys), one wavefront each, items of one interval set
    // contiguous (as preprocess_kernel numbers them)
    for (int item = wv; item < Mq + Mc; item += kWv) {
        const bool chunk = item >= Mq;
        const int it = chunk ? item - Mq : item;
        const int nt = chunk ? n_qc : n_q;
        const int g = it / (B * nt);
        const int rem = it - g * (B * nt);
        const int b = rem / nt;
        const int t = rem - b * nt;
        TileMeta m[NIV];
#pragma unroll
        for (int k = 0; k < NIV; ++k) {
            const int64_t off = (((int64_t)b * n_sets + g) * NIV + k) * N;
            int inv = 0;
            m[k] = chunk ? query_block_meta(col_start + off, col_end + off, t, N, kBwdRows, kBwdKeys, n_kb, lane, &inv)
                         : query_block_meta(col_start + off, col_end + off, t, N, kBr, kBc, n_kv, lane, &inv);
        }
        if (lane == 0) {
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
                if (chunk) {
                    meta_c[it * NIV + k] = m[k];
                    chunk_meta[it * NIV + k] = m[k];
                } else {
                    meta_q[it * NIV + k] = m[k];
                }
            }
        }
    }
    __syncthreads();
    // key-block items (set B + b) n_kb + J: first and last chunk whose
    // non-skip ranges hold J, as one piece
    for (int item = wv; item < Mk; item += kWv) {
        const int sb = item / n_kb;
        const int J = item - sb * n_kb;
        int lo = INT_MAX, hi = INT_MIN, count = 0;
        for (int t = lane; t < n_qc; t += 64) {
            bool live = false;
#pragma unroll
            for (int k = 0; k < NIV; ++k) {
                const TileMeta m = chunk_meta[(sb * n_qc + t) * NIV + k];
                live |= m.x <= J && J <= m.y;
            }
            if (live) {
                lo = min(lo, t);
                hi = max(hi, t);
                ++count;
            }
        }
        lo = wave_min(lo);
        hi = wave_max(hi);
        count = wave_sum(count);
        if (lane == 0) {
            pieces[item] = make_int4(item, count > 0 ? lo : 0, count > 0 ? hi : -1, 1);
            pslot[item] = -1;
        }
    }
    // the places of extra pieces (one interval set) stay unused; identity order
    for (int e = threadIdx.x; e < n_sets * Lp; e += kPrepFusedThreads) {
        order_k[e] = e;
        if (e >= Mk) {
            pieces[e] = make_int4(-1, 0, -1, 0);
            pslot[e] = -1;
        }
    }
}

int use_xcd_heads(int64_t H, int64_t items_per_head) { return (H % 8 == 0 && items_per_head >= 128) ? 1 : 0; }

}  // namespace

hipError_t launch_bwd_rowdot(const void* out, const void* dout, int64_t rows, int64_t d, float* dd,
                             hipStream_t stream) {
    const int64_t threads = rows * (d / 8);
    const int64_t blocks = (threads + 255) / 256;
    auto kernel = d == 128 ? bwd_rowdot_kernel<128> : bwd_rowdot_kernel<64>;
    hipLaunchKernelGGL(kernel, dim3((unsigned)blocks), dim3(256), 0, stream, static_cast<const uint16_t*>(out),
                       static_cast<const uint16_t*>(dout), rows, dd);
    return hipGetLastError();
}

hipError_t launch_kv_ranges(const TileMeta* meta_c, int n_iv, int64_t B, int64_t N, int4* kvr, int32_t* work,
                            hipStream_t stream, int n_sets) {
    const int64_t n_qc = (N + kBwdRows - 1) / kBwdRows;
    const int64_t n_kb = (N + kBwdKeys - 1) / kBwdKeys;
    const int64_t items = n_sets * B * n_kb;
    const int64_t blocks = (items + 3) / 4;
    return dispatch_ranges(n_iv, [&](auto niv) {
        hipLaunchKernelGGL(kv_ranges_kernel<decltype(niv)::value>, dim3((unsigned)blocks), dim3(256), 0, stream,
                           meta_c, (int)n_qc, (int)n_kb, items, kvr, work);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_split(const int4* kvr, int64_t items, int n_sets, int min_chunks, int4* pieces,
                            int32_t* pslot, int32_t* pwork, int4* splits, hipStream_t stream) {
    hipLaunchKernelGGL(bwd_split_kernel, dim3(1), dim3(kSplitThreads), 0, stream, kvr, (int)items, n_sets,
                       min_chunks, pieces, pslot, pwork, splits);
    return hipGetLastError();
}

hipError_t launch_bwd_prep_fused(const int32_t* col_start, const int32_t* col_end, int n_iv, int64_t B, int64_t N,
                                 int n_sets, TileMeta* meta_q, TileMeta* meta_c, int4* pieces, int32_t* pslot,
                                 int32_t* order_k, hipStream_t stream) {
    const int64_t n_qc = (N + kBwdRows - 1) / kBwdRows;
    if (n_sets * B * n_qc > kBwdFusedMaxChunks) return hipErrorInvalidValue;
    const int64_t Lp = bwd_piece_entries(B * ((N + kBwdKeys - 1) / kBwdKeys), n_sets);
    return dispatch_ranges(n_iv, [&](auto niv) {
        hipLaunchKernelGGL(bwd_prep_fused_kernel<decltype(niv)::value>, dim3(1), dim3(kPrepFusedThreads), 0, stream,
                           col_start, col_end, (int)N, (int)B, n_sets, meta_q, meta_c, pieces, pslot, order_k,
                           (int)Lp);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_reduce(const int4* splits, const float* part, int64_t H, int64_t N, int64_t d, int64_t n_kb,
                             float* dk, float* dv, hipStream_t stream) {
    auto kernel = d == 128 ? bwd_reduce_kernel<128> : bwd_reduce_kernel<64>;
    hipLaunchKernelGGL(kernel, dim3(256), dim3(256), 0, stream, splits, part, (int)H, (int)N, (int)n_kb, dk, dv);
    return hipGetLastError();
}

hipError_t launch_bwd_dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                           const float* dd, const int32_t* col_start, const int32_t* col_end, int n_iv,
                           const TileMeta* meta_c, const int4* pieces, const int32_t* pslot, const int32_t* order,
                           int64_t B, int64_t H, int64_t N, int64_t d, float scale, float* dk, float* dv,
                           float* part, hipStream_t stream, int n_sets) {
    const int64_t n_qc = (N + kBwdRows - 1) / kBwdRows;
    const int64_t n_kb = (N + kBwdKeys - 1) / kBwdKeys;
    const int64_t Lp = bwd_piece_entries(B * n_kb, n_sets);
    const int64_t grid = H * Lp;
    const int xcd = use_xcd_heads(H, Lp);
    const float c = scale * kLog2e;
    return dispatch_ranges(n_iv, [&](auto niv) {
        constexpr int NIV = decltype(niv)::value;
        auto kernel = d == 128 ? bwd_dkdv_kernel<128, NIV> : bwd_dkdv_kernel<64, NIV>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(2 * kThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), lse, dd, col_start,
                           col_end, meta_c, pieces, pslot, order, (int)H, (int)N, (int)n_qc, (int)n_kb,
                           (int)(B * n_kb), c, scale, xcd, n_sets > 1 ? 1 : 0, dk, dv, part);
        return hipGetLastError();
    });
}

hipError_t launch_bwd_dq(const void* q, const void* k, const void* v, const void* dout, const float* lse,
                         const float* dd, const int32_t* col_start, const int32_t* col_end, int n_iv,
                         const TileMeta* meta, const int32_t* order, int64_t B, int64_t H, int64_t N, int64_t d,
                         float scale, float* dq, hipStream_t stream, int n_sets) {
    const int64_t n_q = (N + kBr - 1) / kBr;
    const int64_t grid = B * H * n_q;
    const int xcd = use_xcd_heads(H, B * n_q);
    const float c = scale * kLog2e;
    return dispatch_ranges(n_iv, [&](auto niv) {
        constexpr int NIV = decltype(niv)::value;
        auto kernel = d == 128 ? bwd_dq_kernel<128, NIV> : bwd_dq_kernel<64, NIV>;
        hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream,
                           static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                           static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(dout), lse, dd, col_start,
                           col_end, meta, order, (int)H, (int)N, (int)n_q, c, scale, xcd, n_sets > 1 ? 1 : 0, dq);
        return hipGetLastError();
    });
}

}  // namespace fm
