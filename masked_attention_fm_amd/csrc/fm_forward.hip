// The forward pass's launch sequence: workspace plan, then the interval
// preprocessor, the work ordering and the attention kernel, queued on the
// caller's stream.  The C ABI (fm_api.hip) checks the arguments and supplies
// the workspace: the library's per-(device, stream) buffer, or the static
// scratch array of the no-allocation entry point.  Everything that decides
// what the attention launch does (its grid, its order, its tile records) is
// here or in the kernels' own sources.

#include <algorithm>

#include "fm_internal.h"

namespace fm {

FwdPlan fwd_plan(const FwdArgs& a, bool single_launch, bool split_keys, bool across_workgroups,
                 int64_t row_slices_max) {
    FwdPlan p;
    p.n_q = (a.N + kBr - 1) / kBr;
    p.n_kv = (a.N + kBc - 1) / kBc;
    p.n_sets = a.per_head ? a.H : 1;
    p.M = p.n_sets * a.B * p.n_q;
    p.meta_bytes = ((size_t)(p.M * a.n_ranges) * sizeof(TileMeta) + 255) & ~size_t(255);
    p.int_bytes = ((size_t)p.M * sizeof(int32_t) + 255) & ~size_t(255);
    const int64_t sched_ints = schedule_scratch_ints(p.M, a.B * p.n_q, schedule_shift(p.M), (int)p.n_kv);
    p.sched_bytes = ((size_t)sched_ints * sizeof(int32_t) + 255) & ~size_t(255);
    const int64_t items = p.M * a.H / p.n_sets;          // B H n_q workgroups
    p.single = single_launch && a.fp8_scales == nullptr && items <= kSingleLaunchGrid;
    p.split = 1;
    p.groups = 1;
    p.part_bytes = 0;
    p.rows = p.single && split_keys && a.B * a.H * ((a.N + 31) / 32) <= row_slices_max;
    if (p.single && split_keys && !p.rows) {
        // Small problems: a query block's key blocks run one after another
        // in one workgroup while most CUs idle, so long ranges are cut into
        // pieces that run side by side: at d = 128 first over two wavefront
        // groups of the workgroup, then over workgroups.  (At d = 64 a key
        // block's work is mostly the softmax's vector instructions, which two
        // wavefronts on one SIMD cannot overlap: groups were slower there.)
        if (a.d == 128 && p.n_kv >= 2 * kGroupMinBlocks) p.groups = 2;
        const int64_t cap = std::min<int64_t>(std::min<int64_t>(kMaxSplit, kSingleLaunchGrid / items),
                                              p.n_kv / (p.groups * kSplitMinBlocks));
        int64_t s = 1;
        while (2 * s <= cap) s *= 2;
        if (s > 1 && items <= kSplitCounters && across_workgroups) {
            p.split = (int)s;
            p.part_bytes = split_part_bytes(items, s, a.d);
        }
    }
    return p;
}

namespace {
__global__ __launch_bounds__(256) void zero_u32_kernel(unsigned* __restrict__ p, int n) {
    const int i = blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = 0u;
}
}  // namespace

hipError_t launch_zero_u32(unsigned* p, int n, hipStream_t stream) {
    if (n <= 0) return hipSuccess;
    zero_u32_kernel<<<(n + 255) / 256, 256, 0, stream>>>(p, n);
    return hipGetLastError();
}

hipError_t fwd_launch(const FwdArgs& a, const FwdPlan& p, void* ws, unsigned* counters, bool natural,
                      hipEvent_t ev_start, hipEvent_t ev_stop) {
    if (p.rows)
        return launch_attention_rows(a.q, a.k, a.v, a.col_start, a.col_end, a.n_ranges, a.B, a.H, a.N, a.d, a.scale,
                                     a.out, a.lse, a.stream, ev_start, ev_stop, (int)p.n_sets);
    if (p.single)
        return launch_attention(a.q, a.k, a.v, a.col_start, a.col_end, a.n_ranges, nullptr, nullptr, a.B, a.H, a.N,
                                a.d, a.scale, a.out, a.lse, a.stream, ev_start, ev_stop, a.fp8_scales, (int)p.n_sets,
                                a.fp8_weights, p.split, p.split > 1 ? static_cast<float*>(ws) : nullptr,
                                p.split > 1 ? counters : nullptr, p.groups);
    auto* meta = static_cast<TileMeta*>(ws);
    auto* work = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.meta_bytes);
    auto* order = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.meta_bytes + p.int_bytes);
    auto* sched = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + p.meta_bytes + 2 * p.int_bytes);
    hipError_t e;
    if (!natural && p.M <= kPrepSmallMax) {
        // one launch: metadata and longest-first order together
        e = launch_prep_small(a.col_start, a.col_end, a.n_ranges, a.B, a.N, kBr, kBc, meta, work, order, a.stream,
                              (int)p.n_sets);
        if (e != hipSuccess) return e;
    } else {
        e = launch_preprocess(a.col_start, a.col_end, a.n_ranges, a.B, a.N, kBr, kBc, meta, work, nullptr, a.stream,
                              (int)p.n_sets);
        if (e != hipSuccess) return e;
        if (!natural) {
            e = launch_schedule(work, p.M, order, a.stream, a.B * p.n_q, schedule_shift(p.M), (int)p.n_kv, sched);
            if (e != hipSuccess) return e;
        }
    }
    return launch_attention(a.q, a.k, a.v, a.col_start, a.col_end, a.n_ranges, meta, natural ? nullptr : order, a.B,
                            a.H, a.N, a.d, a.scale, a.out, a.lse, a.stream, ev_start, ev_stop, a.fp8_scales,
                            (int)p.n_sets, a.fp8_weights);
}

}  // namespace fm
