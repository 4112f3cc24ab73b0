// C ABI of libflashmask: argument checks, workspace, kernel launches.
// The operations and their contracts are stated in include/flashmask.h.

#include <math.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "flashmask.h"
#include "fm_internal.h"

namespace {

thread_local int g_last_hip_error = 0;

int hip_fail(hipError_t e) {
    g_last_hip_error = (int)e;
    return FM_ERR_HIP;
}

#define FM_HIP(call)                          \
    do {                                      \
        hipError_t e_ = (call);               \
        if (e_ != hipSuccess) return hip_fail(e_); \
    } while (0)

static_assert(fm::kMaxRanges == FM_MAX_RANGES, "range limit of the kernels and of the ABI");

constexpr int64_t kMaxN = int64_t(1) << 28;
// The attention kernel addresses one (b, h) slice of K or V with 32-bit byte
// offsets: N * d * 2 must stay below 2^31.
constexpr int64_t kMaxAttnN = int64_t(1) << 22;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// ---------------------------------------------------------------- options

int g_schedule_mode = 0;   // 0 longest first, 1 natural order
int g_single_launch = 1;   // 1: small problems run the attention kernel alone
int g_split_keys = 1;      // 1: single launches split long key ranges over several workgroups
int64_t g_row_slices = 512;  // single launches of at most this many 32-row slices run the slice kernel
int g_bwd_min_chunks = 32; // smallest piece of a split key block (query chunks); 0: never split
int g_bwd_fused_prep = 1;  // 1: small backward problems prepare both kernels' records in one launch

// ---------------------------------------------------------------- workspace
//
// The forward calls need, per query block, 16 B of tile metadata per range,
// a work count and a place in the launch order; the backward adds the same
// for its query chunks and key blocks and one float per row and head.  One
// buffer per (device, stream) is kept and grown in stream order, so
// back-to-back calls on a stream reuse it and calls on different streams
// never share it.  It lives until the process ends.
//
// A call holds its buffer's lock from the moment it takes the buffer until
// every kernel that uses it is queued.  A second host thread on the same
// (device, stream) that needs a larger buffer therefore queues its
// hipFreeAsync of the old one after those kernels, and stream order keeps
// the old buffer alive until they have run.

struct Workspace {
    std::mutex mu;            // held while a call queues work that uses ptr or counters
    void* ptr = nullptr;
    size_t bytes = 0;
    unsigned* counters = nullptr;   // fm::kSplitCounters arrival counters, zero between calls
    // The backward's second stream (default priority) and its fork/join
    // events: its dQ chain runs beside the dK/dV chain and joins the caller's
    // stream before the call's last launch.
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
};
struct SideStream {
    hipStream_t stream;
    hipEvent_t fork, join;
};
std::mutex g_ws_map_mutex;    // guards the map itself (its nodes never move)
std::map<std::pair<int, hipStream_t>, Workspace> g_ws;

// On success *out is the buffer and `hold` owns its lock; the caller keeps
// `hold` until its last launch that uses the buffer is queued.
// With `counters`, also the stream's split-arrival counters, allocated and
// zero-filled on first use (the kernels that use them leave them zero).
hipError_t get_workspace(hipStream_t stream, size_t bytes, void** out, std::unique_lock<std::mutex>& hold,
                         unsigned** counters = nullptr, SideStream* side = nullptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    Workspace* w = nullptr;
    {
        std::lock_guard<std::mutex> lock(g_ws_map_mutex);
        w = &g_ws[{dev, stream}];
    }
    hold = std::unique_lock<std::mutex>(w->mu);
    if (w->bytes < bytes) {
        if (w->ptr != nullptr) {
            e = hipFreeAsync(w->ptr, stream);
            w->ptr = nullptr;
            w->bytes = 0;
            if (e != hipSuccess) return e;
        }
        size_t nb = std::max(bytes, size_t(64) << 10);
        nb = (nb + 0xFFFF) & ~size_t(0xFFFF);
        e = hipMallocAsync(&w->ptr, nb, stream);
        if (e != hipSuccess) {
            w->ptr = nullptr;
            return e;
        }
        w->bytes = nb;
    }
    if (counters != nullptr) {
        if (w->counters == nullptr) {
            e = hipMallocAsync(reinterpret_cast<void**>(&w->counters), fm::kSplitCounters * sizeof(unsigned), stream);
            if (e != hipSuccess) {
                w->counters = nullptr;
                return e;
            }
            e = fm::launch_zero_u32(w->counters, fm::kSplitCounters, stream);
            if (e != hipSuccess) return e;
        }
        *counters = w->counters;
    }
    if (side != nullptr) {
        if (w->side == nullptr) {
            e = hipStreamCreateWithFlags(&w->side, hipStreamNonBlocking);
            if (e != hipSuccess) {
                w->side = nullptr;
                return e;
            }
        }
        if (w->fork == nullptr) {
            e = hipEventCreateWithFlags(&w->fork, hipEventDisableTiming);
            if (e != hipSuccess) {
                w->fork = nullptr;
                return e;
            }
        }
        if (w->join == nullptr) {
            e = hipEventCreateWithFlags(&w->join, hipEventDisableTiming);
            if (e != hipSuccess) {
                w->join = nullptr;
                return e;
            }
        }
        *side = SideStream{w->side, w->fork, w->join};
    }
    *out = w->ptr;
    return hipSuccess;
}

// ---------------------------------------------------------------- timing

struct Timing {
    std::mutex mu;
    bool enabled = false;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
    std::vector<std::pair<hipEvent_t, hipEvent_t>> pool;
} g_timing;

}  // namespace

extern "C" {

FM_API const char* fm_status_string(int status) {
    switch (status) {
        case FM_OK: return "ok";
        case FM_ERR_INVALID_ARG: return "invalid argument";
        case FM_ERR_UNSUPPORTED: return "unsupported head dimension";
        case FM_ERR_BAD_INTERVAL: return "interval outside 0 <= col_start <= col_end <= N-1";
        case FM_ERR_HIP: return "HIP runtime error";
        case FM_ERR_TOO_LARGE: return "problem needs more than the no-allocation scratch holds";
        default: return "unknown status";
    }
}

FM_API int fm_last_hip_error(void) { return g_last_hip_error; }

FM_API int fm_attn_tile_shape(int64_t d, int32_t* Br, int32_t* Bc) {
    if (Br == nullptr || Bc == nullptr) return FM_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FM_ERR_UNSUPPORTED;
    *Br = fm::kBr;
    *Bc = fm::kBc;
    return FM_OK;
}

FM_API int fm_set_option(int option, int64_t value) {
    if (option == FM_OPT_SCHEDULE) {
        if (value != 0 && value != 1) return FM_ERR_INVALID_ARG;
        g_schedule_mode = (int)value;
        return FM_OK;
    }
    if (option == FM_OPT_SINGLE_LAUNCH) {
        if (value != 0 && value != 1) return FM_ERR_INVALID_ARG;
        g_single_launch = (int)value;
        return FM_OK;
    }
    if (option == FM_OPT_SPLIT_KEYS) {
        if (value != 0 && value != 1) return FM_ERR_INVALID_ARG;
        g_split_keys = (int)value;
        return FM_OK;
    }
    if (option == FM_OPT_ROW_SLICES) {
        if (value < 0 || value > (1 << 20)) return FM_ERR_INVALID_ARG;
        g_row_slices = value;
        return FM_OK;
    }
    if (option == FM_OPT_BWD_FUSED_PREP) {
        if (value != 0 && value != 1) return FM_ERR_INVALID_ARG;
        g_bwd_fused_prep = (int)value;
        return FM_OK;
    }
    if (option == FM_OPT_BWD_SPLIT_CHUNKS) {
        if (value < 0 || value > (1 << 20)) return FM_ERR_INVALID_ARG;
        g_bwd_min_chunks = (int)value;
        return FM_OK;
    }
    return FM_ERR_INVALID_ARG;
}

FM_API int fm_profile_enable(int enable) {
    std::lock_guard<std::mutex> lock(g_timing.mu);
    g_timing.enabled = enable != 0;
    return FM_OK;
}

FM_API int fm_profile_read(double* total_ms, int64_t* launches) {
    if (total_ms == nullptr || launches == nullptr) return FM_ERR_INVALID_ARG;
    std::lock_guard<std::mutex> lock(g_timing.mu);
    double sum = 0.0;
    int status = FM_OK;
    for (auto& ev : g_timing.pending) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(ev.second);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, ev.first, ev.second);
        if (e != hipSuccess) status = hip_fail(e);
        sum += ms;
        g_timing.pool.push_back(ev);
    }
    *launches = (int64_t)g_timing.pending.size();
    *total_ms = sum;
    g_timing.pending.clear();
    return status;
}

FM_API int fm_classify_tiles_multi(const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                                   int64_t N, int32_t Br, int32_t Bc, uint8_t* class_out) {
    if (col_start == nullptr || col_end == nullptr || class_out == nullptr) return FM_ERR_INVALID_ARG;
    if (n_ranges < 1 || n_ranges > fm::kMaxRanges) return FM_ERR_INVALID_ARG;
    if (N < 1 || N > kMaxN || Br < 1 || Bc < 1 || Br > kMaxN || Bc > kMaxN) return FM_ERR_INVALID_ARG;
    if (!aligned(col_start, 4) || !aligned(col_end, 4)) return FM_ERR_INVALID_ARG;
    const int64_t n_q = (N + Br - 1) / Br;
    const int64_t n_kv = (N + Bc - 1) / Bc;
    const size_t meta_bytes = (size_t)(n_q * n_ranges) * sizeof(fm::TileMeta);
    void* buf = nullptr;
    FM_HIP(hipMalloc(&buf, meta_bytes + 16));
    auto* meta = static_cast<fm::TileMeta*>(buf);
    auto* bad = reinterpret_cast<int32_t*>(static_cast<char*>(buf) + meta_bytes);
    int bad_host = 0;
    hipError_t e = hipMemsetAsync(bad, 0, sizeof(int32_t), 0);
    if (e == hipSuccess)
        e = fm::launch_preprocess(col_start, col_end, n_ranges, 1, N, Br, Bc, meta, nullptr, bad, 0);
    if (e == hipSuccess) e = fm::launch_class_table(meta, n_ranges, n_q, n_kv, class_out, 0);
    if (e == hipSuccess) e = hipMemcpy(&bad_host, bad, sizeof(int32_t), hipMemcpyDeviceToHost);
    hipError_t ef = hipFree(buf);
    if (e != hipSuccess) return hip_fail(e);
    if (ef != hipSuccess) return hip_fail(ef);
    return bad_host ? FM_ERR_BAD_INTERVAL : FM_OK;
}

FM_API int fm_classify_tiles(const int32_t* col_start, const int32_t* col_end, int64_t N, int32_t Br,
                             int32_t Bc, uint8_t* class_out) {
    return fm_classify_tiles_multi(col_start, col_end, 1, N, Br, Bc, class_out);
}

FM_API int fm_tile_schedule_multi(const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                                  int64_t B, int64_t N, int64_t d, int32_t* work_out, int32_t* order_out) {
    if (col_start == nullptr || col_end == nullptr || work_out == nullptr || order_out == nullptr)
        return FM_ERR_INVALID_ARG;
    if (n_ranges < 1 || n_ranges > fm::kMaxRanges) return FM_ERR_INVALID_ARG;
    if (B < 1 || N < 1 || N > kMaxN) return FM_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FM_ERR_UNSUPPORTED;
    const int64_t n_q = (N + fm::kBr - 1) / fm::kBr;
    if (B * n_q >= (int64_t(1) << 31)) return FM_ERR_INVALID_ARG;
    const int64_t n_kv = (N + fm::kBc - 1) / fm::kBc;
    const size_t meta_bytes = ((size_t)(B * n_q * n_ranges) * sizeof(fm::TileMeta) + 255) & ~size_t(255);
    const int64_t sched_ints = fm::schedule_scratch_ints(B * n_q, B * n_q, fm::schedule_shift(B * n_q), (int)n_kv);
    void* buf = nullptr;
    FM_HIP(hipMalloc(&buf, meta_bytes + (size_t)sched_ints * sizeof(int32_t)));
    auto* meta = static_cast<fm::TileMeta*>(buf);
    auto* sched = reinterpret_cast<int32_t*>(static_cast<char*>(buf) + meta_bytes);
    // the same path fm_attn_fwd takes for this size
    hipError_t e;
    if (B * n_q <= fm::kPrepSmallMax) {
        e = fm::launch_prep_small(col_start, col_end, n_ranges, B, N, fm::kBr, fm::kBc, meta, work_out,
                                  order_out, 0);
    } else {
        e = fm::launch_preprocess(col_start, col_end, n_ranges, B, N, fm::kBr, fm::kBc, meta, work_out,
                                  nullptr, 0);
        if (e == hipSuccess)
            e = fm::launch_schedule(work_out, B * n_q, order_out, 0, 0, fm::schedule_shift(B * n_q), (int)n_kv,
                                    sched);
    }
    if (e == hipSuccess) e = hipStreamSynchronize(0);
    hipError_t ef = hipFree(buf);
    if (e != hipSuccess) return hip_fail(e);
    if (ef != hipSuccess) return hip_fail(ef);
    return FM_OK;
}

FM_API int fm_tile_schedule(const int32_t* col_start, const int32_t* col_end, int64_t B, int64_t N,
                            int64_t d, int32_t* work_out, int32_t* order_out) {
    return fm_tile_schedule_multi(col_start, col_end, 1, B, N, d, work_out, order_out);
}

}  // extern "C"

namespace {

// ---- the forward pass: host-side checks here; the workspace plan and the
// launches into a given workspace are fm::fwd_plan / fm::fwd_launch.

int fwd_check(const fm::FwdArgs& a) {
    if (a.q == nullptr || a.k == nullptr || a.v == nullptr || a.col_start == nullptr || a.col_end == nullptr ||
        a.out == nullptr || a.lse == nullptr)
        return FM_ERR_INVALID_ARG;
    if (a.n_ranges < 1 || a.n_ranges > fm::kMaxRanges) return FM_ERR_INVALID_ARG;
    if (a.B < 1 || a.H < 1 || a.N < 1 || a.N > kMaxAttnN) return FM_ERR_INVALID_ARG;
    if (a.d != 64 && a.d != 128) return FM_ERR_UNSUPPORTED;
    if (!(a.scale > 0.f) || !isfinite(a.scale)) return FM_ERR_INVALID_ARG;
    if (!aligned(a.q, 16) || !aligned(a.k, 16) || !aligned(a.v, 16) || !aligned(a.out, 16) || !aligned(a.lse, 4) ||
        !aligned(a.col_start, 4) || !aligned(a.col_end, 4))
        return FM_ERR_INVALID_ARG;
    const int64_t n_q = (a.N + fm::kBr - 1) / fm::kBr;
    const int64_t n_sets = a.per_head ? a.H : 1;
    if (a.B * a.H * n_q >= (int64_t(1) << 31) || a.B * n_sets * a.n_ranges * a.N >= (int64_t(1) << 40))
        return FM_ERR_INVALID_ARG;
    return FM_OK;
}

// The forward pass with the library's workspace for (device, stream).
int attn_fwd_impl(const fm::FwdArgs& a) {
    const int st = fwd_check(a);
    if (st != FM_OK) return st;
    const fm::FwdPlan p = fm::fwd_plan(a, g_single_launch == 1, g_split_keys == 1, true, g_row_slices);
    void* ws = nullptr;
    unsigned* counters = nullptr;
    std::unique_lock<std::mutex> ws_hold;       // held until the launches below are queued
    FM_HIP(get_workspace(a.stream, p.total(), &ws, ws_hold, p.split > 1 ? &counters : nullptr));
    std::pair<hipEvent_t, hipEvent_t> ev{nullptr, nullptr};
    {
        std::lock_guard<std::mutex> lock(g_timing.mu);
        if (g_timing.enabled) {
            if (!g_timing.pool.empty()) {
                ev = g_timing.pool.back();
                g_timing.pool.pop_back();
            } else {
                FM_HIP(hipEventCreate(&ev.first));
                FM_HIP(hipEventCreate(&ev.second));
            }
        }
    }
    const hipError_t e = fm::fwd_launch(a, p, ws, counters, g_schedule_mode == 1, ev.first, ev.second);
    const int r = e == hipSuccess ? FM_OK : hip_fail(e);
    if (ev.first != nullptr) {
        std::lock_guard<std::mutex> lock(g_timing.mu);
        if (r == FM_OK) g_timing.pending.push_back(ev);
        else g_timing.pool.push_back(ev);
    }
    return r;
}

fm::FwdArgs fwd_args(const void* q, const void* k, const void* v, const int32_t* col_start, const int32_t* col_end,
                 int32_t n_ranges, int64_t B, int64_t H, int64_t N, int64_t d, float scale, void* out, float* lse,
                 hipStream_t stream, const float* fp8_scales = nullptr, bool per_head = false,
                 bool fp8_weights = false) {
    return fm::FwdArgs{q, k, v, col_start, col_end, n_ranges, B, H, N, d, scale, out, lse, stream, fp8_scales, per_head,
                   fp8_weights};
}

}  // namespace

// ---- the no-allocation forward: a static device scratch array.
//
// In host code `scratch` is only a host-side stand-in: its device address
// comes from hipGetSymbolAddress, taken once per device (with that device
// current) and kept; only that address is ever handed to a kernel.  Each
// device holds its own copy of the array until the process ends.
static __device__ __align__(256) unsigned char scratch[FM_NOALLOC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_addr;   // device -> address of its copy of scratch

hipError_t scratch_address(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_addr.find(dev);
    if (it != g_scratch_addr.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = ptr;
    *out = ptr;
    return hipSuccess;
}

}  // namespace

extern "C" {

FM_API int fm_attn_fwd_multi(const void* q, const void* k, const void* v, const int32_t* col_start,
                             const int32_t* col_end, int32_t n_ranges, int64_t B, int64_t H, int64_t N,
                             int64_t d, float scale, void* out, float* lse, hipStream_t stream) {
    return attn_fwd_impl(fwd_args(q, k, v, col_start, col_end, n_ranges, B, H, N, d, scale, out, lse, stream));
}

FM_API int fm_attn_fwd_per_head(const void* q, const void* k, const void* v, const int32_t* col_start,
                                const int32_t* col_end, int32_t n_ranges, int64_t B, int64_t H, int64_t N,
                                int64_t d, float scale, void* out, float* lse, hipStream_t stream) {
    return attn_fwd_impl(
        fwd_args(q, k, v, col_start, col_end, n_ranges, B, H, N, d, scale, out, lse, stream, nullptr, true));
}

FM_API int fm_attn_fwd_fp8(const void* q8, const void* k8, const void* v8, float q_scale, float k_scale,
                           float v_scale, int32_t mode, const int32_t* col_start, const int32_t* col_end,
                           int32_t n_ranges, int64_t B, int64_t H, int64_t N, int64_t d, float scale, void* out,
                           float* lse, hipStream_t stream) {
    const float scales[3] = {q_scale, k_scale, v_scale};
    for (float x : scales)
        if (!(x > 0.f) || !isfinite(x)) return FM_ERR_INVALID_ARG;
    if (mode != FM_FP8_SCORES && mode != FM_FP8_ALL) return FM_ERR_INVALID_ARG;
    return attn_fwd_impl(fwd_args(q8, k8, v8, col_start, col_end, n_ranges, B, H, N, d, scale, out, lse, stream,
                                  scales, false, mode == FM_FP8_ALL));
}

FM_API int fm_attn_fwd(const void* q, const void* k, const void* v, const int32_t* col_start,
                       const int32_t* col_end, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                       void* out, float* lse, hipStream_t stream) {
    return fm_attn_fwd_multi(q, k, v, col_start, col_end, 1, B, H, N, d, scale, out, lse, stream);
}

FM_API int fm_attn_fwd_noalloc(const void* q, const void* k, const void* v, const int32_t* col_start,
                               const int32_t* col_end, int32_t n_ranges, int64_t B, int64_t H, int64_t N,
                               int64_t d, float scale, void* out, float* lse, hipStream_t stream) {
    const fm::FwdArgs a = fwd_args(q, k, v, col_start, col_end, n_ranges, B, H, N, d, scale, out, lse, stream);
    const int st = fwd_check(a);
    if (st != FM_OK) return st;
    // (no split key ranges here: they need arrival counters that start at zero)
    const fm::FwdPlan p = fm::fwd_plan(a, g_single_launch == 1, g_split_keys == 1, false, g_row_slices);
    if (p.total() > (size_t)FM_NOALLOC_SCRATCH_BYTES) return FM_ERR_TOO_LARGE;
    void* ws = nullptr;
    FM_HIP(scratch_address(&ws));
    FM_HIP(fm::fwd_launch(a, p, ws, nullptr, g_schedule_mode == 1, nullptr, nullptr));
    return FM_OK;
}

}  // extern "C"

namespace {

// The backward pass; per_head: one interval set per head ([B][H][n_ranges][N]).
int attn_bwd_impl(const void* q, const void* k, const void* v, const void* out, const void* dout, const float* lse,
                  const int32_t* col_start, const int32_t* col_end, int32_t n_ranges, int64_t B, int64_t H, int64_t N,
                  int64_t d, float scale, float* dq, float* dk, float* dv, hipStream_t stream, bool per_head) {
    // ---- host-side checks, before any HIP call
    if (q == nullptr || k == nullptr || v == nullptr || out == nullptr || dout == nullptr || lse == nullptr ||
        col_start == nullptr || col_end == nullptr || dq == nullptr || dk == nullptr || dv == nullptr)
        return FM_ERR_INVALID_ARG;
    if (n_ranges < 1 || n_ranges > fm::kMaxRanges) return FM_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || N < 1 || N > kMaxAttnN) return FM_ERR_INVALID_ARG;
    if (d != 64 && d != 128) return FM_ERR_UNSUPPORTED;
    if (!(scale > 0.f) || !isfinite(scale)) return FM_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) || !aligned(dout, 16) ||
        !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) || !aligned(lse, 4) || !aligned(col_start, 4) ||
        !aligned(col_end, 4))
        return FM_ERR_INVALID_ARG;
    const int64_t n_q = (N + fm::kBr - 1) / fm::kBr;
    const int64_t n_qc = (N + fm::kBwdRows - 1) / fm::kBwdRows;
    const int64_t n_kb = (N + fm::kBwdKeys - 1) / fm::kBwdKeys;
    const int64_t n_sets = per_head ? H : 1;   // interval sets per batch element
    if (B * H * n_qc >= (int64_t(1) << 31) || B * n_sets * n_ranges * N >= (int64_t(1) << 40))
        return FM_ERR_INVALID_ARG;

    // ---- workspace: meta_q[Mq][n] | work_q | order_q | meta_c[Mc][n] | kvr[Mk] | work_k | pieces[Mp] |
    // pslot[Mp] | pwork[Mp] | order_k[Mp] | splits | D[B H N] | partial sums of split key blocks
    const int64_t Mq = n_sets * B * n_q, Mc = n_sets * B * n_qc, Mk = n_sets * B * n_kb;
    const int64_t Lp = fm::bwd_piece_entries(B * n_kb, (int)n_sets), Mp = n_sets * Lp;
    auto al = [](size_t x) { return (x + 255) & ~size_t(255); };
    const size_t o_work_q = al((size_t)(Mq * n_ranges) * sizeof(fm::TileMeta));
    const size_t o_order_q = o_work_q + al((size_t)Mq * 4);
    const size_t o_meta_c = o_order_q + al((size_t)Mq * 4);
    const size_t o_kvr = o_meta_c + al((size_t)(Mc * n_ranges) * sizeof(fm::TileMeta));
    const size_t o_work_k = o_kvr + al((size_t)Mk * sizeof(int4));
    const size_t o_pieces = o_work_k + al((size_t)Mk * 4);
    const size_t o_pslot = o_pieces + al((size_t)Mp * sizeof(int4));
    const size_t o_pwork = o_pslot + al((size_t)Mp * 4);
    const size_t o_order_k = o_pwork + al((size_t)Mp * 4);
    const size_t o_splits = o_order_k + al((size_t)Mp * 4);
    const size_t o_dd = o_splits + al((size_t)(1 + fm::kBwdExtraPieces) * sizeof(int4));
    const size_t o_part = o_dd + al((size_t)(B * H * N) * sizeof(float));
    const size_t part_floats = n_sets == 1 ? (size_t)fm::kBwdExtraPieces * H * fm::kBwdKeys * d * 2 : 0;
    const int64_t n_kv = (N + fm::kBc - 1) / fm::kBc;
    // scheduler scratch of the two orders (they run at the same time, on two streams)
    const int64_t sched_q_ints = fm::schedule_scratch_ints(Mq, B * n_q, fm::schedule_shift(Mq), (int)n_kv);
    const int64_t sched_k_ints = fm::schedule_scratch_ints(Mp, Lp, 0, (int)n_qc);
    const size_t o_sched = o_part + al(part_floats * sizeof(float));
    const size_t o_sched_k = o_sched + al((size_t)sched_q_ints * sizeof(int32_t));
    const size_t total = o_sched_k + al((size_t)sched_k_ints * sizeof(int32_t));
    // The dQ chain and the dK/dV chain read the same inputs and write
    // different outputs.  Where the dK/dV grid runs a few rounds on the 256
    // CUs, the dQ chain goes to a second stream, forked after D and joined
    // before the return, so that it fills the CUs that the dK/dV grid's last
    // round leaves idle (C2 -6 %).  A long grid has no such tail and the two
    // kernels then only contend for the L2 (C5 +1.5 %), and on a tiny call the
    // fork and join cost more than they save (C1 +6 %).
    const int64_t dkdv_groups = H * Lp;
    const bool two_streams = dkdv_groups >= 2 * 256 && dkdv_groups <= 24 * 256;
    void* ws = nullptr;
    std::unique_lock<std::mutex> ws_hold;       // held until the last launch below is queued
    SideStream side{stream, nullptr, nullptr};
    FM_HIP(get_workspace(stream, total, &ws, ws_hold, nullptr, two_streams ? &side : nullptr));
    char* w = static_cast<char*>(ws);
    auto* meta_q = reinterpret_cast<fm::TileMeta*>(w);
    auto* work_q = reinterpret_cast<int32_t*>(w + o_work_q);
    auto* order_q = reinterpret_cast<int32_t*>(w + o_order_q);
    auto* meta_c = reinterpret_cast<fm::TileMeta*>(w + o_meta_c);
    auto* kvr = reinterpret_cast<int4*>(w + o_kvr);
    auto* work_k = reinterpret_cast<int32_t*>(w + o_work_k);
    auto* pieces = reinterpret_cast<int4*>(w + o_pieces);
    auto* pslot = reinterpret_cast<int32_t*>(w + o_pslot);
    auto* pwork = reinterpret_cast<int32_t*>(w + o_pwork);
    auto* order_k = reinterpret_cast<int32_t*>(w + o_order_k);
    auto* splits = reinterpret_cast<int4*>(w + o_splits);
    auto* dd = reinterpret_cast<float*>(w + o_dd);
    auto* part = reinterpret_cast<float*>(w + o_part);
    auto* sched_q = reinterpret_cast<int32_t*>(w + o_sched);
    auto* sched_k = reinterpret_cast<int32_t*>(w + o_sched_k);

    FM_HIP(fm::launch_bwd_rowdot(out, dout, B * H * N, d, dd, stream));
    // Small problems whose key blocks cannot split (no block sees more query
    // chunks than the smallest piece holds, so the split would leave every
    // block whole): one launch prepares both kernels' records, the dQ kernel
    // runs in natural order and no reduction follows.  Same results.
    const int min_chunks = g_bwd_min_chunks > 0 ? g_bwd_min_chunks : (1 << 30);
    if (g_bwd_fused_prep == 1 && !two_streams && n_qc <= min_chunks && Mc <= fm::kBwdFusedMaxChunks) {
        FM_HIP(fm::launch_bwd_prep_fused(col_start, col_end, n_ranges, B, N, (int)n_sets, meta_q, meta_c, pieces, pslot,
                                         order_k, stream));
        FM_HIP(fm::launch_bwd_dq(q, k, v, dout, lse, dd, col_start, col_end, n_ranges, meta_q, nullptr, B, H, N, d,
                                 scale, dq, stream, (int)n_sets));
        FM_HIP(fm::launch_bwd_dkdv(q, k, v, dout, lse, dd, col_start, col_end, n_ranges, meta_c, pieces, pslot,
                                   order_k, B, H, N, d, scale, dk, dv, part, stream, (int)n_sets));
        return FM_OK;
    }
    if (two_streams) {
        FM_HIP(hipEventRecord(side.fork, stream));
        FM_HIP(hipStreamWaitEvent(side.stream, side.fork, 0));
    }
#define FM_TRY(call)                           \
    do {                                       \
        const hipError_t e_ = (call);          \
        if (e_ != hipSuccess) return e_;       \
    } while (0)
    // dQ: the forward's query blocks, key blocks and longest-first order
    const hipError_t e_q = [&]() -> hipError_t {
        if (Mq <= fm::kPrepSmallMax) {
            FM_TRY(fm::launch_prep_small(col_start, col_end, n_ranges, B, N, fm::kBr, fm::kBc, meta_q, work_q,
                                         order_q, side.stream, (int)n_sets));
        } else {
            FM_TRY(fm::launch_preprocess(col_start, col_end, n_ranges, B, N, fm::kBr, fm::kBc, meta_q, work_q,
                                         nullptr, side.stream, (int)n_sets));
            FM_TRY(fm::launch_schedule(work_q, Mq, order_q, side.stream, B * n_q, fm::schedule_shift(Mq), (int)n_kv,
                                       sched_q));
        }
        return fm::launch_bwd_dq(q, k, v, dout, lse, dd, col_start, col_end, n_ranges, meta_q, order_q, B, H, N, d,
                                 scale, dq, side.stream, (int)n_sets);
    }();
    // (recorded and waited for whatever happened above, so that nothing
    // queued on the second stream outlives the call's stream order)
    const hipError_t e_join = two_streams ? hipEventRecord(side.join, side.stream) : hipSuccess;
    // dK, dV: query chunks per key block, long key blocks split into pieces,
    // pieces longest first (within each set)
    const hipError_t e_k = [&]() -> hipError_t {
        FM_TRY(fm::launch_preprocess(col_start, col_end, n_ranges, B, N, fm::kBwdRows, fm::kBwdKeys, meta_c,
                                     nullptr, nullptr, stream, (int)n_sets));
        FM_TRY(fm::launch_kv_ranges(meta_c, n_ranges, B, N, kvr, work_k, stream, (int)n_sets));
        FM_TRY(fm::launch_bwd_split(kvr, B * n_kb, (int)n_sets, min_chunks, pieces, pslot, pwork, splits, stream));
        FM_TRY(fm::launch_schedule(pwork, Mp, order_k, stream, Lp, 0, (int)n_qc, sched_k));
        FM_TRY(fm::launch_bwd_dkdv(q, k, v, dout, lse, dd, col_start, col_end, n_ranges, meta_c, pieces, pslot,
                                   order_k, B, H, N, d, scale, dk, dv, part, stream, (int)n_sets));
        if (n_sets == 1) FM_TRY(fm::launch_bwd_reduce(splits, part, H, N, d, n_kb, dk, dv, stream));
        return hipSuccess;
    }();
#undef FM_TRY
    const hipError_t e_wait = !two_streams ? hipSuccess
                              : e_join == hipSuccess ? hipStreamWaitEvent(stream, side.join, 0)
                                                     : e_join;
    FM_HIP(e_q);
    FM_HIP(e_join);
    FM_HIP(e_k);
    FM_HIP(e_wait);
    return FM_OK;
}

}  // namespace

extern "C" {

FM_API int fm_attn_bwd_multi(const void* q, const void* k, const void* v, const void* out, const void* dout,
                             const float* lse, const int32_t* col_start, const int32_t* col_end, int32_t n_ranges,
                             int64_t B, int64_t H, int64_t N, int64_t d, float scale, float* dq, float* dk,
                             float* dv, hipStream_t stream) {
    return attn_bwd_impl(q, k, v, out, dout, lse, col_start, col_end, n_ranges, B, H, N, d, scale, dq, dk, dv, stream,
                         false);
}

FM_API int fm_attn_bwd_per_head(const void* q, const void* k, const void* v, const void* out, const void* dout,
                                const float* lse, const int32_t* col_start, const int32_t* col_end,
                                int32_t n_ranges, int64_t B, int64_t H, int64_t N, int64_t d, float scale,
                                float* dq, float* dk, float* dv, hipStream_t stream) {
    return attn_bwd_impl(q, k, v, out, dout, lse, col_start, col_end, n_ranges, B, H, N, d, scale, dq, dk, dv, stream,
                         true);
}


FM_API int fm_attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
                       const float* lse, const int32_t* col_start, const int32_t* col_end, int64_t B, int64_t H,
                       int64_t N, int64_t d, float scale, float* dq, float* dk, float* dv, hipStream_t stream) {
    return fm_attn_bwd_multi(q, k, v, out, dout, lse, col_start, col_end, 1, B, H, N, d, scale, dq, dk, dv, stream);
}

}  // extern "C"
