// C ABI of libmuon: the launch sequence of one Muon step (planning is in
// plan.cpp), the AdamW entry points, timing and the test hooks.
//
// One call of muon_step_batched enqueues, on the caller's stream:
//   the descriptor-table upload: ceil(table bytes / 16 KB) launches; the
//     table holds one 216-byte descriptor per matrix plus the prefix arrays,
//     so about one launch per 70 matrices;
//   momentum: one launch per elementwise tile kind in use (at most 3);
//   norm finalize: one launch;
//   ns_steps x {gram, poly, update}: one grouped launch per size class in use
//     (at most 3) and phase, plus a reduce launch after a K-split Gram; with
//     more than one class in use, the classes other than the large one go on
//     the handle's second stream, forked from the caller's stream after the
//     norms and joined back into it before the apply (an event each);
//   apply: one launch per elementwise tile kind in use.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <new>
#include <numeric>
#include <vector>

#include "muon_internal.h"
#include "plan.h"

using namespace muon;

namespace {

constexpr float kMuonA = 3.4445f, kMuonB = -4.7750f, kMuonC = 2.0315f;

}  // namespace

struct TimedLaunch {
    int phase;
    hipEvent_t start, stop;
};

struct muon_context {
    int device = 0;
    float* scratch = nullptr;  // this device's copy of `scratch` (below), device address
    int cus_per_xcd = 32;  // compute units per XCD (tile rounds)
    // second stream (default priority) for the Newton-Schulz launches of the
    // size classes other than the large one, forked from and joined back into
    // the caller's stream with two events
    hipStream_t side = nullptr;
    hipEvent_t fork = nullptr, join = nullptr;
    std::vector<char> table;  // host image of the descriptor table (reused)
    bool profiling = false;
    std::vector<TimedLaunch> timed;     // recorded since the last collect
    std::vector<hipEvent_t> event_pool;  // timing events ready for reuse
};

// Device scratch of the allocation-free entry point adamw_step_clipped_noalloc:
// the per-chunk partial sums of squares (one per kAdamwChunk elements) and,
// 256 bytes after the last of them, the clip scale.  Each device holds its
// own copy for the life of the process.  In host code `scratch` names a
// host-side stand-in, not device memory: kernels get the address that
// hipGetSymbolAddress returns for the current device (resolve_scratch), never
// the name itself.
constexpr int kScratchBlocks = 1 << 18;              // 2^30 elements of AdamW tensors
constexpr int kScratchFloats = kScratchBlocks + 64;  // + the scale, on its own 256 bytes
static __device__ __align__(256) float scratch[kScratchFloats];

namespace {

std::mutex g_scratch_mu;
std::vector<float*> g_scratch_addr;  // by device ordinal; null until resolved

// Device address of `scratch` on `device`, which must be the current device.
// Resolved once per device and kept.
hipError_t resolve_scratch(int device, float** out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if ((int)g_scratch_addr.size() <= device) g_scratch_addr.resize(device + 1, nullptr);
    if (!g_scratch_addr[device]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[device] = static_cast<float*>(p);
    }
    *out = g_scratch_addr[device];
    return hipSuccess;
}

}  // namespace

namespace {

struct DeviceGuard {
    int prev = -1;
    bool changed = false;
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev) == hipSuccess && prev != dev) {
            changed = hipSetDevice(dev) == hipSuccess;
        }
    }
    ~DeviceGuard() {
        if (changed) (void)hipSetDevice(prev);
    }
};

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

bool finite(float v) { return isfinite(v) != 0; }

size_t elem_bytes(int32_t dt) { return dt == MUON_BF16 ? 2 : 4; }
bool valid_dtype(int32_t dt) { return dt == MUON_F32 || dt == MUON_BF16; }

muon_status hip_status(hipError_t e) { return e == hipSuccess ? MUON_OK : MUON_ERR_HIP; }

hipEvent_t take_event(muon_context* h) {
    if (!h->event_pool.empty()) {
        hipEvent_t e = h->event_pool.back();
        h->event_pool.pop_back();
        return e;
    }
    // timing only: no system-scope fence (its cache writeback would slow the
    // launches being timed); the host reads nothing but the timestamps
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
}

// Runs `launch` (a callable returning hipError_t); when profiling, brackets it
// with two timing events on stream s.
template <class F>
hipError_t timed(muon_context* h, int phase, hipStream_t s, F&& launch) {
    if (!h->profiling) return launch();
    TimedLaunch t{phase, take_event(h), take_event(h)};
    if (!t.start || !t.stop) return hipErrorOutOfMemory;
    hipError_t e = hipEventRecord(t.start, s);
    if (e == hipSuccess) e = launch();
    if (e == hipSuccess) e = hipEventRecord(t.stop, s);
    h->timed.push_back(t);
    return e;
}

}  // namespace

extern "C" {

const char* muon_status_str(muon_status s) {
    switch (s) {
        case MUON_OK: return "ok";
        case MUON_ERR_INVALID_ARG: return "invalid argument";
        case MUON_ERR_UNSUPPORTED_DEVICE: return "unsupported device (gfx950 required)";
        case MUON_ERR_WORKSPACE: return "workspace missing or too small";
        case MUON_ERR_OVERLAP: return "param/grad/momentum/update ranges overlap";
        case MUON_ERR_HIP: return "HIP runtime error";
        case MUON_ERR_UNALIGNED: return "pointer not aligned to its element size";
        case MUON_ERR_SCRATCH: return "problem larger than the fixed device scratch of the allocation-free entry point";
    }
    return "unknown status";
}

muon_status muon_init(int device, muon_handle* out) {
    if (!out) return MUON_ERR_INVALID_ARG;
    *out = nullptr;
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count)
        return MUON_ERR_UNSUPPORTED_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return MUON_ERR_HIP;
    if (strncmp(prop.gcnArchName, "gfx950", 6) != 0) return MUON_ERR_UNSUPPORTED_DEVICE;
    DeviceGuard g(device);
    muon_context* h = new (std::nothrow) muon_context();
    if (!h) return MUON_ERR_HIP;
    h->device = device;
    h->cus_per_xcd = prop.multiProcessorCount >= 8 ? prop.multiProcessorCount / 8 : 1;
    if (resolve_scratch(device, &h->scratch) != hipSuccess ||
        hipStreamCreateWithFlags(&h->side, hipStreamNonBlocking) != hipSuccess ||
        hipEventCreateWithFlags(&h->fork, hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&h->join, hipEventDisableTiming) != hipSuccess) {
        if (h->join) (void)hipEventDestroy(h->join);
        if (h->fork) (void)hipEventDestroy(h->fork);
        if (h->side) (void)hipStreamDestroy(h->side);
        delete h;
        return MUON_ERR_HIP;
    }
    *out = h;
    return MUON_OK;
}

muon_status muon_destroy(muon_handle h) {
    if (!h) return MUON_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    for (TimedLaunch& t : h->timed) {
        (void)hipEventSynchronize(t.stop);
        h->event_pool.push_back(t.start);
        h->event_pool.push_back(t.stop);
    }
    for (hipEvent_t e : h->event_pool) (void)hipEventDestroy(e);
    (void)hipStreamSynchronize(h->side);
    (void)hipEventDestroy(h->join);
    (void)hipEventDestroy(h->fork);
    (void)hipStreamDestroy(h->side);
    delete h;
    return MUON_OK;
}

muon_status muon_workspace_size(muon_handle h, const muon_matrix* mats, int n,
                                const muon_hparams* hp, size_t* bytes) {
    if (!h || !bytes) return MUON_ERR_INVALID_ARG;
    Plan P;
    muon_status st = make_plan(mats, n, hp, false, 0, h->cus_per_xcd, P);
    if (st != MUON_OK) return st;
    *bytes = P.total;
    return MUON_OK;
}

muon_status muon_step_batched(muon_handle h, const muon_matrix* mats, int n,
                              const muon_hparams* hp, void* workspace, size_t workspace_bytes,
                              void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    const uintptr_t ws = reinterpret_cast<uintptr_t>(workspace);
    if (!workspace || ws % 256) return MUON_ERR_WORKSPACE;
    Plan P;
    muon_status st = make_plan(mats, n, hp, true, ws, h->cus_per_xcd, P);
    if (st != MUON_OK) return st;
    if (workspace_bytes < P.total) return MUON_ERR_WORKSPACE;

    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);

    // descriptor table + prefixes: built on the host, carried to the
    // workspace in kernel arguments.  Nothing waits on the host and nothing
    // refers to host memory after the call, so the step can be captured in a
    // graph and replayed.
    table_image(P, h->table);
    if (launch_table_upload(h->table.data(), P.table_bytes, workspace, s) != hipSuccess)
        return MUON_ERR_HIP;

    const MatDesc* dd = reinterpret_cast<const MatDesc*>(workspace);
    EwGroups eg;  // elementwise kernels: all matrices, by tile kind
    for (int kind = 0; kind < kNumEwKinds; ++kind) {
        eg.prefix[kind] = reinterpret_cast<const int32_t*>(ws + P.off_pek[kind]);
        eg.tiles[kind] = P.total_ek[kind];
    }
    Prefix pc[kNumClasses];
    for (int c = 0; c < kNumClasses; ++c) {
        pc[c].gram = reinterpret_cast<const int32_t*>(ws + P.cls[c].off_pgram);
        pc[c].tri = reinterpret_cast<const int32_t*>(ws + P.cls[c].off_ptri);
        pc[c].upd = reinterpret_cast<const int32_t*>(ws + P.cls[c].off_pupd);
    }

    hipError_t e = timed(h, 0, s, [&] { return launch_momentum(dd, n, eg, hp->momentum, hp->nesterov, s); });
    if (e == hipSuccess) e = timed(h, 1, s, [&] { return launch_norm_finalize(dd, n, hp->eps, s); });
    // The Newton-Schulz launches of different size classes read and write
    // disjoint buffers.  With more than one class in use, every class but the
    // large one runs on the handle's second stream, forked after the norms and
    // joined before the apply: their short launches then use compute units
    // that the large class's launches leave idle in their partial rounds.
    int used = 0;
    for (int c = 0; c < kNumClasses; ++c) used += P.cls[c].count > 0 ? 1 : 0;
    const int primary = P.cls[kLarge].count > 0 ? kLarge : P.cls[kSmall].count > 0 ? kSmall : kF32;
    const bool forked = used > 1;
    hipStream_t cs[kNumClasses];
    for (int c = 0; c < kNumClasses; ++c) cs[c] = (forked && c != primary) ? h->side : s;
    if (e == hipSuccess && forked) {
        e = hipEventRecord(h->fork, s);
        if (e == hipSuccess) e = hipStreamWaitEvent(h->side, h->fork, 0);
    }
    for (int it = 0; it < hp->ns_steps && e == hipSuccess; ++it) {
        float a = kMuonA, b = kMuonB, c = kMuonC;
        if (hp->coeffs) {
            a = hp->coeffs[3 * it];
            b = hp->coeffs[3 * it + 1];
            c = hp->coeffs[3 * it + 2];
        }
        for (int k = 0; k < kNumClasses && e == hipSuccess; ++k) {
            const ClassPlan& C = P.cls[k];
            if (C.count == 0) continue;
            const MatDesc* dc = dd + C.first;
            const hipStream_t sk = cs[k];
            // from the second iteration on, a fused class's Gram parts come
            // from the previous update's strips: only the reduce remains
            if (!(C.fuse_gram && it > 0))
                e = timed(h, 2, sk, [&] {
                    return k == kF32 ? launch_gram_f32(dc, C.count, pc[k], C.total_gram, it, C.kmax_n, sk)
                                     : launch_gram_bf16(dc, C.count, pc[k], C.xs_gram, it, k == kSmall,
                                                        C.gram_split, sk);
                });
            if (e == hipSuccess && C.gram_split)
                e = timed(h, 2, sk, [&] {
                    return launch_gram_reduce_bf16(dc, C.count, pc[k], C.total_tri, it, k == kSmall, sk);
                });
        }
        for (int k = 0; k < kNumClasses && e == hipSuccess; ++k) {
            const ClassPlan& C = P.cls[k];
            // a class updated in strips forms B inside the strips
            if (C.count == 0 || C.strip > 0) continue;
            const MatDesc* dc = dd + C.first;
            const hipStream_t sk = cs[k];
            Prefix pp = pc[k];  // the polynomial's own tiling (128-tiles when poly_small)
            pp.tri = reinterpret_cast<const int32_t*>(ws + C.off_ppoly);
            e = timed(h, 3, sk, [&] {
                return k == kF32 ? launch_poly_f32(dc, C.count, pp, C.total_poly, C.kmax_m, b, c, sk)
                                 : launch_poly_bf16(dc, C.count, pp, C.xs_poly, a, b, c,
                                                    k == kSmall || C.poly_small, sk);
            });
        }
        for (int k = 0; k < kNumClasses && e == hipSuccess; ++k) {
            const ClassPlan& C = P.cls[k];
            if (C.count == 0) continue;
            const MatDesc* dc = dd + C.first;
            const hipStream_t sk = cs[k];
            e = timed(h, 4, sk, [&] {
                if (k == kF32) return launch_update_f32(dc, C.count, pc[k], C.total_upd, it, C.kmax_m, a, sk);
                if (C.strip > 0)
                    return launch_update_strip_bf16(dc, C.count,
                                                    reinterpret_cast<const int32_t*>(ws + C.off_pstrip),
                                                    C.xs_strip, it, C.strip,
                                                    C.fuse_gram && it + 1 < hp->ns_steps, C.stream,
                                                    C.fuse_apply && it + 1 == hp->ns_steps, a, b, c,
                                                    1.f - hp->lr * hp->weight_decay, hp->lr, sk);
                return launch_update_bf16(dc, C.count, pc[k], C.xs_upd, it, k == kSmall, sk);
            });
        }
    }
    if (forked) {
        // joined whatever happened above, so that a capture of the caller's
        // stream never ends with the second stream still forked
        hipError_t ej = hipEventRecord(h->join, h->side);
        if (ej == hipSuccess) ej = hipStreamWaitEvent(s, h->join, 0);
        if (e == hipSuccess) e = ej;
    }
    // a class that applied in its last update is every matrix of the call
    if (e == hipSuccess && !P.cls[kSmall].fuse_apply)
        e = timed(h, 5, s, [&] {
            return launch_apply(dd, n, eg, hp->ns_steps & 1, hp->lr, hp->weight_decay, hp->qk_tau, s);
        });
    return hip_status(e);
}

}  // extern "C"

namespace {

muon_status check_adamw(const adamw_tensor* ts, int n, const adamw_hparams* hp) {
    if (!ts || n < 1 || !hp) return MUON_ERR_INVALID_ARG;
    if (hp->step < 1) return MUON_ERR_INVALID_ARG;
    if (!finite(hp->lr) || !finite(hp->beta1) || !finite(hp->beta2) || !finite(hp->eps) ||
        !finite(hp->weight_decay))
        return MUON_ERR_INVALID_ARG;
    if (hp->beta1 < 0.f || hp->beta1 >= 1.f || hp->beta2 < 0.f || hp->beta2 >= 1.f)
        return MUON_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i) {
        const adamw_tensor& t = ts[i];
        if (t.numel < 0 || !valid_dtype(t.param_dtype) || !valid_dtype(t.grad_dtype))
            return MUON_ERR_INVALID_ARG;
        if (t.numel == 0) continue;
        if (!t.param || !t.grad || !t.exp_avg || !t.exp_avg_sq) return MUON_ERR_INVALID_ARG;
        if (reinterpret_cast<uintptr_t>(t.param) % elem_bytes(t.param_dtype) ||
            reinterpret_cast<uintptr_t>(t.grad) % elem_bytes(t.grad_dtype) ||
            reinterpret_cast<uintptr_t>(t.exp_avg) % 4 || reinterpret_cast<uintptr_t>(t.exp_avg_sq) % 4)
            return MUON_ERR_UNALIGNED;
        if ((t.numel + kAdamwChunk - 1) / kAdamwChunk > INT32_MAX / 4) return MUON_ERR_INVALID_ARG;
    }
    return MUON_OK;
}

// Split the tensor list into launch groups (at most kAdamwGroup tensors and
// INT32_MAX/4 blocks each) and call fn(group, blocks, first_block) per group.
template <class F>
hipError_t for_each_adamw_group(const adamw_tensor* ts, int n, F&& fn) {
    AdamwGroup grp;
    memset(&grp, 0, sizeof(grp));
    int64_t blocks = 0, first = 0;
    auto flush = [&]() -> hipError_t {
        if (grp.count == 0) return hipSuccess;
        grp.block_prefix[grp.count] = (int32_t)blocks;
        hipError_t e = fn(grp, (int)blocks, (int)first);
        first += blocks;
        memset(&grp, 0, sizeof(grp));
        blocks = 0;
        return e;
    };
    for (int i = 0; i < n; ++i) {
        const adamw_tensor& t = ts[i];
        if (t.numel == 0) continue;
        const int64_t nb = (t.numel + kAdamwChunk - 1) / kAdamwChunk;
        if (grp.count == kAdamwGroup || blocks + nb > INT32_MAX / 4) {
            hipError_t e = flush();
            if (e != hipSuccess) return e;
        }
        const int k = grp.count++;
        grp.param[k] = t.param;
        grp.grad[k] = t.grad;
        grp.m[k] = t.exp_avg;
        grp.v[k] = t.exp_avg_sq;
        grp.numel[k] = t.numel;
        grp.block_prefix[k] = (int32_t)blocks;
        grp.param_bf16[k] = t.param_dtype == MUON_BF16;
        grp.grad_bf16[k] = t.grad_dtype == MUON_BF16;
        const size_t pv = 4 * elem_bytes(t.param_dtype), gv = 4 * elem_bytes(t.grad_dtype);
        grp.vec4[k] = reinterpret_cast<uintptr_t>(t.param) % pv == 0 &&
                      reinterpret_cast<uintptr_t>(t.grad) % gv == 0 &&
                      reinterpret_cast<uintptr_t>(t.exp_avg) % 16 == 0 &&
                      reinterpret_cast<uintptr_t>(t.exp_avg_sq) % 16 == 0;
        blocks += nb;
    }
    return flush();
}

int64_t adamw_total_blocks(const adamw_tensor* ts, int n) {
    int64_t b = 0;
    for (int i = 0; i < n; ++i)
        if (ts[i].numel > 0) b += (ts[i].numel + kAdamwChunk - 1) / kAdamwChunk;
    return b;
}

hipError_t adamw_launch_all(muon_context* h, const adamw_tensor* ts, int n, const adamw_hparams* hp,
                            const float* gscale, hipStream_t s) {
    const double bc1 = 1.0 - pow((double)hp->beta1, (double)hp->step);
    const double bc2 = 1.0 - pow((double)hp->beta2, (double)hp->step);
    return for_each_adamw_group(ts, n, [&](const AdamwGroup& grp, int blocks, int) {
        return timed(h, 6, s, [&] {
            return launch_adamw(grp, blocks, hp->lr, hp->beta1, hp->beta2, hp->eps,
                                hp->weight_decay, (float)bc1, (float)bc2, gscale, s);
        });
    });
}

}  // namespace

extern "C" {

muon_status adamw_step(muon_handle h, const adamw_tensor* ts, int n, const adamw_hparams* hp,
                       void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    muon_status st = check_adamw(ts, n, hp);
    if (st != MUON_OK) return st;
    DeviceGuard g(h->device);
    return hip_status(adamw_launch_all(h, ts, n, hp, nullptr, reinterpret_cast<hipStream_t>(stream)));
}

muon_status adamw_workspace_size(muon_handle h, const adamw_tensor* ts, int n, size_t* bytes) {
    if (!h || !bytes || !ts || n < 1) return MUON_ERR_INVALID_ARG;
    for (int i = 0; i < n; ++i)
        if (ts[i].numel < 0) return MUON_ERR_INVALID_ARG;
    *bytes = align_up((size_t)adamw_total_blocks(ts, n) * 4, 256) + 256;
    return MUON_OK;
}

}  // extern "C"

namespace {

// Clipped AdamW with the partial sums at `partials` (nblocks floats) and the
// scale at `scale`, both device memory; arguments already validated.  Every
// partial is written by the sum-of-squares launch before the finalize reads
// it, and the scale by the finalize before AdamW reads it: nothing needs to
// start at zero.
hipError_t clipped_launches(muon_context* h, const adamw_tensor* ts, int n, const adamw_hparams* hp,
                            float max_norm, float* norm_out, float* partials, float* scale,
                            int64_t nblocks, hipStream_t s) {
    hipError_t e = hipSuccess;
    if (nblocks > 0) {
        e = for_each_adamw_group(ts, n, [&](const AdamwGroup& grp, int blocks, int first) {
            return timed(h, 6, s, [&] { return launch_adamw_sumsq(grp, blocks, partials, first, s); });
        });
    }
    if (e == hipSuccess)
        e = timed(h, 6, s, [&] {
            return launch_clip_finalize(partials, (int)nblocks, max_norm, scale, norm_out, s);
        });
    if (e == hipSuccess) e = adamw_launch_all(h, ts, n, hp, scale, s);
    return e;
}

muon_status check_clipped(muon_handle h, const adamw_tensor* ts, int n, const adamw_hparams* hp,
                          float max_norm, float* norm_out) {
    if (!h) return MUON_ERR_INVALID_ARG;
    muon_status st = check_adamw(ts, n, hp);
    if (st != MUON_OK) return st;
    if (!finite(max_norm) || max_norm <= 0.f) return MUON_ERR_INVALID_ARG;
    if (norm_out && reinterpret_cast<uintptr_t>(norm_out) % 4) return MUON_ERR_UNALIGNED;
    if (adamw_total_blocks(ts, n) > INT32_MAX) return MUON_ERR_INVALID_ARG;
    return MUON_OK;
}

}  // namespace

extern "C" {

muon_status adamw_step_clipped(muon_handle h, const adamw_tensor* ts, int n,
                               const adamw_hparams* hp, float max_norm, float* norm_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
    muon_status st = check_clipped(h, ts, n, hp, max_norm, norm_out);
    if (st != MUON_OK) return st;
    const int64_t nblocks = adamw_total_blocks(ts, n);
    const size_t need = align_up((size_t)nblocks * 4, 256) + 256;
    const uintptr_t ws = reinterpret_cast<uintptr_t>(workspace);
    if (!workspace || ws % 256 || workspace_bytes < need) return MUON_ERR_WORKSPACE;
    DeviceGuard g(h->device);
    float* partials = reinterpret_cast<float*>(workspace);
    float* scale = reinterpret_cast<float*>(ws + align_up((size_t)nblocks * 4, 256));
    return hip_status(clipped_launches(h, ts, n, hp, max_norm, norm_out, partials, scale, nblocks,
                                       reinterpret_cast<hipStream_t>(stream)));
}

muon_status adamw_step_clipped_noalloc(muon_handle h, const adamw_tensor* ts, int n,
                                       const adamw_hparams* hp, float max_norm, float* norm_out,
                                       void* stream) {
    muon_status st = check_clipped(h, ts, n, hp, max_norm, norm_out);
    if (st != MUON_OK) return st;
    const int64_t nblocks = adamw_total_blocks(ts, n);
    if (nblocks > kScratchBlocks) return MUON_ERR_SCRATCH;
    if (!h->scratch) return MUON_ERR_HIP;
    DeviceGuard g(h->device);
    // the device address resolved at init, never the host-side name
    float* partials = h->scratch;
    float* scale = h->scratch + kScratchBlocks;
    return hip_status(clipped_launches(h, ts, n, hp, max_norm, norm_out, partials, scale, nblocks,
                                       reinterpret_cast<hipStream_t>(stream)));
}

muon_status muon_profile_enable(muon_handle h, int enable) {
    if (!h) return MUON_ERR_INVALID_ARG;
    h->profiling = enable != 0;
    return MUON_OK;
}

muon_status muon_profile_collect(muon_handle h, muon_phase_times* out) {
    if (!h || !out) return MUON_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    memset(out, 0, sizeof(*out));
    muon_status st = MUON_OK;
    for (TimedLaunch& t : h->timed) {
        // launches may sit on the handle's second stream as well as on the
        // caller's: wait for each one's own stop event
        float ms = 0.f;
        if (st == MUON_OK && hipEventSynchronize(t.stop) != hipSuccess) st = MUON_ERR_HIP;
        if (st == MUON_OK && hipEventElapsedTime(&ms, t.start, t.stop) != hipSuccess) st = MUON_ERR_HIP;
        if (t.phase >= 0 && t.phase < MUON_NUM_PHASES) {
            out->ms[t.phase] += ms;
            out->launches[t.phase] += 1;
        }
        h->event_pool.push_back(t.start);
        h->event_pool.push_back(t.stop);
    }
    h->timed.clear();
    return st;
}

static muon_status check_single(muon_handle h, int64_t m, int64_t n) {
    if (!h) return MUON_ERR_INVALID_ARG;
    const int T = kClassTile[kLarge];
    if (m < T || n < T || m % T || n % T || m > kMaxDim || n > kMaxDim) return MUON_ERR_INVALID_ARG;
    return MUON_OK;
}

muon_status muon_test_split_matrices(muon_handle h, const muon_matrix* mats, int n,
                                     const muon_hparams* hp, int32_t* out, int cap, int* count) {
    if (!h || !count || cap < 0 || (cap > 0 && !out)) return MUON_ERR_INVALID_ARG;
    Plan P;
    muon_status st = make_plan(mats, n, hp, false, 0, h->cus_per_xcd, P);
    if (st != MUON_OK) return st;
    const std::vector<int> idx = split_matrices(P);
    *count = (int)idx.size();
    for (int i = 0; i < cap && i < (int)idx.size(); ++i) out[i] = idx[i];
    return MUON_OK;
}

muon_status muon_test_gram_bf16(muon_handle h, const void* X, void* A, int64_t m, int64_t n,
                                int64_t ldx, int64_t lda, float s2, void* stream) {
    muon_status st = check_single(h, m, n);
    if (st != MUON_OK) return st;
    if (!X || !A || ldx < n || lda < m || ldx % 8 || lda % 8) return MUON_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    return hip_status(launch_gram_bf16_single(X, A, (int)m, (int)n, ldx, lda, s2, h->cus_per_xcd,
                                              reinterpret_cast<hipStream_t>(stream)));
}

muon_status muon_test_poly_bf16(muon_handle h, const void* A, void* B, int64_t m, int64_t lda,
                                float a, float b, float c, void* stream) {
    muon_status st = check_single(h, m, m);
    if (st != MUON_OK) return st;
    if (!A || !B || lda < m || lda % 8) return MUON_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    return hip_status(launch_poly_bf16_single(A, B, (int)m, lda, a, b, c, h->cus_per_xcd,
                                              reinterpret_cast<hipStream_t>(stream)));
}

muon_status muon_test_update_bf16(muon_handle h, const void* X, const void* B, void* Xo,
                                  int64_t m, int64_t n, int64_t ldx, int64_t ldb, float s,
                                  void* stream) {
    muon_status st = check_single(h, m, n);
    if (st != MUON_OK) return st;
    if (!X || !B || !Xo || ldx < n || ldb < m || ldx % 8 || ldb % 8) return MUON_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    return hip_status(launch_update_bf16_single(X, B, Xo, (int)m, (int)n, ldx, ldb, s,
                                                h->cus_per_xcd,
                                                reinterpret_cast<hipStream_t>(stream)));
}

}  // extern "C"
