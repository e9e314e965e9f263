// C ABI of libmuon: validation, workspace planning, descriptor upload and the
// launch sequence of one Muon step; the AdamW entry point.
//
// One call of muon_step_batched enqueues, on the caller's stream:
//   the descriptor-table upload (kernel arguments -> workspace, 2 KB a launch),
//   momentum (one launch per elementwise tile kind in use), norm finalize,
//   ns_steps x {gram, poly, update} (one grouped launch per size class in use),
//   apply (one launch per elementwise tile kind in use).
// The launch count does not depend on the number of matrices.  Matrices are
// ordered by descending Newton-Schulz work in the table so the biggest tiles
// are dispatched first.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <new>
#include <numeric>
#include <vector>

#include "muon_internal.h"

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
    int cus_per_xcd = 32;  // compute units per XCD (tile rounds)
    std::vector<char> table;  // host image of the descriptor table (reused)
    bool profiling = false;
    std::vector<TimedLaunch> timed;     // recorded since the last collect
    std::vector<hipEvent_t> event_pool;  // timing events ready for reuse
};

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
inline int64_t pad_to(int64_t v, int64_t p) { return (v + p - 1) / p * p; }

bool finite(float v) { return isfinite(v) != 0; }

size_t elem_bytes(int32_t dt) { return dt == MUON_BF16 ? 2 : 4; }
bool valid_dtype(int32_t dt) { return dt == MUON_F32 || dt == MUON_BF16; }

struct Range {
    uintptr_t lo, hi;
};
Range span_of(const void* p, int64_t rows, int64_t cols, int64_t ld, size_t es) {
    const uintptr_t b = reinterpret_cast<uintptr_t>(p);
    return Range{b, b + (size_t)((rows - 1) * ld + cols) * es};
}
bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi; }

double shape_multiplier(int mode, int64_t rows, int64_t cols) {
    const double r = (double)rows, c = (double)cols;
    switch (mode) {
        case MUON_SCALE_MOONLIGHT: return 0.2 * sqrt(r > c ? r : c);
        case MUON_SCALE_JORDAN: return sqrt(r / c > 1.0 ? r / c : 1.0);
        case MUON_SCALE_BERNSTEIN: return sqrt(r / c);
        default: return 1.0;
    }
}

muon_status check_hparams(const muon_hparams* hp) {
    if (!hp) return MUON_ERR_INVALID_ARG;
    if (hp->ns_steps < 1 || hp->ns_steps > 1000) return MUON_ERR_INVALID_ARG;
    if (!valid_dtype(hp->ns_dtype)) return MUON_ERR_INVALID_ARG;
    if (hp->scale_mode < MUON_SCALE_MOONLIGHT || hp->scale_mode > MUON_SCALE_NONE)
        return MUON_ERR_INVALID_ARG;
    if (hp->nesterov != 0 && hp->nesterov != 1) return MUON_ERR_INVALID_ARG;
    if (!finite(hp->lr) || !finite(hp->momentum) || !finite(hp->weight_decay) ||
        !finite(hp->eps) || !finite(hp->extra_scale))
        return MUON_ERR_INVALID_ARG;
    if (hp->eps < 0.f) return MUON_ERR_INVALID_ARG;
    if (!finite(hp->qk_tau) || hp->qk_tau < 0.f) return MUON_ERR_INVALID_ARG;
    if (hp->coeffs) {
        for (int i = 0; i < 3 * hp->ns_steps; ++i)
            if (!finite(hp->coeffs[i])) return MUON_ERR_INVALID_ARG;
    }
    return MUON_OK;
}

constexpr int64_t kMaxDim = 1 << 20;
static_assert(kSmallBf16 % kTrTH == 0 && kSmallBf16 % kTrTW == 0,
              "transposing elementwise tiles must divide every bf16 padding");
static_assert(kPadF32 % kEwTile == 0, "fp32 elementwise tiles must divide the fp32 padding");

muon_status check_matrix(const muon_matrix& m, bool need_ptrs) {
    if (m.rows < 1 || m.cols < 1 || m.rows > kMaxDim || m.cols > kMaxDim) return MUON_ERR_INVALID_ARG;
    if (m.ld_param < m.cols || m.ld_grad < m.cols || m.ld_mom < m.cols) return MUON_ERR_INVALID_ARG;
    if (!valid_dtype(m.param_dtype) || !valid_dtype(m.grad_dtype)) return MUON_ERR_INVALID_ARG;
    if (!need_ptrs) return MUON_OK;
    if (!m.param || !m.grad || !m.momentum) return MUON_ERR_INVALID_ARG;
    if (m.qk_smax && (m.qk_block_rows < 1 || m.qk_block_rows > m.rows)) return MUON_ERR_INVALID_ARG;
    if (m.qk_smax && reinterpret_cast<uintptr_t>(m.qk_smax) % 4) return MUON_ERR_UNALIGNED;
    const size_t pes = elem_bytes(m.param_dtype), ges = elem_bytes(m.grad_dtype);
    if (reinterpret_cast<uintptr_t>(m.param) % pes || reinterpret_cast<uintptr_t>(m.grad) % ges ||
        reinterpret_cast<uintptr_t>(m.momentum) % 4 ||
        (m.update_out && reinterpret_cast<uintptr_t>(m.update_out) % 4) ||
        (m.norm_out && reinterpret_cast<uintptr_t>(m.norm_out) % 4))
        return MUON_ERR_UNALIGNED;
    const Range rp = span_of(m.param, m.rows, m.cols, m.ld_param, pes);
    const Range rg = span_of(m.grad, m.rows, m.cols, m.ld_grad, ges);
    const Range rm = span_of(m.momentum, m.rows, m.cols, m.ld_mom, 4);
    if (overlaps(rp, rg) || overlaps(rp, rm) || overlaps(rg, rm)) return MUON_ERR_OVERLAP;
    if (m.update_out) {
        const Range ru = span_of(m.update_out, m.rows, m.cols, m.cols, 4);
        if (overlaps(ru, rp) || overlaps(ru, rg) || overlaps(ru, rm)) return MUON_ERR_OVERLAP;
    }
    return MUON_OK;
}

bool aligned_rows(const void* p, int64_t ld, size_t es) {
    const size_t vec_bytes = 4 * es;
    return reinterpret_cast<uintptr_t>(p) % vec_bytes == 0 && ld % 4 == 0;
}

// Workspace plan for one call.  Matrices are split into two classes with
// their own GEMM tile size: "large" (256-wide tiles and padding) and, for
// bf16 Newton-Schulz, "small" (short side <= 128: 128-wide tiles and
// padding).  The descriptor table holds the large class first; each class has
// its own prefix arrays of Gram/polynomial and update tiles.  The elementwise
// kernels run over all matrices, one launch per tile kind (streaming, or
// through LDS), each with a prefix array of its own.
struct ClassPlan {
    int first = 0, count = 0;           // descriptor range
    std::vector<int32_t> pgram, pupd;   // count + 1 entries each
    size_t off_pgram = 0, off_pupd = 0;
    int total_gram = 0, total_upd = 0;
    XcdSplit xs_gram, xs_poly, xs_upd;  // per-XCD tile ranges of equal work
};

struct Plan {
    std::vector<MatDesc> d;
    std::vector<int32_t> pew;        // elementwise tiles of all kinds (norm partial offsets)
    std::vector<int32_t> pek[2];     // elementwise tiles by kind (launch prefixes)
    ClassPlan cls[2];  // 0 large, 1 small
    size_t off_pek[2] = {0, 0}, table_bytes = 0;
    size_t off_partials = 0, off_invnorm = 0, total = 0;
    int total_ek[2] = {0, 0};
    int ns_f32 = 0;
};

muon_status make_plan(const muon_matrix* mats, int n, const muon_hparams* hp, bool need_ptrs,
                      uintptr_t ws, int cus, Plan& P) {
    if (!mats || n < 1) return MUON_ERR_INVALID_ARG;
    muon_status st = check_hparams(hp);
    if (st != MUON_OK) return st;
    for (int i = 0; i < n; ++i) {
        st = check_matrix(mats[i], need_ptrs);
        if (st != MUON_OK) return st;
    }
    P.ns_f32 = hp->ns_dtype == MUON_F32;
    const size_t es = P.ns_f32 ? 4 : 2;
    auto is_small = [&](int i) {
        return !P.ns_f32 && std::min(mats[i].rows, mats[i].cols) <= kSmallBf16;
    };

    // order: large class first, each class by descending Newton-Schulz work
    std::vector<int> order(n);
    std::iota(order.begin(), order.end(), 0);
    auto work = [&](int i) {
        const double m = (double)std::min(mats[i].rows, mats[i].cols);
        const double nn = (double)std::max(mats[i].rows, mats[i].cols);
        return m * m * nn;
    };
    std::stable_sort(order.begin(), order.end(), [&](int a, int b) {
        if (is_small(a) != is_small(b)) return !is_small(a);
        return work(a) > work(b);
    });

    P.d.assign(n, MatDesc{});
    P.pew.assign(n + 1, 0);
    P.pek[0].assign(n + 1, 0);
    P.pek[1].assign(n + 1, 0);
    int64_t tew = 0, tek[2] = {0, 0};
    int nsmall = 0;
    for (int i = 0; i < n; ++i) nsmall += is_small(i) ? 1 : 0;
    P.cls[0].first = 0;
    P.cls[0].count = n - nsmall;
    P.cls[1].first = n - nsmall;
    P.cls[1].count = nsmall;
    for (int c = 0; c < 2; ++c) {
        P.cls[c].pgram.assign(P.cls[c].count + 1, 0);
        P.cls[c].pupd.assign(P.cls[c].count + 1, 0);
    }
    int64_t tgram[2] = {0, 0}, tupd[2] = {0, 0};
    for (int k = 0; k < n; ++k) {
        const muon_matrix& m = mats[order[k]];
        const int c = k < P.cls[1].first ? 0 : 1;
        const int64_t pad = P.ns_f32 ? kPadF32 : (c ? kSmallBf16 : kPadBf16);
        const int symT = P.ns_f32 ? kTileF32 : gemm_tile_bf16(c);
        const int updM = P.ns_f32 ? kTileF32 : upd_tile_m_bf16(c);
        const int updN = P.ns_f32 ? kTileF32 : upd_tile_n_bf16(c);
        MatDesc& d = P.d[k];
        d.param = m.param;
        d.grad = m.grad;
        d.mom = m.momentum;
        d.update_out = m.update_out;
        d.norm_out = m.norm_out;
        d.qk_smax = m.qk_smax;
        d.qk_block_rows = m.qk_smax ? m.qk_block_rows : 0;
        d.rows = m.rows;
        d.cols = m.cols;
        d.ld_param = m.ld_param;
        d.ld_grad = m.ld_grad;
        d.ld_mom = m.ld_mom;
        d.param_dtype = m.param_dtype;
        d.grad_dtype = m.grad_dtype;
        d.transposed = m.rows > m.cols ? 1 : 0;
        d.rows_pad = (int32_t)pad_to(m.rows, pad);
        d.cols_pad = (int32_t)pad_to(m.cols, pad);
        d.mp = d.transposed ? d.cols_pad : d.rows_pad;
        d.np = d.transposed ? d.rows_pad : d.cols_pad;
        // 16 x 256 streaming tiles unless Y is also needed transposed (the
        // fp32 iteration keeps X^T; bf16 writes Y^T when rows > cols)
        if (P.ns_f32) {
            d.ew_th = d.ew_tw = kEwTile;
        } else if (!d.transposed && d.cols_pad % 256 == 0) {
            d.ew_th = 16;
            d.ew_tw = 256;
        } else {
            d.ew_th = kTrTH;
            d.ew_tw = kTrTW;
        }
        d.ew_tiles_c = d.cols_pad / d.ew_tw;
        d.ew_tiles = (d.rows_pad / d.ew_th) * d.ew_tiles_c;
        d.vec4 = need_ptrs && m.cols % 4 == 0 &&
                 aligned_rows(m.param, m.ld_param, elem_bytes(m.param_dtype)) &&
                 aligned_rows(m.grad, m.ld_grad, elem_bytes(m.grad_dtype)) &&
                 aligned_rows(m.momentum, m.ld_mom, 4);
        d.scale = (float)(shape_multiplier(hp->scale_mode, m.rows, m.cols) * (double)hp->extra_scale);
        const int64_t Ts = d.mp / symT;
        const int64_t gram_tiles = P.ns_f32 ? Ts * Ts : Ts * (Ts + 1) / 2;
        const int64_t upd_tiles = (d.mp / updM) * (d.np / updN);
        tew += d.ew_tiles;
        tek[d.ew_th == 16 ? 0 : 1] += d.ew_tiles;
        tgram[c] += gram_tiles;
        tupd[c] += upd_tiles;
        if (tew > INT32_MAX || tgram[c] > INT32_MAX / 2 || tupd[c] > INT32_MAX / 2)
            return MUON_ERR_INVALID_ARG;
        P.pew[k + 1] = (int32_t)tew;
        P.pek[0][k + 1] = (int32_t)tek[0];
        P.pek[1][k + 1] = (int32_t)tek[1];
        const int kc = k - P.cls[c].first;
        P.cls[c].pgram[kc + 1] = (int32_t)tgram[c];
        P.cls[c].pupd[kc + 1] = (int32_t)tupd[c];
    }
    P.total_ek[0] = (int)tek[0];
    P.total_ek[1] = (int)tek[1];
    for (int c = 0; c < 2; ++c) {
        ClassPlan& C = P.cls[c];
        C.total_gram = (int)tgram[c];
        C.total_upd = (int)tupd[c];
        // tile work = k-steps: the Gram runs over n', the polynomial and the
        // update over m'
        std::vector<int32_t> tg(C.count), tu(C.count);
        std::vector<int64_t> wn(C.count), wm(C.count);
        for (int k = 0; k < C.count; ++k) {
            tg[k] = C.pgram[k + 1] - C.pgram[k];
            tu[k] = C.pupd[k + 1] - C.pupd[k];
            wn[k] = P.d[C.first + k].np;
            wm[k] = P.d[C.first + k].mp;
        }
        // quarter tiles for the short last round: large bf16 class only
        const int quarters = (!P.ns_f32 && c == 0) ? 1 : 0;
        C.xs_gram = xcd_split(tg.data(), wn.data(), C.count, cus, quarters);
        C.xs_poly = xcd_split(tg.data(), wm.data(), C.count, cus, quarters);
        C.xs_upd = xcd_split(tu.data(), wm.data(), C.count, cus, quarters);
    }

    size_t off = align_up((size_t)n * sizeof(MatDesc), 256);
    for (int kind = 0; kind < 2; ++kind) {
        P.off_pek[kind] = off;
        off = align_up(off + (size_t)(n + 1) * 4, 256);
    }
    for (int c = 0; c < 2; ++c) {
        P.cls[c].off_pgram = off;
        off = align_up(off + (size_t)(P.cls[c].count + 1) * 4, 256);
        P.cls[c].off_pupd = off;
        off = align_up(off + (size_t)(P.cls[c].count + 1) * 4, 256);
    }
    P.table_bytes = off;
    P.off_partials = off;
    off = align_up(off + (size_t)tew * 4, 256);
    P.off_invnorm = off;
    off = align_up(off + (size_t)n * 4, 256);
    for (int k = 0; k < n; ++k) {
        MatDesc& d = P.d[k];
        const size_t xb = (size_t)d.mp * (size_t)d.np * es;
        const size_t ab = (size_t)d.mp * (size_t)d.mp * es;
        // X^T is kept only by the fp32 iteration; the bf16 update reads X
        // k-major directly
        d.xt[0] = d.xt[1] = nullptr;
        void** bufs[4] = {&d.x[0], &d.x[1], &d.xt[0], &d.xt[1]};
        const int nbufs = P.ns_f32 ? 4 : 2;
        for (int i = 0; i < nbufs; ++i) {
            *bufs[i] = reinterpret_cast<void*>(ws + off);
            off = align_up(off + xb, 256);
        }
        d.a = reinterpret_cast<void*>(ws + off);
        off = align_up(off + ab, 256);
        d.b = reinterpret_cast<void*>(ws + off);
        off = align_up(off + ab, 256);
        d.partials = reinterpret_cast<float*>(ws + P.off_partials) + (P.pew[k]);
        d.inv_norm = reinterpret_cast<float*>(ws + P.off_invnorm) + k;
    }
    P.total = off;
    return MUON_OK;
}

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
    h->table.assign(P.table_bytes, 0);
    char* hb = h->table.data();
    memcpy(hb, P.d.data(), (size_t)n * sizeof(MatDesc));
    for (int kind = 0; kind < 2; ++kind)
        memcpy(hb + P.off_pek[kind], P.pek[kind].data(), (size_t)(n + 1) * 4);
    for (const ClassPlan& c : P.cls) {
        memcpy(hb + c.off_pgram, c.pgram.data(), (size_t)(c.count + 1) * 4);
        memcpy(hb + c.off_pupd, c.pupd.data(), (size_t)(c.count + 1) * 4);
    }
    if (launch_table_upload(hb, P.table_bytes, workspace, s) != hipSuccess) return MUON_ERR_HIP;

    const MatDesc* dd = reinterpret_cast<const MatDesc*>(workspace);
    EwGroups eg;  // elementwise kernels: all matrices, by tile kind
    for (int kind = 0; kind < 2; ++kind) {
        eg.prefix[kind] = reinterpret_cast<const int32_t*>(ws + P.off_pek[kind]);
        eg.tiles[kind] = P.total_ek[kind];
    }
    Prefix pc[2];
    for (int c = 0; c < 2; ++c) {
        pc[c].gram = reinterpret_cast<const int32_t*>(ws + P.cls[c].off_pgram);
        pc[c].upd = reinterpret_cast<const int32_t*>(ws + P.cls[c].off_pupd);
    }

    hipError_t e = timed(h, 0, s, [&] {
        return launch_momentum(dd, n, eg, hp->momentum, hp->nesterov, P.ns_f32, s);
    });
    if (e == hipSuccess) e = timed(h, 1, s, [&] { return launch_norm_finalize(dd, n, hp->eps, s); });
    for (int it = 0; it < hp->ns_steps && e == hipSuccess; ++it) {
        float a = kMuonA, b = kMuonB, c = kMuonC;
        if (hp->coeffs) {
            a = hp->coeffs[3 * it];
            b = hp->coeffs[3 * it + 1];
            c = hp->coeffs[3 * it + 2];
        }
        if (P.ns_f32) {
            const ClassPlan& L = P.cls[0];
            e = timed(h, 2, s, [&] { return launch_gram_f32(dd, L.count, pc[0], L.total_gram, it, s); });
            if (e == hipSuccess)
                e = timed(h, 3, s, [&] { return launch_poly_f32(dd, L.count, pc[0], L.total_gram, b, c, s); });
            if (e == hipSuccess)
                e = timed(h, 4, s, [&] { return launch_update_f32(dd, L.count, pc[0], L.total_upd, it, a, s); });
            continue;
        }
        // the two classes' launches of one phase are independent of each other
        for (int k = 0; k < 2 && e == hipSuccess; ++k) {
            const ClassPlan& C = P.cls[k];
            if (C.count == 0) continue;
            const MatDesc* dc = dd + C.first;
            e = timed(h, 2, s, [&] { return launch_gram_bf16(dc, C.count, pc[k], C.xs_gram, it, k, s); });
        }
        for (int k = 0; k < 2 && e == hipSuccess; ++k) {
            const ClassPlan& C = P.cls[k];
            if (C.count == 0) continue;
            const MatDesc* dc = dd + C.first;
            e = timed(h, 3, s, [&] { return launch_poly_bf16(dc, C.count, pc[k], C.xs_poly, a, b, c, k, s); });
        }
        for (int k = 0; k < 2 && e == hipSuccess; ++k) {
            const ClassPlan& C = P.cls[k];
            if (C.count == 0) continue;
            const MatDesc* dc = dd + C.first;
            e = timed(h, 4, s, [&] { return launch_update_bf16(dc, C.count, pc[k], C.xs_upd, it, k, s); });
        }
    }
    if (e == hipSuccess)
        e = timed(h, 5, s, [&] {
            return launch_apply(dd, n, eg, hp->ns_steps & 1, hp->lr, hp->weight_decay,
                                hp->qk_tau, P.ns_f32, s);
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

muon_status adamw_step_clipped(muon_handle h, const adamw_tensor* ts, int n,
                               const adamw_hparams* hp, float max_norm, float* norm_out,
                               void* workspace, size_t workspace_bytes, void* stream) {
    if (!h) return MUON_ERR_INVALID_ARG;
    muon_status st = check_adamw(ts, n, hp);
    if (st != MUON_OK) return st;
    if (!finite(max_norm) || max_norm <= 0.f) return MUON_ERR_INVALID_ARG;
    if (norm_out && reinterpret_cast<uintptr_t>(norm_out) % 4) return MUON_ERR_UNALIGNED;
    const int64_t nblocks = adamw_total_blocks(ts, n);
    const size_t need = align_up((size_t)nblocks * 4, 256) + 256;
    const uintptr_t ws = reinterpret_cast<uintptr_t>(workspace);
    if (!workspace || ws % 256 || workspace_bytes < need) return MUON_ERR_WORKSPACE;
    if (nblocks > INT32_MAX) return MUON_ERR_INVALID_ARG;
    DeviceGuard g(h->device);
    hipStream_t s = reinterpret_cast<hipStream_t>(stream);
    float* partials = reinterpret_cast<float*>(workspace);
    float* scale = reinterpret_cast<float*>(ws + align_up((size_t)nblocks * 4, 256));
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
    return hip_status(e);
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
    if (!h->timed.empty() && hipEventSynchronize(h->timed.back().stop) != hipSuccess) st = MUON_ERR_HIP;
    for (TimedLaunch& t : h->timed) {
        float ms = 0.f;
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
    const int T = gemm_tile_bf16(0);
    if (m < T || n < T || m % T || n % T || m > kMaxDim || n > kMaxDim) return MUON_ERR_INVALID_ARG;
    if (upd_tile_m_bf16(0) != T || n % upd_tile_n_bf16(0)) return MUON_ERR_INVALID_ARG;
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
