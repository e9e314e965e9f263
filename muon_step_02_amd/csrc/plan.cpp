// Host-side planning of one Muon step (see plan.h).
#include "plan.h"

#include <math.h>
#include <string.h>

#include <algorithm>
#include <numeric>

// Bounds checks of the planner's own indexing: on in the sanitizer build of
// this file, compiled out in the library.
#ifdef MUON_PLAN_CHECKS
#include <stdio.h>
#include <stdlib.h>
#define PLAN_CHECK(c)                                                           \
    do {                                                                        \
        if (!(c)) {                                                             \
            fprintf(stderr, "plan check failed: %s (%s:%d)\n", #c, __FILE__, __LINE__); \
            abort();                                                            \
        }                                                                       \
    } while (0)
#else
#define PLAN_CHECK(c) ((void)0)
#endif

namespace muon {

namespace {

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

int size_class(const muon_matrix& m, bool ns_f32) {
    const int64_t s = std::min(m.rows, m.cols);
    if (ns_f32 || s <= kTinyF32) return kF32;
    return s <= kSmallBf16 ? kSmall : kLarge;
}

// index k of the largest prefix[k] <= t (prefix[0] = 0 <= t < prefix[count])
int owner(const std::vector<int32_t>& prefix, int32_t t) {
    PLAN_CHECK(!prefix.empty() && prefix.front() <= t && t < prefix.back());
    return (int)(std::upper_bound(prefix.begin(), prefix.end(), t) - prefix.begin()) - 1;
}

}  // namespace

double shape_multiplier(int mode, int64_t rows, int64_t cols) {
    const double r = (double)rows, c = (double)cols;
    switch (mode) {
        case MUON_SCALE_MOONLIGHT: return 0.2 * sqrt(r > c ? r : c);
        case MUON_SCALE_JORDAN: return sqrt(r / c > 1.0 ? r / c : 1.0);
        case MUON_SCALE_BERNSTEIN: return sqrt(r / c);
        default: return 1.0;
    }
}

XcdSplit xcd_split(const int32_t* ntiles, const int64_t* weight, int n, int cus, int quarters,
                   int interleaved) {
    XcdSplit xs;
    const int C = cus > 0 ? cus : 1;
    xs.cus = C;
    xs.interleaved = interleaved ? 1 : 0;
    int64_t total_t = 0;
    for (int k = 0; k < n; ++k) total_t += ntiles[k];
    // interleaved: the full rounds are dealt chunk by chunk; the tiles after
    // them, like every tile in range mode, are cut into 8 ranges of equal work
    const int64_t R = interleaved ? total_t / (8 * C) : 0;
    const int64_t skip = R * 8 * C;
    xs.rounds = (int32_t)R;
    int64_t total_w = 0;
    {
        int64_t cum_t = 0;
        for (int k = 0; k < n; ++k) {
            const int64_t first = std::max<int64_t>(skip, cum_t), last = cum_t + ntiles[k];
            if (last > first) total_w += (last - first) * (weight[k] > 0 ? weight[k] : 1);
            cum_t = last;
        }
    }
    // boundary x: first tile whose preceding work (after `skip`) reaches x/8 of the total
    xs.b[0] = (int32_t)skip;
    int x = 1;
    int64_t cum_w = 0, cum_t = 0;
    for (int k = 0; k < n && x < 8; ++k) {
        const int64_t w = weight[k] > 0 ? weight[k] : 1;
        const int64_t first = std::max<int64_t>(skip, cum_t), last = cum_t + ntiles[k];
        cum_t = last;
        if (last <= first) continue;
        const int64_t cnt = last - first;
        const int64_t end_w = cum_w + cnt * w;
        while (x < 8 && end_w * 8 >= (int64_t)x * total_w) {
            // smallest t in [0, cnt] with (cum_w + t*w) * 8 >= x * total_w
            const int64_t need = (int64_t)x * total_w - cum_w * 8;
            int64_t t = need <= 0 ? 0 : (need + 8 * w - 1) / (8 * w);
            if (t > cnt) t = cnt;
            PLAN_CHECK(x >= 1 && x < 9);
            xs.b[x++] = (int32_t)(first + t);
        }
        cum_w = end_w;
    }
    while (x < 9) xs.b[x++] = (int32_t)total_t;
    xs.b[8] = (int32_t)total_t;
    xs.per = 0;
    for (int i = 0; i < 8; ++i) {
        if (xs.b[i + 1] < xs.b[i]) xs.b[i + 1] = xs.b[i];
        const int T = xs.b[i + 1] - xs.b[i];
        // last round of R tiles on C CUs: as 4R quarter tiles when R <= C/2
        const int Rr = T % C;
        xs.sub[i] = (quarters && Rr > 0 && 2 * Rr <= C) ? Rr : 0;
        const int tasks = xs.rounds * C + T + 3 * xs.sub[i];
        if (tasks > xs.per) xs.per = tasks;
    }
    return xs;
}

std::vector<int32_t> gram_splits(const std::vector<int32_t>& tiles,
                                 const std::vector<int32_t>& slabs, int cus_total) {
    const size_t n = tiles.size();
    std::vector<int32_t> S(n, 1);
    int64_t total = 0, work = 0, longest = 0;
    for (size_t k = 0; k < n; ++k) {
        total += tiles[k];
        work += (int64_t)tiles[k] * slabs[k];
        longest = std::max<int64_t>(longest, slabs[k]);
    }
    // Split only a launch whose tiles fill at most a quarter of the slots:
    // with every compute unit busy a tile's K loop runs about twice as slowly
    // per slab as in a launch that leaves most of the chip idle, and the
    // reduce launch re-reads the partial tiles, so fewer than four parts per
    // tile do not pay (measured on the d=1024 block: 70 tiles of up to 64
    // slabs, split or not, both about 52 us).
    if (total == 0 || 4 * total > cus_total) return S;
    // parts of at least `len` slabs each
    auto parts = [&](size_t k, int64_t len) {
        return (int32_t)std::max<int64_t>(1, std::min<int64_t>(kMaxSplit, slabs[k] / len));
    };
    int64_t len = std::max<int64_t>(kMinSplitSlabs, (work + cus_total - 1) / cus_total);
    for (; len < longest; ++len) {
        int64_t tasks = 0;
        for (size_t k = 0; k < n; ++k) tasks += (int64_t)tiles[k] * parts(k, len);
        if (tasks <= cus_total) break;
    }
    for (size_t k = 0; k < n; ++k) S[k] = parts(k, len);
    return S;
}

// Workspace plan for one call.  Matrices are split into the size classes of
// layout.h, each with its own GEMM tile and padding and its own prefix arrays
// of Gram/polynomial and update tiles; the descriptor table holds kLarge
// first, then kSmall, then kF32, each by descending Newton-Schulz work, so
// the longest tiles are dispatched first.  The elementwise kernels run over
// all matrices, one launch per tile kind, each with a prefix array of its own.
muon_status make_plan(const muon_matrix* mats, int n, const muon_hparams* hp, bool need_ptrs,
                      uintptr_t ws, int cus, Plan& P) {
    P = Plan{};  // nothing carries over from an earlier plan in P
    if (!mats || n < 1) return MUON_ERR_INVALID_ARG;
    muon_status st = check_hparams(hp);
    if (st != MUON_OK) return st;
    for (int i = 0; i < n; ++i) {
        st = check_matrix(mats[i], need_ptrs);
        if (st != MUON_OK) return st;
    }
    const bool ns_f32 = hp->ns_dtype == MUON_F32;

    std::vector<int> cls_of(n);
    int count[kNumClasses] = {0, 0, 0};
    for (int i = 0; i < n; ++i) {
        cls_of[i] = size_class(mats[i], ns_f32);
        ++count[cls_of[i]];
    }
    auto work = [&](int i) {
        const double m = (double)std::min(mats[i].rows, mats[i].cols);
        const double nn = (double)std::max(mats[i].rows, mats[i].cols);
        return m * m * nn;
    };
    P.order.resize(n);
    std::iota(P.order.begin(), P.order.end(), 0);
    std::stable_sort(P.order.begin(), P.order.end(), [&](int a, int b) {
        if (cls_of[a] != cls_of[b]) return cls_of[a] < cls_of[b];
        return work(a) > work(b);
    });

    P.d.assign(n, MatDesc{});
    P.pew.assign(n + 1, 0);
    for (int kind = 0; kind < kNumEwKinds; ++kind) P.pek[kind].assign(n + 1, 0);
    int first = 0;
    for (int c = 0; c < kNumClasses; ++c) {
        ClassPlan& C = P.cls[c];
        C.first = first;
        C.count = count[c];
        first += count[c];
        C.pgram.assign(C.count + 1, 0);
        C.ptri.assign(C.count + 1, 0);
        C.ppoly.assign(C.count + 1, 0);
        C.pupd.assign(C.count + 1, 0);
    }
    int64_t tew = 0, tek[kNumEwKinds] = {0, 0, 0};
    int64_t tgram[kNumClasses] = {0, 0, 0}, tupd[kNumClasses] = {0, 0, 0};
    for (int k = 0; k < n; ++k) {
        const muon_matrix& m = mats[P.order[k]];
        const int c = cls_of[P.order[k]];
        PLAN_CHECK(k >= P.cls[c].first && k < P.cls[c].first + P.cls[c].count);
        const int64_t pad = kClassPad[c];
        const int64_t tile = kClassTile[c];
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
        d.cls = c;
        d.transposed = m.rows > m.cols ? 1 : 0;
        d.rows_pad = (int32_t)pad_to(m.rows, pad);
        d.cols_pad = (int32_t)pad_to(m.cols, pad);
        d.mp = d.transposed ? d.cols_pad : d.rows_pad;
        d.np = d.transposed ? d.rows_pad : d.cols_pad;
        int kind;
        if (c == kF32) {
            kind = kEwF32;
            d.ew_th = d.ew_tw = kEwTile;
        } else if (!d.transposed && d.cols_pad % 256 == 0) {
            // the bf16 iteration reads Y as it is: streaming tiles
            kind = kEwStream;
            d.ew_th = 16;
            d.ew_tw = 256;
        } else {
            kind = kEwTrans;
            d.ew_th = kTrTH;
            d.ew_tw = kTrTW;
        }
        PLAN_CHECK(d.rows_pad % d.ew_th == 0 && d.cols_pad % d.ew_tw == 0);
        d.ew_tiles_c = d.cols_pad / d.ew_tw;
        d.ew_tiles = (d.rows_pad / d.ew_th) * d.ew_tiles_c;
        d.vec4 = need_ptrs && m.cols % 4 == 0 &&
                 aligned_rows(m.param, m.ld_param, elem_bytes(m.param_dtype)) &&
                 aligned_rows(m.grad, m.ld_grad, elem_bytes(m.grad_dtype)) &&
                 aligned_rows(m.momentum, m.ld_mom, 4);
        d.scale = (float)(shape_multiplier(hp->scale_mode, m.rows, m.cols) * (double)hp->extra_scale);
        d.gram_split = 1;
        const int64_t Ts = d.mp / tile;
        // the bf16 kernels compute the symmetric products on the lower
        // triangle of tiles; the fp32 ones compute every tile
        const int64_t gram_tiles = c == kF32 ? Ts * Ts : Ts * (Ts + 1) / 2;
        const int64_t upd_tiles = (d.mp / tile) * (d.np / tile);
        tew += d.ew_tiles;
        tek[kind] += d.ew_tiles;
        tgram[c] += gram_tiles;
        tupd[c] += upd_tiles;
        if (tew > INT32_MAX || tgram[c] > INT32_MAX / 2 || tupd[c] > INT32_MAX / 2)
            return MUON_ERR_INVALID_ARG;
        P.pew[k + 1] = (int32_t)tew;
        for (int kk = 0; kk < kNumEwKinds; ++kk) P.pek[kk][k + 1] = (int32_t)tek[kk];
        const int kc = k - P.cls[c].first;
        P.cls[c].kmax_n = std::max<int>(P.cls[c].kmax_n, d.np);
        P.cls[c].kmax_m = std::max<int>(P.cls[c].kmax_m, d.mp);
        P.cls[c].ptri[kc + 1] = (int32_t)tgram[c];
        P.cls[c].pupd[kc + 1] = (int32_t)tupd[c];
    }
    for (int kind = 0; kind < kNumEwKinds; ++kind) P.total_ek[kind] = (int)tek[kind];
    for (int c = 0; c < kNumClasses; ++c) {
        ClassPlan& C = P.cls[c];
        C.total_tri = (int)tgram[c];
        C.total_upd = (int)tupd[c];
        std::vector<int32_t> tg(C.count), tu(C.count), slabs(C.count);
        for (int k = 0; k < C.count; ++k) {
            tg[k] = C.ptri[k + 1] - C.ptri[k];
            tu[k] = C.pupd[k + 1] - C.pupd[k];
            slabs[k] = P.d[C.first + k].np / kGemmBK;
        }
        // Gram tasks: its tiles, or tiles * parts when the launch is K-split
        std::vector<int32_t> S(C.count, 1);
        // compute slots: two 128-tile workgroups fit one compute unit's LDS
        const int slots = 8 * cus * (c == kSmall ? 2 : 1);
        if (c != kF32 && C.count > 0) S = gram_splits(tg, slabs, slots);
        // The small class's update in strips: as many consecutive column
        // tiles per workgroup as it takes to fill the compute units once,
        // when that is at least two (one tile per workgroup runs the copy
        // latency and the epilogue back to back).  Alone in the call, the
        // class streams its strips at one workgroup per compute unit, and a
        // K-split Gram takes as many parts per matrix as the matrix has
        // strips (at most kMaxSplit, each of at least kMinSplitSlabs slabs),
        // so that from the second iteration on
        // the update's strips form the parts.  Beside another class (on the
        // other stream) it runs two workgroups per compute unit, and the
        // strips form the Gram parts when their count per matrix already
        // equals the split's.
        C.strip = 0;
        C.stream = false;
        C.fuse_apply = false;
        C.fuse_gram = false;
        C.pstrip.assign(C.count + 1, 0);
        std::vector<int32_t> ts;
        if (c == kSmall && C.count > 0) {
            const bool alone = P.cls[kLarge].count == 0 && P.cls[kF32].count == 0;
            const int64_t wgs = (alone ? 8 : 16) * (int64_t)cus;
            int64_t upd = 0;
            for (int k = 0; k < C.count; ++k) upd += tu[k];
            const int64_t L = (upd + wgs - 1) / wgs;
            if (L >= 2) {
                C.strip = (int)L;
                C.stream = alone;
                C.fuse_apply = alone && need_ptrs;
                for (int k = 0; k < C.count && C.fuse_apply; ++k) {
                    const MatDesc& d = P.d[C.first + k];
                    C.fuse_apply = !d.transposed && d.rows == kClassPad[kSmall] && d.rows == d.mp &&
                                   d.cols == d.np && d.param_dtype == MUON_F32 && d.vec4 &&
                                   !d.update_out && !d.qk_smax &&
                                   ((d.rows - 1) * d.ld_param + d.cols) * 4 < ((int64_t)1 << 31);
                }
                ts.resize(C.count);
                bool split = false, several = false, fits = true, same = true;
                for (int k = 0; k < C.count; ++k) {
                    ts[k] = (int32_t)((tu[k] + L - 1) / L);
                    C.pstrip[k + 1] = C.pstrip[k] + ts[k];
                    split = split || S[k] > 1;
                    several = several || ts[k] > 1;
                    fits = fits && ts[k] <= kMaxSplit && (int64_t)ts[k] * kMinSplitSlabs <= slabs[k];
                    same = same && ts[k] == S[k];
                }
                C.total_strips = C.pstrip[C.count];
                if (alone) {
                    C.fuse_gram = split && several && fits;
                    if (C.fuse_gram)
                        for (int k = 0; k < C.count; ++k) S[k] = ts[k];
                } else {
                    C.fuse_gram = split && same;
                }
            }
        }
        int64_t tasks = 0;
        for (int k = 0; k < C.count; ++k) {
            P.d[C.first + k].gram_split = S[k];
            C.gram_split = C.gram_split || S[k] > 1;
        }
        for (int k = 0; k < C.count; ++k) {
            tasks += (int64_t)tg[k] * (C.gram_split ? S[k] : 1);
            if (tasks > INT32_MAX / 2) return MUON_ERR_INVALID_ARG;
            C.pgram[k + 1] = (int32_t)tasks;
        }
        C.total_gram = (int)tasks;
        // The polynomial of a large-class launch whose 256-tiles fill at most
        // half the compute units (every XCD would run them as quarter tiles,
        // one workgroup per compute unit, four slots per tile) runs on the
        // triangle of 128-tiles instead, two workgroups per compute unit, when
        // those fit one round: the 128-triangle skips the upper quarter of
        // each diagonal tile.  (d=1024 block: 70 tiles of 256 as 280 quarter
        // slots over 256 CUs against 252 tiles of 128 in one round.)
        std::vector<int32_t> tp(tg);
        if (c == kLarge && C.count > 0 && 2 * (int64_t)C.total_tri <= 8 * (int64_t)cus) {
            int64_t t128 = 0;
            for (int k = 0; k < C.count; ++k) {
                const int64_t T = P.d[C.first + k].mp / kClassTile[kSmall];
                t128 += T * (T + 1) / 2;
            }
            C.poly_small = t128 <= 2 * 8 * (int64_t)cus;
        }
        if (C.poly_small)
            for (int k = 0; k < C.count; ++k) {
                const int64_t T = P.d[C.first + k].mp / kClassTile[kSmall];
                tp[k] = (int32_t)(T * (T + 1) / 2);
            }
        for (int k = 0; k < C.count; ++k) C.ppoly[k + 1] = C.ppoly[k] + tp[k];
        C.total_poly = C.ppoly[C.count];
        if (c == kF32 || C.count == 0) continue;
        // tile work = k-steps: the Gram runs over n' (a part of it when
        // split), the polynomial and the update over m'
        std::vector<int32_t> tk(C.count);
        std::vector<int64_t> wn(C.count), wm(C.count);
        for (int k = 0; k < C.count; ++k) {
            tk[k] = C.pgram[k + 1] - C.pgram[k];
            wn[k] = C.gram_split ? (slabs[k] + S[k] - 1) / S[k] : P.d[C.first + k].np;
            wm[k] = P.d[C.first + k].mp;
        }
        // quarter tiles for the short last round: 256-tile class only, and not
        // in a K-split Gram (its tasks fit one round)
        const int quarters = c == kLarge ? 1 : 0;
        // Gram and update tiles in interleaved rounds, polynomial tiles in
        // ranges (each measured faster that way on the 8 x 4096^2 and the
        // 192-matrix MoE workloads)
        C.xs_gram = xcd_split(tk.data(), wn.data(), C.count, cus, C.gram_split ? 0 : quarters, 1);
        C.xs_poly = xcd_split(tp.data(), wm.data(), C.count, cus, C.poly_small ? 0 : quarters, 0);
        C.xs_upd = xcd_split(tu.data(), wm.data(), C.count, cus, quarters, 1);
        if (C.strip > 0) {
            std::vector<int64_t> wsz(C.count, C.strip);
            C.xs_strip = xcd_split(ts.data(), wsz.data(), C.count, cus, 0, 0);
        }
    }

    size_t off = align_up((size_t)n * sizeof(MatDesc), 256);
    for (int kind = 0; kind < kNumEwKinds; ++kind) {
        P.off_pek[kind] = off;
        off = align_up(off + (size_t)(n + 1) * 4, 256);
    }
    for (int c = 0; c < kNumClasses; ++c) {
        P.cls[c].off_pgram = off;
        off = align_up(off + (size_t)(P.cls[c].count + 1) * 4, 256);
        P.cls[c].off_ptri = off;
        off = align_up(off + (size_t)(P.cls[c].count + 1) * 4, 256);
        P.cls[c].off_ppoly = off;
        off = align_up(off + (size_t)(P.cls[c].count + 1) * 4, 256);
        P.cls[c].off_pstrip = off;
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
        const size_t es = d.cls == kF32 ? 4 : 2;
        const size_t xb = (size_t)d.mp * (size_t)d.np * es;
        const size_t ab = (size_t)d.mp * (size_t)d.mp * es;
        // X^T is kept only by the fp32 iteration; the bf16 update reads X
        // k-major directly
        d.xt[0] = d.xt[1] = nullptr;
        void** bufs[4] = {&d.x[0], &d.x[1], &d.xt[0], &d.xt[1]};
        const int nbufs = d.cls == kF32 ? 4 : 2;
        for (int i = 0; i < nbufs; ++i) {
            *bufs[i] = reinterpret_cast<void*>(ws + off);
            off = align_up(off + xb, 256);
        }
        d.a = reinterpret_cast<void*>(ws + off);
        off = align_up(off + ab, 256);
        d.b = reinterpret_cast<void*>(ws + off);
        off = align_up(off + ab, 256);
        d.partials = reinterpret_cast<float*>(ws + P.off_partials) + P.pew[k];
        d.inv_norm = reinterpret_cast<float*>(ws + P.off_invnorm) + k;
        d.gram_part = nullptr;
        const ClassPlan& C = P.cls[d.cls];
        if (C.gram_split) {
            const int kc = k - C.first;
            const size_t tile = (size_t)kClassTile[d.cls];
            const size_t tasks = (size_t)(C.pgram[kc + 1] - C.pgram[kc]);
            d.gram_part = reinterpret_cast<float*>(ws + off);
            off = align_up(off + tasks * tile * tile * 4, 256);
        }
    }
    P.total = off;
    return MUON_OK;
}

void table_image(const Plan& P, std::vector<char>& out) {
    const int n = (int)P.d.size();
    out.assign(P.table_bytes, 0);
    char* hb = out.data();
    PLAN_CHECK((size_t)n * sizeof(MatDesc) <= P.table_bytes);
    memcpy(hb, P.d.data(), (size_t)n * sizeof(MatDesc));
    for (int kind = 0; kind < kNumEwKinds; ++kind) {
        PLAN_CHECK(P.off_pek[kind] + (size_t)(n + 1) * 4 <= P.table_bytes);
        memcpy(hb + P.off_pek[kind], P.pek[kind].data(), (size_t)(n + 1) * 4);
    }
    for (const ClassPlan& c : P.cls) {
        PLAN_CHECK(c.off_pgram + (size_t)(c.count + 1) * 4 <= P.table_bytes);
        PLAN_CHECK(c.off_pupd + (size_t)(c.count + 1) * 4 <= P.table_bytes);
        PLAN_CHECK(c.off_ptri + (size_t)(c.count + 1) * 4 <= P.table_bytes);
        PLAN_CHECK(c.off_ppoly + (size_t)(c.count + 1) * 4 <= P.table_bytes);
        memcpy(hb + c.off_pgram, c.pgram.data(), (size_t)(c.count + 1) * 4);
        memcpy(hb + c.off_ptri, c.ptri.data(), (size_t)(c.count + 1) * 4);
        memcpy(hb + c.off_ppoly, c.ppoly.data(), (size_t)(c.count + 1) * 4);
        if (!c.pstrip.empty()) {
            PLAN_CHECK(c.off_pstrip + (size_t)(c.count + 1) * 4 <= P.table_bytes);
            memcpy(hb + c.off_pstrip, c.pstrip.data(), (size_t)(c.count + 1) * 4);
        }
        memcpy(hb + c.off_pupd, c.pupd.data(), (size_t)(c.count + 1) * 4);
    }
}

std::vector<int> split_matrices(const Plan& P) {
    std::vector<int> out;
    for (int c = kLarge; c <= kSmall; ++c) {
        const ClassPlan& C = P.cls[c];
        if (C.count == 0) continue;
        // the update launch deals strips when the class runs it in strips
        const XcdSplit* splits[3] = {&C.xs_gram, &C.xs_poly, C.strip > 0 ? &C.xs_strip : &C.xs_upd};
        const std::vector<int32_t>* prefixes[3] = {&C.pgram, &C.ppoly, C.strip > 0 ? &C.pstrip : &C.pupd};
        for (int s = 0; s < 3; ++s) {
            const XcdSplit& xs = *splits[s];
            const std::vector<int32_t>& pre = *prefixes[s];
            auto mark = [&](int32_t t) { out.push_back(P.order[C.first + owner(pre, t)]); };
            // interleaved rounds: the chunks that start and end each round
            for (int r = 0; r < xs.rounds; ++r)
                for (int x = 0; x < 8; ++x) {
                    const int32_t c0 = (8 * r + x) * xs.cus;
                    if (r == 0 || r == xs.rounds - 1 || x == 0 || x == 7) {
                        mark(c0);
                        mark(c0 + xs.cus - 1);
                    }
                }
            for (int x = 0; x < 8; ++x) {
                if (xs.b[x] == xs.b[x + 1]) continue;
                mark(xs.b[x]);
                mark(xs.b[x + 1] - 1);
                for (int32_t t = xs.b[x + 1] - xs.sub[x]; t < xs.b[x + 1]; ++t) mark(t);
            }
        }
    }
    std::sort(out.begin(), out.end());
    out.erase(std::unique(out.begin(), out.end()), out.end());
    return out;
}

}  // namespace muon
