// Host check of the Muon step planner (muon_step_02_amd/csrc/plan.cpp), built
// with g++ under AddressSanitizer and UndefinedBehaviorSanitizer and with the
// planner's own bounds checks on (MUON_PLAN_CHECKS).  No device is involved:
// tensor pointers are made-up, non-overlapping addresses.
//
// For thousands of random batches (shapes from 1 x 1 to 2^20 long, ragged,
// strided, mixed dtypes, both Newton-Schulz dtypes) it checks every invariant
// the kernels rely on: the descriptor order is a permutation grouped by size
// class and sorted by work, padded shapes and tile counts follow the class
// rules, every prefix array is the running sum of the per-matrix counts, the
// per-XCD ranges cover each tile once, and every workspace buffer is 256-byte
// aligned, inside the workspace and disjoint from every other.  It also checks
// that invalid inputs are rejected with the documented status.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <random>
#include <vector>

#include "plan.h"

using namespace muon;

static int failures = 0;
#define EXPECT(c)                                                                       \
    do {                                                                                \
        if (!(c)) {                                                                     \
            if (failures < 20) fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, #c); \
            ++failures;                                                                 \
        }                                                                               \
    } while (0)

struct Batch {
    std::vector<muon_matrix> mats;
    muon_hparams hp;
    std::vector<float> coeffs;
};

static int64_t pad_to(int64_t v, int64_t p) { return (v + p - 1) / p * p; }

static Batch random_batch(std::mt19937_64& rng, int n, bool big) {
    Batch b;
    uintptr_t next = (uintptr_t)1 << 40;  // made-up device addresses
    auto take = [&](size_t bytes, size_t align) {
        next = (next + align - 1) / align * align;
        uintptr_t p = next;
        next += bytes + 4096;
        return p;
    };
    auto dim = [&]() -> int64_t {
        switch (rng() % 6) {
            case 0: return 1 + rng() % 8;
            case 1: return 1 + rng() % 64;
            case 2: return 1 + rng() % 300;
            case 3: return 128 * (1 + rng() % 8) + (int64_t)(rng() % 3) - 1;
            case 4: return 256 * (1 + rng() % 16);
            default: return 1 + rng() % 2000;
        }
    };
    for (int i = 0; i < n; ++i) {
        muon_matrix m;
        memset(&m, 0, sizeof(m));
        m.rows = dim();
        m.cols = dim();
        if (big && i == 0) {
            // a 2^20-long row or column
            if (rng() & 1) { m.rows = 1 + rng() % 3; m.cols = kMaxDim; }
            else { m.rows = kMaxDim; m.cols = 1 + rng() % 3; }
        }
        m.param_dtype = rng() % 2 ? MUON_BF16 : MUON_F32;
        m.grad_dtype = rng() % 2 ? MUON_BF16 : MUON_F32;
        m.ld_param = m.cols + (rng() % 4 == 0 ? (int64_t)(rng() % 17) : 0);
        m.ld_grad = m.cols + (rng() % 4 == 0 ? (int64_t)(rng() % 9) : 0);
        m.ld_mom = m.cols + (rng() % 4 == 0 ? (int64_t)(rng() % 5) : 0);
        const size_t pe = m.param_dtype == MUON_BF16 ? 2 : 4, ge = m.grad_dtype == MUON_BF16 ? 2 : 4;
        // some pointers only element-aligned (the kernels' scalar paths)
        const size_t odd = rng() % 3 == 0 ? 1 : 0;
        m.param = (void*)(take((size_t)(m.rows * m.ld_param) * pe, 256) + odd * pe);
        m.grad = (const void*)(take((size_t)(m.rows * m.ld_grad) * ge, 256));
        m.momentum = (float*)take((size_t)(m.rows * m.ld_mom) * 4, 256);
        if (rng() % 3 == 0) m.update_out = (float*)take((size_t)(m.rows * m.cols) * 4, 256);
        if (rng() % 3 == 0) m.norm_out = (float*)take(4, 4);
        if (rng() % 5 == 0) {
            m.qk_block_rows = 1 + (int64_t)(rng() % (uint64_t)m.rows);
            m.qk_smax = (const float*)take((size_t)((m.rows + m.qk_block_rows - 1) / m.qk_block_rows) * 4, 4);
        }
        b.mats.push_back(m);
    }
    memset(&b.hp, 0, sizeof(b.hp));
    b.hp.lr = 2e-4f;
    b.hp.momentum = 0.95f;
    b.hp.weight_decay = 0.1f;
    b.hp.eps = 1e-7f;
    b.hp.extra_scale = 1.f;
    b.hp.nesterov = (int)(rng() % 2);
    b.hp.ns_steps = 1 + (int)(rng() % 6);
    b.hp.ns_dtype = rng() % 4 == 0 ? MUON_F32 : MUON_BF16;
    b.hp.scale_mode = (int)(rng() % 4);
    b.hp.qk_tau = 100.f;
    if (rng() % 3 == 0) {
        b.coeffs.resize(3 * b.hp.ns_steps, 1.f);
        b.hp.coeffs = b.coeffs.data();
    }
    return b;
}

struct Interval {
    uintptr_t lo, hi;
    const char* what;
};

// The kernels' mapping of workgroup b to (tile, quarter), restated for the
// check (gemm_bf16.hip, xcd_task): false means no task.
static bool task_of(const XcdSplit& xs, int b, int& tile, int& quarter) {
    const int x = b & 7;
    int t = b >> 3;
    const int full = xs.rounds * xs.cus;
    if (t < full) {
        const int r = t / xs.cus;
        tile = (8 * r + x) * xs.cus + (t - r * xs.cus);
        quarter = -1;
        return true;
    }
    t -= full;
    const int whole = xs.b[x + 1] - xs.b[x] - xs.sub[x];
    if (t < whole) {
        tile = xs.b[x] + t;
        quarter = -1;
        return true;
    }
    const int u = t - whole;
    if (u >= 4 * xs.sub[x]) return false;
    tile = xs.b[x] + whole + (u >> 2);
    quarter = u & 3;
    return true;
}

// every tile is computed exactly once: by one whole task or by its four
// quarters; no task outside [0, total); the grid covers every task
static void check_split(const XcdSplit& xs, int total, int cus, int quarters) {
    EXPECT(xs.b[8] == total && xs.cus == cus);
    if (!xs.interleaved) EXPECT(xs.b[0] == 0 && xs.rounds == 0);
    else EXPECT(xs.b[0] == xs.rounds * 8 * cus && xs.rounds == total / (8 * cus));
    int per = 0;
    for (int x = 0; x < 8; ++x) {
        const int T = xs.b[x + 1] - xs.b[x];
        EXPECT(T >= 0);
        const int R = T % cus;
        const int want = (quarters && R > 0 && 2 * R <= cus) ? R : 0;
        EXPECT(xs.sub[x] == want);
        per = std::max(per, xs.rounds * cus + T + 3 * xs.sub[x]);
    }
    EXPECT(per == xs.per);
    std::vector<int> whole(total, 0), quarter_mask(total, 0);
    for (int b = 0; b < 8 * std::max(xs.per, 1); ++b) {
        int tile, q;
        if (!task_of(xs, b, tile, q)) continue;
        EXPECT(tile >= 0 && tile < total);
        if (tile < 0 || tile >= total) continue;
        if (q < 0) ++whole[tile];
        else {
            EXPECT(!(quarter_mask[tile] & (1 << q)));
            quarter_mask[tile] |= 1 << q;
        }
    }
    for (int t = 0; t < total; ++t)
        EXPECT((whole[t] == 1 && quarter_mask[t] == 0) || (whole[t] == 0 && quarter_mask[t] == 15));
}

static void check_plan(const Batch& b, const Plan& P, uintptr_t ws, int cus) {
    const int n = (int)b.mats.size();
    const bool f32 = b.hp.ns_dtype == MUON_F32;
    EXPECT((int)P.d.size() == n && (int)P.order.size() == n);
    std::vector<int> seen(n, 0);
    for (int k = 0; k < n; ++k) {
        EXPECT(P.order[k] >= 0 && P.order[k] < n);
        if (P.order[k] >= 0 && P.order[k] < n) ++seen[P.order[k]];
    }
    for (int i = 0; i < n; ++i) EXPECT(seen[i] == 1);

    // classes: contiguous, in class order, descending work inside
    int64_t ew_run = 0, ek_run[kNumEwKinds] = {0, 0, 0};
    int64_t g_run[kNumClasses] = {0, 0, 0}, u_run[kNumClasses] = {0, 0, 0};
    int64_t p_run[kNumClasses] = {0, 0, 0};
    EXPECT(P.pew[0] == 0);
    std::vector<Interval> iv;
    iv.push_back({ws, ws + P.table_bytes, "table"});
    for (int k = 0; k < n; ++k) {
        const muon_matrix& m = b.mats[P.order[k]];
        const MatDesc& d = P.d[k];
        const int64_t s = std::min(m.rows, m.cols);
        const int want_cls = (f32 || s <= kTinyF32) ? kF32 : (s <= kSmallBf16 ? kSmall : kLarge);
        EXPECT(d.cls == want_cls);
        const ClassPlan& C = P.cls[d.cls];
        EXPECT(k >= C.first && k < C.first + C.count);
        if (k > 0) {
            EXPECT(P.d[k - 1].cls <= d.cls);
            if (P.d[k - 1].cls == d.cls) {
                const muon_matrix& q = b.mats[P.order[k - 1]];
                const double wq = (double)std::min(q.rows, q.cols) * std::min(q.rows, q.cols) * std::max(q.rows, q.cols);
                const double wm = (double)s * s * std::max(m.rows, m.cols);
                EXPECT(wq >= wm);
            }
        }
        EXPECT(d.rows == m.rows && d.cols == m.cols && d.param == m.param && d.grad == m.grad);
        const int pad = kClassPad[d.cls], tile = kClassTile[d.cls];
        EXPECT(d.rows_pad == pad_to(m.rows, pad) && d.cols_pad == pad_to(m.cols, pad));
        EXPECT(d.transposed == (m.rows > m.cols ? 1 : 0));
        EXPECT(d.mp == (d.transposed ? d.cols_pad : d.rows_pad));
        EXPECT(d.np == (d.transposed ? d.rows_pad : d.cols_pad));
        EXPECT(d.mp <= d.np);
        EXPECT(d.rows_pad % d.ew_th == 0 && d.cols_pad % d.ew_tw == 0);
        EXPECT(d.ew_tiles == (d.rows_pad / d.ew_th) * (d.cols_pad / d.ew_tw));
        int kind = d.cls == kF32 ? kEwF32 : (d.ew_th == 16 ? kEwStream : kEwTrans);
        if (kind == kEwStream) EXPECT(!d.transposed && d.ew_tw == 256 && d.cols_pad % 256 == 0);
        if (kind == kEwTrans) EXPECT(d.ew_th == kTrTH && d.ew_tw == kTrTW);
        if (kind == kEwF32) EXPECT(d.ew_th == kEwTile && d.ew_tw == kEwTile);
        // vec4 only when every row start is 16-byte aligned
        if (d.vec4) {
            EXPECT(m.cols % 4 == 0);
            EXPECT((uintptr_t)m.param % (4 * (m.param_dtype == MUON_BF16 ? 2 : 4)) == 0);
            EXPECT(m.ld_param % 4 == 0 && m.ld_grad % 4 == 0 && m.ld_mom % 4 == 0);
        }
        ew_run += d.ew_tiles;
        ek_run[kind] += d.ew_tiles;
        EXPECT(P.pew[k + 1] == ew_run);
        for (int kk = 0; kk < kNumEwKinds; ++kk) EXPECT(P.pek[kk][k + 1] == ek_run[kk]);
        const int64_t Ts = d.mp / tile;
        g_run[d.cls] += d.cls == kF32 ? Ts * Ts : Ts * (Ts + 1) / 2;
        u_run[d.cls] += (d.mp / tile) * (d.np / tile);
        const int kc = k - C.first;
        EXPECT(C.ptri[kc + 1] == g_run[d.cls] && C.pupd[kc + 1] == u_run[d.cls]);
        // polynomial tiles: the triangle, or the triangle of 128-tiles
        if (C.poly_small) {
            EXPECT(d.cls == kLarge && d.mp % kClassTile[kSmall] == 0);
            const int64_t T = d.mp / kClassTile[kSmall];
            p_run[d.cls] += T * (T + 1) / 2;
        } else {
            p_run[d.cls] += d.cls == kF32 ? Ts * Ts : Ts * (Ts + 1) / 2;
        }
        EXPECT(C.ppoly[kc + 1] == p_run[d.cls]);
        // Gram tasks: the triangle tiles, times the K-parts when the class splits
        const int64_t tri = C.ptri[kc + 1] - C.ptri[kc];
        EXPECT(d.gram_split >= 1 && d.gram_split <= kMaxSplit);
        if (!C.gram_split) EXPECT(d.gram_split == 1 && C.pgram[kc + 1] == C.ptri[kc + 1]);
        if (C.gram_split) {
            EXPECT(d.cls != kF32);
            EXPECT(C.pgram[kc + 1] - C.pgram[kc] == tri * d.gram_split);
            // the kernel's part ranges cover the K slabs once, each part >= kMinSplitSlabs
            const int slabs = d.np / kGemmBK, S = d.gram_split;
            int covered = 0;
            for (int part = 0; part < S; ++part) {
                const int k0 = part * slabs / S, k1 = (part + 1) * slabs / S;
                EXPECT(k0 == covered && k1 > k0);
                if (S > 1) EXPECT(k1 - k0 >= kMinSplitSlabs);
                covered = k1;
            }
            EXPECT(covered == slabs);
            const size_t tt = (size_t)kClassTile[d.cls];
            EXPECT(d.gram_part != nullptr);
            iv.push_back({(uintptr_t)d.gram_part,
                          (uintptr_t)d.gram_part + (size_t)(tri * d.gram_split) * tt * tt * 4, "part"});
        } else {
            EXPECT(d.gram_part == nullptr);
        }
        // workspace buffers
        const size_t es = d.cls == kF32 ? 4 : 2;
        const size_t xb = (size_t)d.mp * d.np * es, ab = (size_t)d.mp * d.mp * es;
        const void* xs[4] = {d.x[0], d.x[1], d.xt[0], d.xt[1]};
        for (int i = 0; i < 4; ++i) {
            if (i >= 2 && d.cls != kF32) { EXPECT(xs[i] == nullptr); continue; }
            iv.push_back({(uintptr_t)xs[i], (uintptr_t)xs[i] + xb, "x"});
        }
        iv.push_back({(uintptr_t)d.a, (uintptr_t)d.a + ab, "a"});
        iv.push_back({(uintptr_t)d.b, (uintptr_t)d.b + ab, "b"});
        EXPECT((uintptr_t)d.partials == ws + P.off_partials + 4 * (size_t)P.pew[k]);
        EXPECT((uintptr_t)d.inv_norm == ws + P.off_invnorm + 4 * (size_t)k);
    }
    iv.push_back({ws + P.off_partials, ws + P.off_partials + 4 * (size_t)ew_run, "partials"});
    iv.push_back({ws + P.off_invnorm, ws + P.off_invnorm + 4 * (size_t)n, "inv_norm"});
    for (int kind = 0; kind < kNumEwKinds; ++kind) EXPECT(P.total_ek[kind] == ek_run[kind]);
    std::sort(iv.begin(), iv.end(), [](const Interval& a, const Interval& c) { return a.lo < c.lo; });
    for (size_t i = 0; i < iv.size(); ++i) {
        EXPECT(iv[i].lo % 256 == 0);
        EXPECT(iv[i].lo >= ws && iv[i].hi <= ws + P.total);
        if (i > 0) EXPECT(iv[i - 1].hi <= iv[i].lo);
    }
    // the table's pieces lie inside it and do not overlap
    std::vector<Interval> tv;
    tv.push_back({0, (size_t)n * sizeof(MatDesc), "desc"});
    for (int kind = 0; kind < kNumEwKinds; ++kind)
        tv.push_back({P.off_pek[kind], P.off_pek[kind] + 4 * (size_t)(n + 1), "pek"});
    for (int c = 0; c < kNumClasses; ++c) {
        EXPECT(P.cls[c].total_tri == g_run[c] && P.cls[c].total_upd == u_run[c]);
        EXPECT(P.cls[c].total_poly == p_run[c]);
        {
            int kn = 0, km = 0;
            for (int k = P.cls[c].first; k < P.cls[c].first + P.cls[c].count; ++k) {
                kn = std::max<int>(kn, P.d[k].np);
                km = std::max<int>(km, P.d[k].mp);
            }
            EXPECT(P.cls[c].kmax_n == kn && P.cls[c].kmax_m == km);
        }
        // 128-tiles for the polynomial exactly when the 256-tiles fill at most
        // half the compute units and the 128-tiles fit one round at two per unit
        if (c == kLarge && P.cls[c].count > 0) {
            int64_t t128 = 0;
            for (int k = P.cls[c].first; k < P.cls[c].first + P.cls[c].count; ++k) {
                const int64_t T = P.d[k].mp / kClassTile[kSmall];
                t128 += T * (T + 1) / 2;
            }
            const bool want = 2 * (int64_t)P.cls[c].total_tri <= 8 * (int64_t)cus && t128 <= 16 * (int64_t)cus;
            EXPECT(P.cls[c].poly_small == want);
        } else {
            EXPECT(!P.cls[c].poly_small);
        }
        EXPECT(P.cls[c].total_gram == P.cls[c].pgram[P.cls[c].count]);
        // a split launch fits one round; a launch is split only when starved
        if (P.cls[c].gram_split) {
            const int slots = 8 * cus * (c == kSmall ? 2 : 1);
            EXPECT(P.cls[c].total_gram <= slots);
            EXPECT(4 * P.cls[c].total_tri <= slots);
        }
        tv.push_back({P.cls[c].off_pgram, P.cls[c].off_pgram + 4 * (size_t)(P.cls[c].count + 1), "pg"});
        tv.push_back({P.cls[c].off_ptri, P.cls[c].off_ptri + 4 * (size_t)(P.cls[c].count + 1), "pt"});
        tv.push_back({P.cls[c].off_ppoly, P.cls[c].off_ppoly + 4 * (size_t)(P.cls[c].count + 1), "pp"});
        tv.push_back({P.cls[c].off_pstrip, P.cls[c].off_pstrip + 4 * (size_t)(P.cls[c].count + 1), "ps"});
        tv.push_back({P.cls[c].off_pupd, P.cls[c].off_pupd + 4 * (size_t)(P.cls[c].count + 1), "pu"});
    }
    std::sort(tv.begin(), tv.end(), [](const Interval& a, const Interval& c) { return a.lo < c.lo; });
    for (size_t i = 0; i < tv.size(); ++i) {
        EXPECT(tv[i].hi <= P.table_bytes);
        if (i > 0) EXPECT(tv[i - 1].hi <= tv[i].lo);
    }
    std::vector<char> img;
    table_image(P, img);
    EXPECT(img.size() == P.table_bytes);
    EXPECT(memcmp(img.data(), P.d.data(), (size_t)n * sizeof(MatDesc)) == 0);
    for (int c = 0; c < kNumClasses; ++c) {
        const ClassPlan& C = P.cls[c];
        EXPECT(memcmp(img.data() + C.off_pupd, C.pupd.data(), 4 * (size_t)(C.count + 1)) == 0);
        EXPECT(memcmp(img.data() + C.off_ptri, C.ptri.data(), 4 * (size_t)(C.count + 1)) == 0);
        EXPECT(memcmp(img.data() + C.off_ppoly, C.ppoly.data(), 4 * (size_t)(C.count + 1)) == 0);
        EXPECT(memcmp(img.data() + C.off_pgram, C.pgram.data(), 4 * (size_t)(C.count + 1)) == 0);
        if (c == kF32 || C.count == 0) continue;
        check_split(C.xs_gram, C.total_gram, cus, c == kLarge && !C.gram_split);
        EXPECT(C.xs_gram.interleaved == 1 && C.xs_poly.interleaved == 0 && C.xs_upd.interleaved == 1);
        check_split(C.xs_poly, C.total_poly, cus, c == kLarge && !C.poly_small);
        // the small class's update in strips exactly when two or more tiles per
        // workgroup fill the compute units once (one workgroup each, streamed,
        // when the class is alone in the call, else two); strips cover each
        // matrix's column tiles once, in order
        if (c == kSmall) {
            const bool alone = P.cls[kLarge].count == 0 && P.cls[kF32].count == 0;
            const int64_t slots = (alone ? 8 : 16) * (int64_t)cus;
            const int64_t L = (C.total_upd + slots - 1) / slots;
            EXPECT(C.strip == (L >= 2 ? (int)L : 0));
            EXPECT(C.stream == (C.strip > 0 && alone));
            {
                // the strips apply the step themselves only when every matrix
                // is a plain fp32 weight of 128 x 128k rows
                bool plain = C.stream;
                for (int k = 0; k < C.count; ++k) {
                    const MatDesc& d = P.d[C.first + k];
                    const muon_matrix& m = b.mats[P.order[C.first + k]];
                    plain = plain && m.rows == 128 && m.cols % 128 == 0 && m.param_dtype == MUON_F32 &&
                            !m.update_out && !m.qk_smax && d.vec4 &&
                            ((m.rows - 1) * m.ld_param + m.cols) * 4 < ((int64_t)1 << 31);
                }
                EXPECT(C.fuse_apply == plain);
            }
            if (C.strip > 0) {
                int64_t run = 0;
                EXPECT(C.pstrip.size() == (size_t)C.count + 1 && C.pstrip[0] == 0);
                for (int k = 0; k < C.count; ++k) {
                    const MatDesc& d = P.d[C.first + k];
                    EXPECT(d.mp == kClassTile[kSmall]);
                    const int64_t tiles = d.np / kClassTile[kSmall];
                    EXPECT(tiles == C.pupd[k + 1] - C.pupd[k]);
                    run += (tiles + C.strip - 1) / C.strip;
                    EXPECT(C.pstrip[k + 1] == run);
                    // the last strip of the matrix is not empty
                    EXPECT((int64_t)(C.pstrip[k + 1] - C.pstrip[k] - 1) * C.strip < tiles);
                }
                EXPECT(C.total_strips == run);
                bool fuse = C.gram_split;
                for (int k = 0; k < C.count; ++k)
                    fuse = fuse && C.pstrip[k + 1] - C.pstrip[k] == P.d[C.first + k].gram_split;
                EXPECT(C.fuse_gram == fuse);
                check_split(C.xs_strip, C.total_strips, cus, 0);
                EXPECT(memcmp(img.data() + C.off_pstrip, C.pstrip.data(), 4 * (size_t)(C.count + 1)) == 0);
            }
        } else {
            EXPECT(C.strip == 0 && !C.fuse_gram && !C.stream);
        }
        check_split(C.xs_upd, C.total_upd, cus, c == kLarge);
    }
    const std::vector<int> sm = split_matrices(P);
    for (size_t i = 0; i < sm.size(); ++i) {
        EXPECT(sm[i] >= 0 && sm[i] < n);
        if (i > 0) EXPECT(sm[i - 1] < sm[i]);
        if (sm[i] >= 0 && sm[i] < n) {
            const muon_matrix& m = b.mats[sm[i]];
            EXPECT(f32 == false && std::min(m.rows, m.cols) > kTinyF32);
        }
    }
}

static void check_rejections(std::mt19937_64& rng) {
    Batch b = random_batch(rng, 3, false);
    Plan P;
    const uintptr_t ws = (uintptr_t)1 << 36;
    EXPECT(make_plan(b.mats.data(), 3, &b.hp, true, ws, 32, P) == MUON_OK);
    EXPECT(make_plan(nullptr, 3, &b.hp, true, ws, 32, P) == MUON_ERR_INVALID_ARG);
    EXPECT(make_plan(b.mats.data(), 0, &b.hp, true, ws, 32, P) == MUON_ERR_INVALID_ARG);
    EXPECT(make_plan(b.mats.data(), 3, nullptr, true, ws, 32, P) == MUON_ERR_INVALID_ARG);
    auto with = [&](auto edit, muon_status want) {
        Batch c = b;
        edit(c);
        EXPECT(make_plan(c.mats.data(), 3, &c.hp, true, ws, 32, P) == want);
    };
    with([](Batch& c) { c.mats[1].rows = 0; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.mats[1].cols = kMaxDim + 1; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.mats[2].ld_grad = c.mats[2].cols - 1; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.mats[0].param_dtype = 7; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.mats[0].grad = nullptr; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.mats[0].grad = c.mats[0].param; c.mats[0].grad_dtype = c.mats[0].param_dtype; }, MUON_ERR_OVERLAP);
    with([](Batch& c) { c.mats[1].momentum = (float*)((uintptr_t)c.mats[1].momentum + 2); }, MUON_ERR_UNALIGNED);
    with([](Batch& c) { c.mats[1].qk_smax = c.mats[1].momentum; c.mats[1].qk_block_rows = c.mats[1].rows + 1; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.hp.ns_steps = 0; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.hp.ns_dtype = 9; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.hp.scale_mode = 4; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.hp.lr = __builtin_nanf(""); }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.hp.eps = -1.f; }, MUON_ERR_INVALID_ARG);
    with([](Batch& c) { c.hp.qk_tau = -1.f; }, MUON_ERR_INVALID_ARG);
    // without pointers (workspace sizing) the pointer checks are skipped
    Batch c = b;
    c.mats[0].grad = nullptr;
    EXPECT(make_plan(c.mats.data(), 3, &c.hp, false, 0, 32, P) == MUON_OK);
}

int main(int argc, char** argv) {
    const int trials = argc > 1 ? atoi(argv[1]) : 3000;
    std::mt19937_64 rng(12345);
    for (int t = 0; t < trials && failures == 0; ++t) {
        const int n = t % 50 == 0 ? 1 + (int)(rng() % 3000) : 1 + (int)(rng() % 40);
        Batch b = random_batch(rng, n, t % 97 == 0);
        const int cus = t % 5 == 0 ? 1 + (int)(rng() % 40) : 32;
        Plan P;
        const uintptr_t ws = ((uintptr_t)1 << 36) + 256 * (uintptr_t)(rng() % 1000);
        const muon_status st = make_plan(b.mats.data(), n, &b.hp, true, ws, cus, P);
        EXPECT(st == MUON_OK);
        if (st == MUON_OK) check_plan(b, P, ws, cus);
        // sizing without pointers gives the same total
        Plan Q;
        EXPECT(make_plan(b.mats.data(), n, &b.hp, false, 0, cus, Q) == MUON_OK && Q.total == P.total);
    }
    for (int t = 0; t < 200; ++t) check_rejections(rng);
    // gram_splits on its own: the per-head shape (64 tiles of 112 slabs) and c1's block
    {
        std::vector<int32_t> S = gram_splits(std::vector<int32_t>(64, 1), std::vector<int32_t>(64, 112), 256);
        for (int32_t v : S) EXPECT(v == 4);
        S = gram_splits(std::vector<int32_t>(64, 1), std::vector<int32_t>(64, 112), 512);
        for (int32_t v : S) EXPECT(v == 8);
        std::vector<int32_t> tiles = {10, 10, 10, 10, 10, 10, 10}, slabs = {64, 64, 64, 16, 16, 16, 16};
        S = gram_splits(tiles, slabs, 256);
        for (int32_t v : S) EXPECT(v == 1);   // 70 tiles: more than a quarter of the slots
        tiles = {10, 10, 10, 10, 10};
        slabs = {64, 64, 64, 16, 16};
        S = gram_splits(tiles, slabs, 256);
        int64_t tasks = 0;
        for (size_t k = 0; k < S.size(); ++k) tasks += tiles[k] * S[k];
        EXPECT(tasks <= 256 && S[0] > 1 && S[0] == S[1] && S[3] >= 1);
        S = gram_splits(std::vector<int32_t>(2, 136), std::vector<int32_t>(2, 64), 256);
        EXPECT(S[0] == 1 && S[1] == 1);   // 272 tiles: no split
        S = gram_splits(std::vector<int32_t>(1, 136), std::vector<int32_t>(1, 64), 256);
        EXPECT(S[0] == 1);                // 2 parts would take two rounds
        S = gram_splits(std::vector<int32_t>(3, 1), std::vector<int32_t>(3, 7), 256);
        for (int32_t v : S) EXPECT(v == 1);   // shorter than a part
        S = gram_splits(std::vector<int32_t>(1, 1), std::vector<int32_t>(1, 16384), 256);
        EXPECT(S[0] == kMaxSplit);
    }
    // the polynomial's tiling on workloads whose launch shapes are known
    {
        auto plan_of = [&](const std::vector<std::pair<int64_t, int64_t>>& shapes, Plan& P) {
            Batch b;
            uintptr_t next = (uintptr_t)1 << 40;
            for (const auto& sh : shapes) {
                muon_matrix m;
                memset(&m, 0, sizeof(m));
                m.rows = sh.first;
                m.cols = sh.second;
                m.param_dtype = m.grad_dtype = MUON_F32;
                m.ld_param = m.ld_grad = m.ld_mom = m.cols;
                const size_t bytes = (size_t)(m.rows * m.cols) * 4 + 4096;
                m.param = (void*)next;
                next += bytes;
                m.grad = (const void*)next;
                next += bytes;
                m.momentum = (float*)next;
                next += bytes;
                b.mats.push_back(m);
            }
            memset(&b.hp, 0, sizeof(b.hp));
            b.hp.lr = 2e-4f;
            b.hp.momentum = 0.95f;
            b.hp.eps = 1e-7f;
            b.hp.extra_scale = 1.f;
            b.hp.nesterov = 1;
            b.hp.ns_steps = 5;
            b.hp.ns_dtype = MUON_BF16;
            const uintptr_t ws = (uintptr_t)1 << 36;
            EXPECT(make_plan(b.mats.data(), (int)shapes.size(), &b.hp, true, ws, 32, P) == MUON_OK);
            check_plan(b, P, ws, 32);
        };
        Plan P;
        // d=1024 block: 70 tiles of 256 -> 7 x 36 tiles of 128 in one round
        plan_of({{1024, 1024}, {1024, 1024}, {1024, 1024}, {1024, 1024}, {4096, 1024}, {4096, 1024},
                 {1024, 4096}}, P);
        EXPECT(P.cls[kLarge].poly_small && P.cls[kLarge].total_tri == 70 && P.cls[kLarge].total_poly == 252);
        EXPECT(P.cls[kLarge].xs_poly.per == 32);
        // one 4096^2 matrix: 136 tiles fill more than half the units
        plan_of({{4096, 4096}}, P);
        EXPECT(!P.cls[kLarge].poly_small && P.cls[kLarge].total_poly == 136);
        // 105 tiles of 256 (3584^2) would be 420 quarter slots; 406 tiles of 128 fit one round
        plan_of({{3584, 3584}}, P);
        EXPECT(P.cls[kLarge].poly_small && P.cls[kLarge].total_poly == 406);
        // per head alone: 64 blocks of 128 x 7168 (56 column tiles each) in
        // streamed strips of 14, the K-split Gram in as many parts (4)
        plan_of(std::vector<std::pair<int64_t, int64_t>>(64, {128, 7168}), P);
        EXPECT(P.cls[kSmall].strip == 14 && P.cls[kSmall].total_strips == 256 && P.cls[kSmall].stream);
        EXPECT(P.cls[kSmall].gram_split && P.cls[kSmall].fuse_gram && P.d[0].gram_split == 4);
        EXPECT(P.cls[kSmall].fuse_apply);  // plain fp32 weights: the last strips apply the step
        // the same blocks beside a 4096^2 matrix: strips of 7 for two
        // workgroups per compute unit, 8 Gram parts, not streamed
        {
            std::vector<std::pair<int64_t, int64_t>> sh(64, {128, 7168});
            sh.push_back({4096, 4096});
            plan_of(sh, P);
            EXPECT(P.cls[kSmall].strip == 7 && P.cls[kSmall].total_strips == 512 && !P.cls[kSmall].stream);
            EXPECT(P.cls[kSmall].gram_split && P.cls[kSmall].fuse_gram);
            EXPECT(P.d[P.cls[kSmall].first].gram_split == 8 && !P.cls[kSmall].fuse_apply);
        }
        // 16 blocks of 100 x 4900 (39 tiles, 78 slabs each), alone: streamed
        // strips of 3, 13 per block; 13 Gram parts would be shorter than
        // kMinSplitSlabs, so the Gram keeps its own 9 parts and no fusion
        plan_of(std::vector<std::pair<int64_t, int64_t>>(16, {100, 4900}), P);
        EXPECT(P.cls[kSmall].strip == 3 && P.cls[kSmall].total_strips == 16 * 13 && P.cls[kSmall].stream);
        EXPECT(P.cls[kSmall].gram_split && !P.cls[kSmall].fuse_gram && P.d[0].gram_split == 9);
        EXPECT(!P.cls[kSmall].fuse_apply);  // 100 rows: padded, the apply launch runs
        // few small tiles: one tile per workgroup
        plan_of({{128, 4096}, {100, 3000}}, P);
        EXPECT(P.cls[kSmall].strip == 0 && !P.cls[kSmall].fuse_gram && !P.cls[kSmall].stream);
        // 64 heads of 128 x 3584 alone: strips of 7 (4 per head), 4 Gram parts
        plan_of(std::vector<std::pair<int64_t, int64_t>>(64, {128, 3584}), P);
        EXPECT(P.cls[kSmall].strip == 7 && P.d[0].gram_split == 4 && P.cls[kSmall].fuse_gram);
        // beside a large matrix, 16 blocks of 100 x 4900: strips of 2 against
        // 9 Gram parts, no fusion
        {
            std::vector<std::pair<int64_t, int64_t>> sh(16, {100, 4900});
            sh.push_back({1024, 1024});
            plan_of(sh, P);
            EXPECT(P.cls[kSmall].strip == 2 && !P.cls[kSmall].stream);
            EXPECT(P.cls[kSmall].gram_split && !P.cls[kSmall].fuse_gram);
        }
    }
    // xcd_split on its own: degenerate inputs
    {
        for (int il = 0; il < 2; ++il) {
            const int32_t none[3] = {0, 0, 0};
            const int64_t w[3] = {1, 5, 0};
            XcdSplit xs = xcd_split(none, w, 3, 32, 1, il);
            check_split(xs, 0, 32, 1);
            const int32_t one[1] = {1};
            xs = xcd_split(one, w, 1, 32, 1, il);
            check_split(xs, 1, 32, 1);
            const int32_t zw[2] = {7, 9};
            const int64_t zero[2] = {0, 0};
            xs = xcd_split(zw, zero, 2, 3, 0, il);
            check_split(xs, 16, 3, 0);
            // the 8 x 4096^2 update (2048 tiles) and Gram (1088 tiles)
            const int32_t upd[8] = {256, 256, 256, 256, 256, 256, 256, 256};
            const int32_t tri[8] = {136, 136, 136, 136, 136, 136, 136, 136};
            const int64_t k[8] = {4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096};
            xs = xcd_split(upd, k, 8, 32, 1, il);
            check_split(xs, 2048, 32, 1);
            EXPECT(xs.per == 256);
            xs = xcd_split(tri, k, 8, 32, 1, il);
            check_split(xs, 1088, 32, 1);
            EXPECT(xs.per == 128 + 4 * 8);  // four rounds, then 8 tiles as 32 quarters
        }
        // random tile lists in both modes
        std::mt19937_64 r2(99);
        for (int t = 0; t < 3000; ++t) {
            const int n = 1 + (int)(r2() % 12);
            std::vector<int32_t> tl(n);
            std::vector<int64_t> wl(n);
            int total = 0;
            for (int k = 0; k < n; ++k) {
                tl[k] = (int32_t)(r2() % (t % 3 ? 700 : 5));
                wl[k] = 1 + (int64_t)(r2() % 256);
                total += tl[k];
            }
            const int cus = t % 2 ? 32 : 1 + (int)(r2() % 40);
            const int q = (t >> 1) & 1, il = (t >> 2) & 1;
            const XcdSplit xs = xcd_split(tl.data(), wl.data(), n, cus, q, il);
            check_split(xs, total, cus, q);
            // the ranges after the interleaved rounds hold equal work, within one tile
            std::vector<int64_t> tw;
            int64_t wmax = 1;
            for (int k = 0; k < n; ++k) {
                for (int i = 0; i < tl[k]; ++i) tw.push_back(wl[k]);
                wmax = std::max(wmax, wl[k]);
            }
            int64_t tail_w = 0;
            for (int i = xs.b[0]; i < total; ++i) tail_w += tw[i];
            for (int x = 0; x < 8; ++x) {
                int64_t w = 0;
                for (int i = xs.b[x]; i < xs.b[x + 1]; ++i) w += tw[i];
                EXPECT(w * 8 <= tail_w + 8 * wmax);
            }
        }
    }
    if (failures) {
        printf("%d failures\n", failures);
        return 1;
    }
    printf("ok\n");
    return 0;
}
