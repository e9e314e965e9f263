// MFMA kernels of the quintic Newton-Schulz iteration (gfx950): the bf16
// products, and at the end of the file the fp32 option's products on the same
// slab machinery (v_mfma_f32_32x32x2f32).
//
// One iteration X <- a X + b (X X^T) X + c (X X^T)^2 X is computed on the
// small Gram as three products ("About Muon: Why Not Adam", kiungsong.github.io,
// section "Making It Actually Run": the odd polynomial acts on singular values
// only, and running it on X X^T after the short-side transpose gives the same
// result):
//
//   gram:   A = X X^T                    m' x m', symmetric
//   poly:   B = a I + b A + c A A        m' x m', symmetric (A A = A A^T)
//   update: X <- B X                     m' x n'
//
// (a X + (b A + c A A) X = B X with the identity term folded into B's
// diagonal; the update then reads nothing but its two operands.)
//
// The Gram and the polynomial are "NT" products C[i][j] = sum_k P[i][k] Q[j][k]
// with both operands read along contiguous rows (X's rows; A's rows, A being
// symmetric).  The update C[i][j] = sum_k B[i][k] X[k][j] reads B by rows and
// X in its natural k-major layout: slabs of X rows are copied to LDS as they
// are and the MFMA operand is gathered with the transposing LDS read
// (ds_read_b64_tr_b16), so no transposed copy of X is ever stored.
//
// The Gram and the polynomial outputs are symmetric: only tiles on or below
// the diagonal are computed and each off-diagonal tile is stored twice (as
// itself and mirrored).
//
// Tiling: a workgroup computes a BM x BN tile with WM x WN waves, each wave a
// (BM/WM) x (BN/WN) block of 32 x 32 MFMA tiles (v_mfma_f32_32x32x16_bf16,
// fp32 accumulation).  K advances in slabs of 64: operand slabs are copied
// global->LDS with buffer_load_dwordx4 ... lds (16 bytes per lane, no VGPR
// staging) into LDS stages (two for 256 x 256 tiles, four for 128 x 128), so
// the copies of later slabs overlap the MFMAs on slab k.  The epilogue goes
// through LDS so that every global access is a coalesced 16-byte one.  LDS
// rows are XOR-swizzled (see swz, swzk) so fragment reads are free of bank
// conflicts.
//
// Each XCD takes a contiguous range of tiles; a short last round is run as
// quarter tiles (see XcdSplit).
//
// Grouped launch: one launch per phase covers every matrix; workgroup ->
// (matrix, tile) through prefix sums of tiles per matrix.
#include "muon_internal.h"

#include <type_traits>

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource over `base` (gfx9 family: 32-bit data format, no
// stride, no swizzle; offsets up to 2 GB).  A slab copy through it needs one
// 32-bit offset register per lane instead of a 64-bit address.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t slab_rsrc(const uint16_t* base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, 0x7fffffff, 0x00020000);
}

enum { GRAM = 0, POLY = 1, UPDATE = 2 };

// LDS is four 32 KB arrays (see Stages).
constexpr int kLdsArr = 16384;  // bf16 elements per array

template <int BM_, int BN_, int WM_, int WN_, int BK_ = 64, int NS_ = 2>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int BK = BK_;   // k per LDS stage (32 or 64)
    static constexpr int NS = NS_;   // LDS stages
    static constexpr int NW = WM * WN;
    static constexpr int NT = 64 * NW;
    static constexpr int TM = BM / WM, TN = BN / WN;
    static constexpr int FM = TM / 32, FN = TN / 32;
    static constexpr int CH = BK / 8;          // 16-byte chunks per LDS row
    static constexpr int RPI = 64 / CH;        // rows per 1 KB slab copy
    static constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per LDS stage
    static constexpr int LPS = ((BM + BN) / RPI) / NW;  // slab copies per stage per wave
    static constexpr int LPS1 = (BM / RPI) / NW;        // ... when both operands are one slab
    // a stage is one LDS array (P slab, then Q slab) or, when each slab fills
    // an array by itself, two (P, Q)
    static constexpr int SPLIT = STAGE > kLdsArr ? 1 : 0;
    static constexpr int NARR = SPLIT ? 2 * NS : NS;  // LDS arrays used
    // epilogue: bands of RB rows staged as fp32 in array 0
    static constexpr int RB = 32;  // = the MFMA tile height: a band is one row block
    static_assert(SPLIT ? (BM * BK == kLdsArr && BN * BK == kLdsArr) : STAGE <= kLdsArr,
                  "a stage is one array, or one array per operand");
    static_assert(NARR <= 4, "four LDS arrays");
    static_assert(RB * BN * 4 <= kLdsArr * 2, "epilogue band must fit one array");
    static_assert(BN % 64 == 0, "the band swizzle permutes columns within runs of 64");
    static_assert(BK == 32 || BK == 64, "BK is 32 or 64");
    static_assert(NS >= 2 && NS <= 4, "2 to 4 stages");
    static_assert(FM >= 1 && FN >= 1, "wave tile must hold a 32x32 MFMA tile");
    static_assert((BM / RPI) % NW == 0 && (BN / RPI) % NW == 0, "slab rows must split over waves");
    static_assert((RB * BN / 8) % NT == 0 && (BN * RB / 8) % NT == 0, "epilogue chunks must split");
};

// LDS: four 32 KB arrays, each its own __shared__ variable (declared in the
// kernel) so the compiler can tell that a copy into one array does not alias
// the fragment reads from another; otherwise it waits for every outstanding
// copy before each read and the prefetch is lost.  A 256 x 256 tile keeps two
// stages of two arrays (P slab, Q slab); a 128 x 128 tile keeps up to four
// stages of one array each.
struct Stages {
    uint16_t* s[4];
};

__device__ __forceinline__ uint16_t* lds_arr(const Stages& st, int i) {
    return i == 0 ? st.s[0] : i == 1 ? st.s[1] : i == 2 ? st.s[2] : st.s[3];
}
template <class C>
__device__ __forceinline__ uint16_t* stage_p(const Stages& st, int i) {
    return C::SPLIT ? lds_arr(st, 2 * i) : lds_arr(st, i);
}
template <class C>
__device__ __forceinline__ uint16_t* stage_q(const Stages& st, int i) {
    return C::SPLIT ? lds_arr(st, 2 * i + 1) : lds_arr(st, i) + C::BM * C::BK;
}

// Epilogue band buffer (fp32, RB x BN, in array 0), unpadded: column c of row
// r sits at c ^ ((r & 4) << 3) ^ ((r >> 3) << 4).  The first term puts the two
// half-waves of an accumulator store (rows r and r + 4) 32 banks apart; the
// second puts the four rows r, r + 8, r + 16, r + 24 that one instruction of
// the transposed pass reads for each column 16 banks apart.  Both leave runs
// of 16 columns contiguous.
template <class C>
__device__ __forceinline__ int sbi(int r, int c) {
    return r * C::BN + (c ^ ((r & 4) << 3) ^ ((r >> 3) << 4));
}

// LDS slab layout: row r holds BK bf16 = CH chunks of 16 bytes; logical chunk
// c of row r sits at chunk position c ^ swz(r).  A fragment read has 16
// lanes per LDS cycle (16 x 16 B = all 64 banks) reading the same logical
// chunk of 16 consecutive rows; 256 bytes hold 256 / (2 BK) rows, so the 16
// reads are conflict-free iff (r mod rows-per-256B, position) differs
// across them.
template <int BK>
__device__ __forceinline__ int swz(int row) {
    return BK == 64 ? ((row >> 1) & 7) : ((row >> 2) & 3);
}

// Copy rows [0, R) x k-chunk [0, BK) of a row-major bf16 operand (rows start
// at `g`, leading dimension ld) into an LDS slab, swizzled.  One
// buffer_load_dwordx4 ... lds moves 1 KB (RPI rows, contiguous in LDS); lane L
// fills chunk position L % CH of row L / CH, i.e. it fetches logical chunk
// (L % CH) ^ swz(row).
template <class C, int R>
__device__ __forceinline__ void load_slab(const uint16_t* __restrict__ g, int64_t ld, uint16_t* slab,
                                          int wave, int lane) {
    constexpr int PER_WAVE = (R / C::RPI) / C::NW;
    const __amdgpu_buffer_rsrc_t r = slab_rsrc(g);
    const int lrow = lane / C::CH;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
        const int grp = wave * PER_WAVE + q;
        const int row = grp * C::RPI + lrow;
        const int lch = (lane % C::CH) ^ swz<C::BK>(row);
        const uint32_t off = (uint32_t)(row * (int)ld + lch * 8) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slab + grp * C::RPI * C::BK), 16,
                                                 off, 0, 0, 0);
    }
}

template <class C>
__device__ __forceinline__ bf16x8 read_frag(const uint16_t* slab, int row, int lch) {
    const int pch = lch ^ swz<C::BK>(row);
    return *reinterpret_cast<const bf16x8*>(slab + row * C::BK + pch * 8);
}

// k-major operand (the update's X): an LDS slab holds BK rows k of BN
// columns, 2 BN bytes per row, the 16-byte chunk c of row k at position
// c ^ swzk(k).  A transposing read by 16 lanes covers 4 consecutive rows x
// 64 bytes; swzk spreads those 4 rows over disjoint quarters of the 256-byte
// bank space.
__device__ __forceinline__ int swzk(int k) { return (k & 3) << 2; }

// Copy rows [0, BK) (k) x columns [0, BN) of a row-major bf16 matrix (row k
// at g + k * ld) into a k-major slab.  One buffer_load_dwordx4 ... lds moves 1 KB
// = 1024 / (2 BN) rows; lane L fills chunk position L % CQ of row L / CQ.
template <class C>
__device__ __forceinline__ void load_slab_kn(const uint16_t* __restrict__ g, int64_t ld,
                                             uint16_t* slab, int wave, int lane) {
    constexpr int CQ = C::BN / 8;          // 16-byte chunks per row
    constexpr int RPK = 64 / CQ;           // rows per copy
    constexpr int PER_WAVE = (C::BK / RPK) / C::NW;
    static_assert((C::BK / RPK) % C::NW == 0, "k-major slab rows must split over waves");
    const __amdgpu_buffer_rsrc_t r = slab_rsrc(g);
    const int lrow = lane / CQ;
    const int p = lane % CQ;
#pragma unroll
    for (int q = 0; q < PER_WAVE; ++q) {
        const int grp = wave * PER_WAVE + q;
        const int k = grp * RPK + lrow;
        const uint32_t off = (uint32_t)(k * (int)ld + (p ^ swzk(k)) * 8) * 2u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(slab + grp * RPK * C::BN), 16, off,
                                                 0, 0, 0);
    }
}

// MFMA B-operand fragment (lane l: column n0 + l % 32, k = k0 + 8 (l / 32) +
// 0..7) from a k-major slab, as two transposing 8-byte reads.  In each group
// of 16 lanes, lane a + 4 b addresses row b, columns 4a..4a+3 of a 4 x 16
// block and receives column (lane % 16) of rows 0..3.
template <class C>
__device__ __forceinline__ bf16x8 read_frag_kn(const uint16_t* slab, int k0, int n0, int lane) {
    const int g = lane >> 4, s16 = lane & 15;
    const int a = s16 & 3, b = s16 >> 2;
    const int n = n0 + 16 * (g & 1) + 4 * a;
    i16x4 h[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int k = k0 + 8 * (g >> 1) + 4 * t + b;
        const uint16_t* p = slab + k * C::BN + (((n >> 3) ^ swzk(k)) << 3) + (n & 7);
        h[t] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) i16x4*)(p));
    }
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(h[0], h[1], 0, 1, 2, 3, 4, 5, 6, 7));
}

// Output stores of the epilogue: streaming (nt) and at device scope (sc1), so
// they are written through L2 without displacing the operand slabs that the
// other tiles of the XCD are still reading.  `base` is uniform (a row band or
// a column band of the output); the byte offset stays far below 2 GB.
constexpr int kStreamStore = 2 | 16;  // cache policy bits: nt | sc1
__device__ __forceinline__ void store_out(uint16_t* base, uint32_t byte_off, const uint4& v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(GWord<16>::T, v), slab_rsrc(base),
                                           byte_off, 0, kStreamStore);
}

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    return (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
}

struct Epi {
    // output (row-major, ld) and, when `outT` is set, its transpose
    uint16_t* out;
    // K-split Gram: the raw fp32 tile (row-major, ld BN) instead of `out`
    float* outF;
    int64_t ld_out;
    uint16_t* outT;
    int64_t ld_outT;
    // v = post * (coef_acc * product + coef_e * E[i][j]) + diag * [i == j]
    // (E only if HAS_E; diag only on tiles that hold part of the diagonal)
    const uint16_t* E;
    int64_t ld_e;
    float coef_e;
    float coef_acc;
    float post;
    float diag;
};

// Copy the operand slabs of k-range [k0, k0 + BK) into one LDS stage: the
// BM x BK slab of P, then Q's (BN x BK, or BK x BN k-major).  SAME: Q is the
// same rows of the same matrix as P (a diagonal tile of a symmetric product),
// whose fragments are then read from P's slab.
template <class C, bool QKN, bool SAME = false>
__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ P0, int64_t ldp,
                                           const uint16_t* __restrict__ Q0, int64_t ldq,
                                           int64_t k0, const Stages& st, int i, int wave, int lane) {
    load_slab<C, C::BM>(P0 + k0, ldp, stage_p<C>(st, i), wave, lane);
    if (SAME) return;
    if (QKN)
        load_slab_kn<C>(Q0 + k0 * ldq, ldq, stage_q<C>(st, i), wave, lane);
    else
        load_slab<C, C::BN>(Q0 + k0, ldq, stage_q<C>(st, i), wave, lane);
}

// Fragments of MFMA k-step kk (16 deep) of one LDS slab: FM row blocks of
// the P operand and FN of the Q operand for this wave.
template <class C>
struct Frags {
    bf16x8 a[C::FM], b[C::FN];
};

template <class C, bool QKN, bool SAME = false>
__device__ __forceinline__ void read_frags(const Stages& st, int i, int kk, int wm, int wn,
                                           int frow, int khalf, int lane, Frags<C>& f) {
    const uint16_t* sp = stage_p<C>(st, i);
    const uint16_t* sq = SAME ? sp : stage_q<C>(st, i);
    const int lch = 2 * kk + khalf;
#pragma unroll
    for (int i = 0; i < C::FM; ++i) f.a[i] = read_frag<C>(sp, wm * C::TM + i * 32 + frow, lch);
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
        f.b[j] = QKN ? read_frag_kn<C>(sq, 16 * kk, wn * C::TN + j * 32, lane)
                     : read_frag<C>(sq, wn * C::TN + j * 32 + frow, lch);
}

template <class C>
__device__ __forceinline__ void mfma_frags(f32x16 (&acc)[C::FM][C::FN], const Frags<C>& f) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.a[i], f.b[j], acc[i][j], 0, 0, 0);
}

// Scheduling pattern for one k-step: the NR LDS reads of the next k-step's
// fragments go out RPM at a time between this k-step's NM MFMAs, so they are
// issued early and their latency hides under the matrix work.
template <int NR, int NM, int RPM, int T = 0>
__device__ __forceinline__ void interleave_reads_mfma() {
    constexpr int G = (NR + RPM - 1) / RPM;  // MFMAs that carry reads
    if constexpr (T < G && T < NM) {
        constexpr int nr = (T + 1) * RPM <= NR ? RPM : NR - T * RPM;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, nr, 0);  // DS read
        interleave_reads_mfma<NR, NM, RPM, T + 1>();
    } else if constexpr (NM > T) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM - T, 0);
    }
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// Workgroup barrier without a memory fence: the wave's own LDS reads are
// waited for (lgkmcnt 0, no other counter), then s_barrier; compiler-only
// fences keep every LDS access on its side.  Global->LDS copies in flight
// stay in flight (__syncthreads() would wait for them).
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7: lgkmcnt(0) only
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <bool LIGHT>
__device__ __forceinline__ void epi_barrier() {
    if constexpr (LIGHT) lds_barrier(); else __syncthreads();
}


// E chunks of one epilogue band, in the order the combine pass reads them.
template <class C, int QN>
__device__ __forceinline__ void load_e_band(const Epi& ep, int64_t row0, int64_t col0, int band,
                                            uint4 (&e)[QN]) {
    const int64_t brow = row0 + (int64_t)band * C::RB;
#pragma unroll
    for (int q = 0; q < QN; ++q) {
        const int ch = q * C::NT + threadIdx.x;
        const int rr = ch / (C::BN / 8), c8 = (ch % (C::BN / 8)) * 8;
        e[q] = gld(reinterpret_cast<const uint4*>(ep.E + (brow + rr) * ep.ld_e + col0 + c8));
    }
}

// Epilogue through LDS, in bands of RB rows: the waves holding the band
// write their fp32 accumulators (MFMA 32x32 layout: lane l, register r is
// row (r & 3) + 4*(l >> 5) + 8*(r >> 2), column l & 31); then every thread
// combines 8 consecutive columns with E and stores 16 bytes of the output,
// and, for the transposed copy, 8 consecutive rows of one column.  sb: the
// fp32 band buffer (RB x BN).
//
// The band loop is unrolled so the compiler can count outstanding memory
// operations exactly: no wait ever covers the stores of earlier bands, and
// E is loaded one band ahead so its latency hides behind the LDS work.
// LIGHT: the band barriers carry no memory fence, for a caller that has
// global->LDS copies in flight into other arrays which the epilogue must not
// wait for.
// (wm, wn): the wave's position in the WM x WN grid; frow = lane & 31,
// khalf = lane >> 5.
template <class C, bool HAS_E, bool F32OUT, bool LIGHT = false>
__device__ __forceinline__ void epilogue_bands(const f32x16 (&acc)[C::FM][C::FN], int64_t row0,
                                               int64_t col0, const Epi& ep, float* sb, int wm,
                                               int wn, int frow, int khalf) {
    constexpr int QN = (C::RB * C::BN / 8) / C::NT;  // 16-byte chunks per thread per band
    uint4 ecur[QN], enxt[QN];
    if (HAS_E) load_e_band<C, QN>(ep, row0, col0, 0, ecur);
#pragma unroll
    for (int band = 0; band < C::BM / C::RB; ++band) {
        if (HAS_E && band + 1 < C::BM / C::RB) load_e_band<C, QN>(ep, row0, col0, band + 1, enxt);
        epi_barrier<LIGHT>();
        // the band is MFMA row block i of the waves with wm * TM + 32 i == 32 band
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            if (wm * C::TM + i * 32 == band * C::RB) {
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const int c = wn * C::TN + j * 32 + frow;
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        const int rr = 8 * (r >> 2) + 4 * khalf + (r & 3);
                        sb[sbi<C>(rr, c)] = acc[i][j][r];
                    }
                }
            }
        }
        epi_barrier<LIGHT>();
        const int64_t brow = row0 + (int64_t)band * C::RB;
#pragma unroll
        for (int q = 0; q < (C::RB * C::BN / 8) / C::NT; ++q) {
            const int ch = q * C::NT + threadIdx.x;
            const int rr = ch / (C::BN / 8), c8 = (ch % (C::BN / 8)) * 8;
            const float4 a0 = *reinterpret_cast<const float4*>(sb + sbi<C>(rr, c8));
            const float4 a1 = *reinterpret_cast<const float4*>(sb + sbi<C>(rr, c8) + 4);
            float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            if (HAS_E) {
                const uint32_t ew[4] = {ecur[q].x, ecur[q].y, ecur[q].z, ecur[q].w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const uint32_t w = ew[e >> 1];
                    const float xe = __builtin_bit_cast(float, (e & 1) ? (w & 0xffff0000u) : (w << 16));
                    v[e] = ep.post * (ep.coef_acc * v[e] + ep.coef_e * xe);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = ep.post * (ep.coef_acc * v[e]);
            }
            if (ep.diag != 0.f) {
                const int64_t dc = brow + rr - (col0 + c8);  // column of the diagonal, relative
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] += (dc == e) ? ep.diag : 0.f;
            }
            if constexpr (F32OUT) {
                // a partial tile of a K-split Gram: fp32, tile-local, no mirror
                float* o = ep.outF + (int64_t)(band * C::RB + rr) * C::BN + c8;
                gst(reinterpret_cast<float4*>(o), make_float4(v[0], v[1], v[2], v[3]));
                gst(reinterpret_cast<float4*>(o + 4), make_float4(v[4], v[5], v[6], v[7]));
                continue;
            }
            uint4 o;
            o.x = pack2(v[0], v[1]);
            o.y = pack2(v[2], v[3]);
            o.z = pack2(v[4], v[5]);
            o.w = pack2(v[6], v[7]);
            store_out(ep.out + brow * ep.ld_out + col0, (uint32_t)(rr * ep.ld_out + c8) * 2u, o);
            if (ep.outT) {
                *reinterpret_cast<float4*>(sb + sbi<C>(rr, c8)) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4*>(sb + sbi<C>(rr, c8) + 4) = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
        if (!F32OUT && ep.outT) {
            epi_barrier<LIGHT>();
#pragma unroll
            for (int q = 0; q < (C::BN * C::RB / 8) / C::NT; ++q) {
                const int ch = q * C::NT + threadIdx.x;
                const int c = ch / (C::RB / 8), i8 = (ch % (C::RB / 8)) * 8;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = sb[sbi<C>(i8 + e, c)];
                uint4 o;
                o.x = pack2(v[0], v[1]);
                o.y = pack2(v[2], v[3]);
                o.z = pack2(v[4], v[5]);
                o.w = pack2(v[6], v[7]);
                store_out(ep.outT + col0 * ep.ld_outT + brow, (uint32_t)(c * ep.ld_outT + i8) * 2u, o);
            }
        }
        if (HAS_E) {
#pragma unroll
            for (int q = 0; q < QN; ++q) ecur[q] = enxt[q];
        }
    }
}

// C tile = sum_k P[i][k] Q'[k][j] for the BM rows starting at P0 (leading
// dimension ldp) and BN columns of Q' (K a multiple of BK), then the
// epilogue.  Q' is read as Q'[k][j] = Q0[j * ldq + k] (NT) or, with QKN, as
// Q0[k * ldq + j] (k-major).
template <class C, bool HAS_E, bool QKN = false, bool F32OUT = false, bool SAME = false>
__device__ __forceinline__ void gemm_tile(const uint16_t* __restrict__ P0, int64_t ldp,
                                          const uint16_t* __restrict__ Q0, int64_t ldq, int K,
                                          int64_t row0, int64_t col0, const Epi& ep,
                                          const Stages& st) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int frow = lane & 31;
    const int khalf = lane >> 5;

    f32x16 acc[C::FM][C::FN];
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Software pipeline.  All NS stages are filled up front; while the
    // MFMAs of k-step kk run, the fragments of k-step kk + 1 are read from
    // LDS into the other register buffer.  The fragments of a slab's last
    // k-step are read before the barrier that frees its stage and their
    // MFMAs are issued after it, so the matrix cores have queued work while
    // the waves meet.  The copy of slab kt + NS goes into the stage that slab
    // kt leaves.
    const int KT = K / C::BK;
    constexpr int KS = C::BK / 16;  // MFMA k-steps per slab (even)
#pragma unroll
    for (int u = 0; u < C::NS; ++u) {
        if (u < KT) {
            load_stage<C, QKN, SAME>(P0, ldp, Q0, ldq, (int64_t)u * C::BK, st, u, wave, lane);
        }
    }
    constexpr int LPS = SAME ? C::LPS1 : C::LPS;
    if (KT >= C::NS) wait_vmcnt<(C::NS - 1) * LPS>(); else wait_vmcnt<0>();
    __syncthreads();
    Frags<C> f[2];
    read_frags<C, QKN, SAME>(st, 0, 0, wm, wn, frow, khalf, lane, f[0]);

    for (int kt0 = 0; kt0 < KT; kt0 += C::NS) {
#pragma unroll
        for (int u = 0; u < C::NS; ++u) {
            const int kt = kt0 + u;
            if (kt < KT) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    if (kk + 1 < KS) {
                        read_frags<C, QKN, SAME>(st, u, kk + 1, wm, wn, frow, khalf, lane,
                                           f[(kk + 1) & 1]);
                    } else {
                        // slab kt + 1 has landed once only the copies of the
                        // slabs after it are outstanding; then every wave's.
                        // The last slab takes the same path (its reads of
                        // the next stage are unused) so every slab has one
                        // straight-line sequence of LDS waits.
                        if (kt + C::NS - 1 < KT) wait_vmcnt<(C::NS - 2) * LPS>(); else wait_vmcnt<0>();
                        __syncthreads();
                        if (kt + C::NS < KT) {
                            load_stage<C, QKN, SAME>(P0, ldp, Q0, ldq, (int64_t)(kt + C::NS) * C::BK,
                                               st, u, wave, lane);
                        }
                        read_frags<C, QKN, SAME>(st, (u + 1) % C::NS, 0, wm, wn, frow, khalf, lane, f[0]);
                    }
                    mfma_frags<C>(acc, f[kk & 1]);
                    // two reads with each of the first MFMAs: the reads go out early
                    // (k-major fragments are two reads each)
                    interleave_reads_mfma<C::FM + (QKN ? 2 : 1) * C::FN, C::FM * C::FN, 2>();
                }
            }
        }
    }

    float* sb = reinterpret_cast<float*>(lds_arr(st, 0));
    wait_vmcnt<0>();  // every slab copy has landed: the band buffer is free
    epilogue_bands<C, HAS_E, F32OUT>(acc, row0, col0, ep, sb, wm, wn, frow, khalf);
}

// Task of this workgroup under an XcdSplit: a whole tile (quarter = -1) or
// quarter q of a tile (rows (q >> 1), columns (q & 1) of its 2 x 2 split).
// False: no task, exit.
__device__ __forceinline__ bool xcd_task(const XcdSplit& xs, int& tile, int& quarter) {
    const int b = (int)blockIdx.x;
    const int x = b & 7;
    int t = b >> 3;
    const int full = xs.rounds * xs.cus;  // 0 unless interleaved
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

// The configuration that computes a quarter of a C tile (same waves, same
// threads, half the rows and columns).
template <class C>
using QuarterCfg = Cfg<C::BM / 2, C::BN / 2, C::WM, C::WN, C::BK, 4>;

// LDS arrays a kernel on tiles of C needs (with quarter tiles for 256 x 256).
template <class C>
constexpr int lds_arrays() {
    return C::BM == 256 ? (C::NARR > QuarterCfg<C>::NARR ? C::NARR : QuarterCfg<C>::NARR) : C::NARR;
}

__device__ __forceinline__ void tri_index(int lt, int& ti, int& tj) {
    int t = (int)((sqrtf(8.f * (float)lt + 1.f) - 1.f) * 0.5f);
    while (t * (t + 1) / 2 > lt) --t;
    while ((t + 1) * (t + 2) / 2 <= lt) ++t;
    ti = t;
    tj = lt - t * (t + 1) / 2;
}

// The Gram and polynomial launches take a matrix's triangle tiles in blocked
// order: super-rows of S tile-rows, and within one the S x S blocks left of
// the diagonal (row-major), then the diagonal block's triangle.  A super-row
// holds the same tiles as S rows of the row-major order, permuted, so a window
// of concurrent tiles on an XCD touches fewer operand row panels (measured on
// the Llama-style layer: Gram and polynomial 3% faster; unchanged on 4096^2
// batches, and the same order as row-major up to S tile-rows).
__device__ __forceinline__ void tri_index_blocked(int lt, int T, int& ti, int& tj) {
    constexpr int S = 8;
    int t, u;
    tri_index(lt, t, u);
    const int I = t / S;
    const int r = min(S, T - I * S);  // tile-rows in super-row I
    const int loc = lt - (I * S) * (I * S + 1) / 2;
    if (loc < r * S * I) {
        const int J = loc / (r * S), l2 = loc - J * r * S;
        ti = I * S + l2 / S;
        tj = J * S + l2 % S;
    } else {
        int a, b;
        tri_index(loc - r * S * I, a, b);
        ti = I * S + a;
        tj = I * S + b;
    }
}

// Update tiles in groups of kUpdGroup tile-rows: within a group the column
// index advances slowest, so concurrently running tiles reuse a few B
// row-panels and X column-panels.
constexpr int kUpdGroup = 8;
__device__ __forceinline__ void grouped_index(int lt, int trows, int tcols, int& ti, int& tj) {
    const int g = lt / (kUpdGroup * tcols);
    const int rows_in = min(kUpdGroup, trows - g * kUpdGroup);
    const int in = lt - g * kUpdGroup * tcols;
    ti = g * kUpdGroup + in % rows_in;
    tj = in / rows_in;
}

// Gram and polynomial: SYRK-like over the lower triangle of tiles.
template <class C, int PHASE>
__global__ __launch_bounds__(C::NT) void ns_sym_kernel(const MatDesc* __restrict__ descs, int n,
                                                       const int32_t* __restrict__ prefix,
                                                       XcdSplit xs, int it, float ca, float cb,
                                                       float cc) {
    constexpr int NA = lds_arrays<C>();
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[kLdsArr];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[NA > 1 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds2[NA > 2 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds3[NA > 3 ? kLdsArr : 8];
    const Stages st{{lds0, lds1, lds2, lds3}};
    int tile, q;
    if (!xcd_task(xs, tile, q)) return;
    const int mi = find_matrix(prefix, n, tile);
    const MatDesc& d = descs[mi];
    int ti, tj;
    tri_index_blocked(tile - prefix[mi], (int)(d.mp / C::BM), ti, tj);
    // a quarter above the diagonal of a diagonal tile is the mirror of the
    // quarter below it
    if (q >= 0 && ti == tj && (q >> 1) < (q & 1)) return;
    // the tile (or quarter) holds part of the diagonal: stored once, no mirror
    const bool on_diag = ti == tj && (q < 0 || (q >> 1) == (q & 1));
    const int64_t mp = d.mp, np = d.np;
    Epi ep;
    ep.outF = nullptr;
    ep.out = reinterpret_cast<uint16_t*>(PHASE == GRAM ? d.a : d.b);
    ep.ld_out = mp;
    ep.outT = on_diag ? nullptr : ep.out;
    ep.ld_outT = mp;
    const uint16_t* src;
    int64_t ld;
    if (PHASE == GRAM) {
        src = reinterpret_cast<const uint16_t*>(d.x[it & 1]);
        ld = np;
        const float s = (it == 0) ? gld(d.inv_norm) : 1.f;
        ep.E = nullptr;
        ep.ld_e = 0;
        ep.coef_e = 0.f;
        ep.coef_acc = s * s;
        ep.post = 1.f;
        ep.diag = 0.f;
    } else {
        src = reinterpret_cast<const uint16_t*>(d.a);
        ld = mp;
        ep.E = src;
        ep.ld_e = mp;
        ep.coef_e = cb;
        ep.coef_acc = cc;
        ep.post = 1.f;
        ep.diag = on_diag ? ca : 0.f;
    }
    // a tile (or quarter) on the diagonal multiplies the same rows by
    // themselves: one slab copy serves both operands
    if (q < 0) {
        const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
        if (on_diag)
            gemm_tile<C, PHASE == POLY, false, false, true>(src + r0 * ld, ld, src + c0 * ld, ld, (int)ld,
                                                             r0, c0, ep, st);
        else
            gemm_tile<C, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, (int)ld, r0, c0, ep, st);
    } else if constexpr (C::BM == 256) {
        using Q = QuarterCfg<C>;
        const int64_t r0 = (int64_t)ti * C::BM + (q >> 1) * Q::BM;
        const int64_t c0 = (int64_t)tj * C::BN + (q & 1) * Q::BN;
        if (on_diag)
            gemm_tile<Q, PHASE == POLY, false, false, true>(src + r0 * ld, ld, src + c0 * ld, ld, (int)ld,
                                                             r0, c0, ep, st);
        else
            gemm_tile<Q, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, (int)ld, r0, c0, ep, st);
    }
}

// K-split Gram (launches with fewer tiles than compute units): task t of a
// matrix is part t / T of triangle tile t % T (T tiles), i.e. the product
// over K slabs [part * slabs / S, (part + 1) * slabs / S) of S; its raw fp32
// tile goes to gram_part[t].  ns_gram_reduce_kernel then forms A.
template <class C>
__global__ __launch_bounds__(C::NT) void ns_gram_split_kernel(const MatDesc* __restrict__ descs, int n,
                                                              const int32_t* __restrict__ prefix,
                                                              XcdSplit xs, int it) {
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[kLdsArr];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[C::NARR > 1 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds2[C::NARR > 2 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds3[C::NARR > 3 ? kLdsArr : 8];
    const Stages st{{lds0, lds1, lds2, lds3}};
    int task, q;
    if (!xcd_task(xs, task, q)) return;  // no quarter tasks: the split launch fits one round
    const int mi = find_matrix(prefix, n, task);
    const MatDesc& d = descs[mi];
    const int lt = task - prefix[mi];
    const int64_t np = d.np;
    const int tm = (int)(d.mp / C::BM);
    const int T = tm * (tm + 1) / 2;
    const int part = lt / T;
    int ti, tj;
    tri_index(lt - part * T, ti, tj);
    const int S = d.gram_split;
    const int slabs = (int)(np / C::BK);
    const int64_t k0 = (int64_t)(part * slabs / S) * C::BK;
    const int64_t k1 = (int64_t)((part + 1) * slabs / S) * C::BK;
    const uint16_t* src = reinterpret_cast<const uint16_t*>(d.x[it & 1]);
    Epi ep;
    ep.outF = d.gram_part + (int64_t)lt * C::BM * C::BN;
    ep.out = nullptr;
    ep.ld_out = 0;
    ep.outT = nullptr;
    ep.ld_outT = 0;
    ep.E = nullptr;
    ep.ld_e = 0;
    ep.coef_e = 0.f;
    ep.coef_acc = 1.f;
    ep.post = 1.f;
    ep.diag = 0.f;
    const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
    if (ti == tj)
        gemm_tile<C, false, false, true, true>(src + r0 * np + k0, np, src + c0 * np + k0, np,
                                               (int)(k1 - k0), 0, 0, ep, st);
    else
        gemm_tile<C, false, false, true>(src + r0 * np + k0, np, src + c0 * np + k0, np, (int)(k1 - k0),
                                         0, 0, ep, st);
}

// Sum of the K-parts of a split Gram, in part order (so the result does not
// depend on timing), scaled by s^2 on the first iteration, rounded to bf16
// and stored into A at the tile and, off the diagonal, at its mirror.  One
// workgroup per 64 x 64 chunk of a triangle tile; thread t: row t / 4,
// columns 16 (t % 4) ... + 15 of the chunk.
template <int BT>
__global__ __launch_bounds__(256) void ns_gram_reduce_kernel(const MatDesc* __restrict__ descs, int n,
                                                             const int32_t* __restrict__ prefix_tri,
                                                             int it) {
    constexpr int CH = BT / 64;
    __shared__ float tr[64][65];
    const int g = blockIdx.x;
    const int tile = g / (CH * CH);
    const int chunk = g - tile * (CH * CH);
    const int mi = find_matrix(prefix_tri, n, tile);
    const MatDesc& d = descs[mi];
    const int lt = tile - prefix_tri[mi];
    const int T = prefix_tri[mi + 1] - prefix_tri[mi];
    int ti, tj;
    tri_index(lt, ti, tj);
    const int cr = chunk / CH, cc = chunk - cr * CH;
    const int S = d.gram_split;
    const int r = threadIdx.x >> 2, c16 = (threadIdx.x & 3) * 16;
    float v[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.f;
    for (int p = 0; p < S; ++p) {
        const float* src = d.gram_part + ((int64_t)(p * T + lt) * BT + cr * 64 + r) * BT + cc * 64 + c16;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = gld(reinterpret_cast<const float4*>(src + 4 * q));
            v[4 * q] += f.x;
            v[4 * q + 1] += f.y;
            v[4 * q + 2] += f.z;
            v[4 * q + 3] += f.w;
        }
    }
    const float s = it == 0 ? gld(d.inv_norm) : 1.f;
    const float s2 = s * s;
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] *= s2;
    uint16_t* A = reinterpret_cast<uint16_t*>(d.a);
    const int64_t lda = d.mp;
    const int64_t row = (int64_t)ti * BT + cr * 64 + r, col = (int64_t)tj * BT + cc * 64 + c16;
    uint4 o0, o1;
    o0.x = pack2(v[0], v[1]); o0.y = pack2(v[2], v[3]); o0.z = pack2(v[4], v[5]); o0.w = pack2(v[6], v[7]);
    o1.x = pack2(v[8], v[9]); o1.y = pack2(v[10], v[11]); o1.z = pack2(v[12], v[13]); o1.w = pack2(v[14], v[15]);
    gst(reinterpret_cast<uint4*>(A + row * lda + col), o0);
    gst(reinterpret_cast<uint4*>(A + row * lda + col + 8), o1);
    if (ti == tj) return;  // a diagonal tile is computed whole: no mirror
#pragma unroll
    for (int e = 0; e < 16; ++e) tr[r][c16 + e] = v[e];
    __syncthreads();
    float w[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) w[e] = tr[c16 + e][r];
    const int64_t trow = (int64_t)tj * BT + cc * 64 + r, tcol = (int64_t)ti * BT + cr * 64 + c16;
    o0.x = pack2(w[0], w[1]); o0.y = pack2(w[2], w[3]); o0.z = pack2(w[4], w[5]); o0.w = pack2(w[6], w[7]);
    o1.x = pack2(w[8], w[9]); o1.y = pack2(w[10], w[11]); o1.z = pack2(w[12], w[13]); o1.w = pack2(w[14], w[15]);
    gst(reinterpret_cast<uint4*>(A + trow * lda + tcol), o0);
    gst(reinterpret_cast<uint4*>(A + trow * lda + tcol + 8), o1);
}

template <class C>
__global__ __launch_bounds__(C::NT) void ns_update_kernel(const MatDesc* __restrict__ descs, int n,
                                                          const int32_t* __restrict__ prefix,
                                                          XcdSplit xs, int it) {
    constexpr int NA = lds_arrays<C>();
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[kLdsArr];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[NA > 1 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds2[NA > 2 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds3[NA > 3 ? kLdsArr : 8];
    const Stages st{{lds0, lds1, lds2, lds3}};
    int tile, q;
    if (!xcd_task(xs, tile, q)) return;
    const int mi = find_matrix(prefix, n, tile);
    const MatDesc& d = descs[mi];
    const int lt = tile - prefix[mi];
    const int64_t mp = d.mp, np = d.np;
    int ti, tj;
    grouped_index(lt, (int)(mp / C::BM), (int)(np / C::BN), ti, tj);
    const uint16_t* B = reinterpret_cast<const uint16_t*>(d.b);
    const uint16_t* X = reinterpret_cast<const uint16_t*>(d.x[it & 1]);
    Epi ep;
    ep.outF = nullptr;
    ep.out = reinterpret_cast<uint16_t*>(d.x[(it + 1) & 1]);
    ep.ld_out = np;
    ep.outT = nullptr;
    ep.ld_outT = 0;
    ep.E = nullptr;
    ep.ld_e = 0;
    ep.coef_e = 0.f;
    ep.coef_acc = 1.f;
    ep.post = (it == 0) ? gld(d.inv_norm) : 1.f;
    ep.diag = 0.f;
    if (q < 0) {
        const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
        gemm_tile<C, false, true>(B + r0 * mp, mp, X + c0, np, (int)mp, r0, c0, ep, st);
    } else if constexpr (C::BM == 256) {
        using Q = QuarterCfg<C>;
        const int64_t r0 = (int64_t)ti * C::BM + (q >> 1) * Q::BM;
        const int64_t c0 = (int64_t)tj * C::BN + (q & 1) * Q::BN;
        gemm_tile<Q, false, true>(B + r0 * mp, mp, X + c0, np, (int)mp, r0, c0, ep, st);
    }
}

// The products with the operand roles exchanged: acc[i][j] += Q-block j times
// P-block i, i.e. the transpose of the P Q' block.  Lane l, register r then
// holds row (l & 31) of the P block and column 8 (r >> 2) + 4 (l >> 5) +
// (r & 3) of the Q block: four consecutive columns of one row per group of
// four registers, which the strip epilogue stores without a pass through LDS.
template <class C>
__device__ __forceinline__ void mfma_frags_rows(f32x16 (&acc)[C::FM][C::FN], const Frags<C>& f) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.b[j], f.a[i], acc[i][j], 0, 0, 0);
}

// Strip epilogue, first half: the tile held in rows (mfma_frags_rows) is
// scaled, rounded to bf16 and written to LDS as two row slabs of 64 columns
// (xo[0], xo[1]; load_slab's layout), four columns (8 bytes) per write.
template <class C>
__device__ __forceinline__ void rows_to_slabs(const f32x16 (&acc)[C::FM][C::FN], const Epi& ep,
                                              int wm, int wn, int frow, int khalf,
                                              uint16_t* const* xo) {
    static_assert(C::BN == 128 && C::BK == 64 && C::TN == 64, "a wave's columns are one 64-column slab");
    // the wave's slab (a select, not an index, so the LDS address space is kept)
    uint16_t* const xs = wn == 0 ? xo[0] : xo[1];
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::TM + i * 32 + frow;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int lch = 4 * j + g;  // chunk of columns j * 32 + 8 g .. + 7 within the slab
                float v[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = ep.post * (ep.coef_acc * acc[i][j][4 * g + e]);
                const bf16x4 h = __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4);
                *reinterpret_cast<uint2*>(xs + row * C::BK + ((lch ^ swz<C::BK>(row)) << 3) + 4 * khalf) =
                    __builtin_bit_cast(uint2, h);
            }
        }
    }
}

// Second half: every thread reads 8 chunks of 16 bytes from the slabs, so
// that one wave's store covers 8 rows x 64 columns: eight whole 128-byte
// lines.  Chunk q of thread t: row 32 (q >> 1) + t / 8, slab q & 1, logical
// chunk t % 8 (16 lanes read two rows of one slab: all 64 banks once).
template <class C>
struct SlabRows {
    uint4 v[8];
};
template <class C>
__device__ __forceinline__ void read_slab_rows(uint16_t* const* xo, SlabRows<C>& r) {
    static_assert(C::NT == 256 && C::BM == 128, "8 chunks per thread cover the 128 x 128 tile");
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 32 * (q >> 1) + (t >> 3), lch = t & 7;
        const uint16_t* xs = (q & 1) ? xo[1] : xo[0];
        r.v[q] = *reinterpret_cast<const uint4*>(xs + row * C::BK + ((lch ^ swz<C::BK>(row)) << 3));
    }
}
template <class C>
__device__ __forceinline__ void store_slab_rows(const SlabRows<C>& r, int64_t col0, const Epi& ep) {
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 32 * (q >> 1) + (t >> 3), c = 64 * (q & 1) + 8 * (t & 7);
        store_out(ep.out + col0, (uint32_t)(row * ep.ld_out + c) * 2u, r.v[q]);
    }
}

// Update of the small class in strips.  Its matrices have m' = 128, so A and
// B are one 128 x 128 tile each and an update tile is B times one 128-column
// block of X (K = 128: two slabs).  A workgroup takes `strip` consecutive
// column tiles of one matrix.  It first forms B = a I + b A + c A A itself
// from A (the polynomial, 4 MFLOP, once per strip instead of a launch of its
// own), in LDS, then runs its tiles; the X block of the next tile is copied
// while the current tile's epilogue runs.  One tile per workgroup spent most
// of its time in the copy latency and the epilogue, one after the other.
//
// The products are held in rows (mfma_frags_rows), so the epilogue writes
// each tile once to LDS as bf16, in the X slabs the block has vacated, and
// stores it from there as whole 128-byte lines.
//
// NEXT_GRAM: the strip also forms its share of the next iteration's Gram.  A
// strip covers the same columns as one part of the K-split Gram (the planner
// makes the strip count per matrix equal the part count), so once a tile's
// bf16 values sit in LDS the workgroup multiplies them by themselves into a
// second accumulator, and stores that as its part's raw fp32 tile at the end:
// the values and the summation order of the split Gram, without reading X
// back from memory.
//
// LDS, in variables of their own so that the compiler can tell the copies
// into one from the accesses to another: A's (then B's) two slabs (32 KB),
// the X block's two k-major slabs (k 0..63, 64..127; later the tile's two
// 64-column row slabs; 16 KB each) and the fp32 band buffer of the final
// Gram store (16 KB).
template <class C, bool NEXT_GRAM>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(2, 2))) void ns_update_strip_kernel(
    const MatDesc* __restrict__ descs, int n, const int32_t* __restrict__ prefix, XcdSplit xs, int it,
    int strip, float ca, float cb, float cc) {
    static_assert(C::BM == 128 && C::BN == 128 && C::BK == 64 && C::NT == 256,
                  "two 64-deep slabs hold the whole K of 128");
    __shared__ __attribute__((aligned(1024))) uint16_t lp[2 * C::BM * C::BK];
    __shared__ __attribute__((aligned(1024))) uint16_t lx0[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) uint16_t lx1[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) float band[C::RB * C::BN];
    int task, q;
    if (!xcd_task(xs, task, q)) return;  // no quarter tasks
    const int mi = find_matrix(prefix, n, task);
    const MatDesc& d = descs[mi];
    const int64_t mp = d.mp, np = d.np;  // mp == 128
    const int tiles = (int)(np / C::BN);
    const int part = task - prefix[mi];
    const int j0 = part * strip;
    const int j1 = min(j0 + strip, tiles);
    const uint16_t* A = reinterpret_cast<const uint16_t*>(d.a);
    const uint16_t* X = reinterpret_cast<const uint16_t*>(d.x[it & 1]);
    Epi ep;
    ep.outF = nullptr;
    ep.out = reinterpret_cast<uint16_t*>(d.x[(it + 1) & 1]);
    ep.ld_out = np;
    ep.outT = nullptr;
    ep.ld_outT = 0;
    ep.E = nullptr;
    ep.ld_e = 0;
    ep.coef_e = 0.f;
    ep.coef_acc = 1.f;
    ep.post = (it == 0) ? gld(d.inv_norm) : 1.f;
    ep.diag = 0.f;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int frow = lane & 31;
    const int khalf = lane >> 5;
    constexpr int KS = C::BK / 16;
    uint16_t* const xo[2] = {lx0, lx1};
    uint16_t* const lp0 = lp;
    uint16_t* const lp1 = lp + C::BM * C::BK;
    // fragments of k-step kk of slab u: rows of the (A or B) slab against rows
    // of the same slab (RR), or against the k-major X block (else)
    auto frags = [&](int u, int kk, bool xkn, bool xrows, Frags<C>& f) {
        const uint16_t* sp = xrows ? (u ? lx1 : lx0) : (u ? lp1 : lp0);
        const uint16_t* sq = (xkn || xrows) ? (u ? lx1 : lx0) : sp;
        const int lch = 2 * kk + khalf;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) f.a[i] = read_frag<C>(sp, wm * C::TM + i * 32 + frow, lch);
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj)
            f.b[jj] = xkn ? read_frag_kn<C>(sq, 16 * kk, wn * C::TN + jj * 32, lane)
                          : read_frag<C>(sq, wn * C::TN + jj * 32 + frow, lch);
    };
    f32x16 acc[C::FM][C::FN];
    f32x16 accg[C::FM][C::FN];
    auto zero = [](f32x16(&t)[C::FM][C::FN]) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) t[i][jj][r] = 0.f;
    };
    if constexpr (NEXT_GRAM) zero(accg);

    // A's slabs, then the first X block; A is waited for alone
    load_slab<C, C::BM>(A, mp, lp0, wave, lane);
    load_slab<C, C::BM>(A + C::BK, mp, lp1, wave, lane);
    load_slab_kn<C>(X + (int64_t)j0 * C::BN, np, lx0, wave, lane);
    load_slab_kn<C>(X + (int64_t)C::BK * np + (int64_t)j0 * C::BN, np, lx1, wave, lane);
    constexpr int LX = 2 * ((C::BK / (64 / (C::BN / 8))) / C::NW);  // this wave's X copies
    wait_vmcnt<LX>();
    lds_barrier();
    // B = a I + b A + c A A (the polynomial's epilogue arithmetic), written
    // over A in place once every wave has read A
    {
        zero(acc);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                Frags<C> f;
                frags(u, kk, false, false, f);
                mfma_frags_rows<C>(acc, f);
            }
        // The wave's columns wn*64 .. +63 of A are slab wn; a lane's four
        // columns are half khalf of chunk 4 jj + g of its row.  LDS is read
        // and written in whole 16-byte chunks: lanes l and l + 32 trade halves
        // (chunk g of a pair goes through lane l, chunk g + 1 through lane
        // l + 32).  Paired 8-byte accesses would be merged into one
        // instruction, which the compiler's copy tracking cannot tell apart
        // from the X copies in flight; it would wait for those.
        auto trade = [](uint2 v) {
            return make_uint2((uint32_t)__shfl_xor((int)v.x, 32, 64), (uint32_t)__shfl_xor((int)v.y, 32, 64));
        };
        auto poly_epilogue = [&](uint16_t* ps) {
            uint2 e[C::FM][C::FN][4];
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < C::FN; ++jj)
#pragma unroll
                    for (int gp = 0; gp < 4; gp += 2) {
                        const int row = wm * C::TM + i * 32 + frow;
                        const int ck = 4 * jj + gp + khalf;
                        const uint4 r = *reinterpret_cast<const uint4*>(ps + row * C::BK + ((ck ^ swz<C::BK>(row)) << 3));
                        const uint2 lo = make_uint2(r.x, r.y), hi = make_uint2(r.z, r.w);
                        const uint2 got = trade(khalf ? lo : hi);
                        e[i][jj][gp] = khalf ? got : lo;
                        e[i][jj][gp + 1] = khalf ? hi : got;
                    }
            lds_barrier();  // every wave has read A
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int jj = 0; jj < C::FN; ++jj) {
                    const int row = wm * C::TM + i * 32 + frow;
                    uint2 o[4];
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        const int col = wn * C::TN + jj * 32 + 8 * g + 4 * khalf;
                        const uint32_t w[2] = {e[i][jj][g].x, e[i][jj][g].y};
                        float v[4];
#pragma unroll
                        for (int t = 0; t < 4; ++t) {
                            const uint32_t h = w[t >> 1];
                            const float av = __builtin_bit_cast(float, (t & 1) ? (h & 0xffff0000u) : (h << 16));
                            v[t] = 1.f * (cc * acc[i][jj][4 * g + t] + cb * av);
                            if (row == col + t) v[t] += ca;
                        }
                        o[g] = __builtin_bit_cast(uint2, __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4));
                    }
#pragma unroll
                    for (int gp = 0; gp < 4; gp += 2) {
                        const int ck = 4 * jj + gp + khalf;
                        const uint2 got = trade(khalf ? o[gp] : o[gp + 1]);
                        const uint4 wv = khalf ? make_uint4(got.x, got.y, o[gp + 1].x, o[gp + 1].y)
                                               : make_uint4(o[gp].x, o[gp].y, got.x, got.y);
                        *reinterpret_cast<uint4*>(ps + row * C::BK + ((ck ^ swz<C::BK>(row)) << 3)) = wv;
                    }
                }
        };
        poly_epilogue(lp + wn * (C::BM * C::BK));
    }

    for (int j = j0; j < j1; ++j) {
        wait_vmcnt<0>();  // this tile's X has landed (and the last tile's stores)
        __syncthreads();  // ... in every wave; B is written
        zero(acc);
#pragma unroll
        for (int u = 0; u < 2; ++u)
#pragma unroll
            for (int kk = 0; kk < KS; ++kk) {
                Frags<C> f;
                frags(u, kk, true, false, f);
                mfma_frags_rows<C>(acc, f);
            }
        // the tile's bf16 values go to the X slabs this block has vacated;
        // from there they are stored (and, for NEXT_GRAM, multiplied into the
        // Gram accumulator) before the next X block is copied in
        lds_barrier();  // every wave is done with this X block
        rows_to_slabs<C>(acc, ep, wm, wn, frow, khalf, xo);
        lds_barrier();
        SlabRows<C> out;
        read_slab_rows<C>(xo, out);
        if constexpr (NEXT_GRAM) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    Frags<C> f;
                    frags(u, kk, false, true, f);
                    mfma_frags<C>(accg, f);
                }
        }
        lds_barrier();  // the tile's slabs are read: the next X block may go there
        if (j + 1 < j1) {
            load_slab_kn<C>(X + (int64_t)(j + 1) * C::BN, np, lx0, wave, lane);
            load_slab_kn<C>(X + (int64_t)C::BK * np + (int64_t)(j + 1) * C::BN, np, lx1, wave, lane);
        }
        store_slab_rows<C>(out, (int64_t)j * C::BN, ep);
    }
    if constexpr (NEXT_GRAM) {
        // this strip's part of the next Gram: raw fp32, as the K-split Gram stores it
        Epi eg;
        eg.outF = d.gram_part + (int64_t)part * C::BM * C::BN;
        eg.out = nullptr;
        eg.ld_out = 0;
        eg.outT = nullptr;
        eg.ld_outT = 0;
        eg.E = nullptr;
        eg.ld_e = 0;
        eg.coef_e = 0.f;
        eg.coef_acc = 1.f;
        eg.post = 1.f;
        eg.diag = 0.f;
        epilogue_bands<C, false, true, true>(accg, 0, 0, eg, band, wm, wn, frow, khalf);
    }
}

// The streaming strip kernel's epilogue, first half: the tile held in rows
// (mfma_frags_rows) is scaled, rounded to bf16 and written to LDS as two row
// slabs of 64 columns (x0, x1, two arrays; load_slab's layout).  The
// streaming kernel gives wave (wm, wn) the
// column blocks 64 jj + 32 wn .. + 31 (jj = 0, 1), so block jj lies in slab
// jj whatever the wave and every write names its array at compile time.
// Lanes l and l + 32 hold the two halves (four columns each) of the same
// 8-column chunks of one row; v_permlane32_swap trades them so that every
// lane writes one whole chunk of 16 bytes: lane l chunk g, lane l + 32 chunk
// g + 1, for g = 0, 2.  (Pairs of 8-byte writes would be merged into one
// instruction whose target the compiler's copy tracking cannot place; it
// would wait for every copy in flight.)
template <class C>
__device__ __forceinline__ void rows_to_slab_pair(const f32x16 (&acc)[C::FM][C::FN], const Epi& ep,
                                              int wm, int wn, int frow, int khalf, uint16_t* x0,
                                              uint16_t* x1) {
    static_assert(C::BN == 128 && C::BK == 64 && C::FN == 2, "one 32-column block per slab and wave");
    auto half = [&](const f32x16& a, int g) {
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ep.post * (ep.coef_acc * a[4 * g + e]);
        return __builtin_bit_cast(uint2, __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4));
    };
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        const int row = wm * C::TM + i * 32 + frow;
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            uint16_t* const xs = j ? x1 : x0;
#pragma unroll
            for (int g = 0; g < 4; g += 2) {
                const uint2 x = half(acc[i][j], g), y = half(acc[i][j], g + 1);
                const auto sx = __builtin_amdgcn_permlane32_swap(x.x, y.x, false, false);
                const auto sy = __builtin_amdgcn_permlane32_swap(x.y, y.y, false, false);
                const int lch = 4 * wn + g + khalf;  // chunk of columns 8 lch .. + 7 within the slab
                *reinterpret_cast<uint4*>(xs + row * C::BK + ((lch ^ swz<C::BK>(row)) << 3)) =
                    make_uint4(sx[0], sy[0], sx[1], sy[1]);
            }
        }
    }
}

// Second half: as read_slab_rows, from two arrays.
template <class C>
__device__ __forceinline__ void read_slab_pair(const uint16_t* x0, const uint16_t* x1, SlabRows<C>& r) {
    static_assert(C::NT == 256 && C::BM == 128, "8 chunks per thread cover the 128 x 128 tile");
    const int t = threadIdx.x;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int row = 32 * (q >> 1) + (t >> 3), lch = t & 7;
        const uint16_t* xs = (q & 1) ? x1 : x0;
        r.v[q] = *reinterpret_cast<const uint4*>(xs + row * C::BK + ((lch ^ swz<C::BK>(row)) << 3));
    }
}
// The tile's values as the streaming kernel's APPLY variant reads them:
// chunk k of thread t is 4 columns 4 (t % 16) of slab k & 1 in row
// 16 (k >> 1) + t / 16, so that a wave's 64 lanes cover 4 rows x 64 columns
// and its 16-byte fp32 accesses to W whole 128-byte lines.  The offsets are
// laundered one by one: two reads a fixed distance apart would be merged into
// one instruction that the compiler's copy tracking cannot place.
template <class C>
struct SlabQuads {
    uint2 v[16];
};
template <class C>
__device__ __forceinline__ void read_slab_quads(const uint16_t* x0, const uint16_t* x1, SlabQuads<C>& r) {
    static_assert(C::NT == 256 && C::BM == 128 && C::BK == 64, "16 chunks per thread cover the 128 x 128 tile");
    const int t = threadIdx.x;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        const int row = 16 * (k >> 1) + (t >> 4), c4 = t & 15;
        int off = row * C::BK + ((((c4 >> 1) ^ swz<C::BK>(row)) << 3) | ((c4 & 1) << 2));
        asm volatile("" : "+v"(off));
        const uint16_t* xs = (k & 1) ? x1 : x0;
        r.v[k] = *reinterpret_cast<const uint2*>(xs + off);
    }
}
// The small class's update in strips when the class runs alone in a call:
// the same work as ns_update_strip_kernel (B formed in the strip, the next
// Gram's part, the tile's values stored from LDS as whole lines), but one
// workgroup per compute unit, with twice the tiles per strip, streams its
// tiles: the X blocks go through three LDS stages, so the copies of the next
// two blocks are in flight while a tile is multiplied, written out and
// (NEXT_GRAM) multiplied into the Gram part.  With half the strips, the
// class's K-split Gram has half the parts to write and reduce.  (Beside a
// large class on the other stream, two workgroups per compute unit share
// the chip better: ns_update_strip_kernel.)
//
// The tile's values go into the X slabs its block has vacated and are
// stored at the start of the next tile, after the wait for that tile's X
// block (which then never has to cover them).  The stage takes the block
// three tiles on once the tile's values have been read out.
//
// NEXT_GRAM: as in ns_update_strip_kernel, the planner makes the part count
// of the class's K-split Gram equal the strip count per matrix.
//
// APPLY (the last iteration, fp32 weights of exactly 128 x 128k, not
// transposed, no QK-Clip, no separate update output): instead of storing X,
// each tile updates its block of W in place, W <- decay W - lr scale X, with
// X rounded to bf16 first, as the apply kernel does.  W goes through
// registers: a tile's block of W is loaded at the end of the tile before,
// ahead of that tile's copy of the X block three tiles on, and the tile
// applies it at its own end, once its values are out of LDS; waiting for
// those loads then leaves the next X block's copies in flight.
//
// LDS (128 KB) in eight arrays of 16 KB, each a copy target of its own:
// A's (then B's) two slabs and three stages of the X block's two k-major
// slabs (k 0..63, 64..127; later the tile's two 64-column row slabs).  The
// compiler tracks copies into LDS per array, for at most eight arrays, and
// places its own waits before LDS accesses by the copies that may still be
// in flight on any path it can see.  So every access names its array, the
// tile loop is unrolled over the three stages, and its body has no
// conditional copy or store: the first tile and the last few are issued
// apart, with their conditions.
template <class C, bool NEXT_GRAM, bool APPLY>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(1, 1))) void ns_update_stream_kernel(
    const MatDesc* __restrict__ descs, int n, const int32_t* __restrict__ prefix, XcdSplit xs, int it,
    int strip, float ca, float cb, float cc, float decay, float lr) {
    static_assert(C::BM == 128 && C::BN == 128 && C::BK == 64 && C::NT == 256,
                  "two 64-deep slabs hold the whole K of 128");
    static_assert(!(NEXT_GRAM && APPLY), "only the last iteration applies");
    static_assert(C::RB * C::BN * 4 <= C::BK * C::BN * 2, "the Gram band fits one slab");
    __shared__ __attribute__((aligned(1024))) uint16_t lp0[C::BM * C::BK];
    __shared__ __attribute__((aligned(1024))) uint16_t lp1[C::BM * C::BK];
    __shared__ __attribute__((aligned(1024))) uint16_t la0[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) uint16_t la1[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) uint16_t lb0[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) uint16_t lb1[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) uint16_t lc0[C::BK * C::BN];
    __shared__ __attribute__((aligned(1024))) uint16_t lc1[C::BK * C::BN];
    int task, q;
    if (!xcd_task(xs, task, q)) return;  // no quarter tasks
    const int mi = find_matrix(prefix, n, task);
    const MatDesc& d = descs[mi];
    const int64_t mp = d.mp, np = d.np;  // mp == 128
    const int tiles = (int)(np / C::BN);
    const int part = task - prefix[mi];
    const int j0 = part * strip;
    const int j1 = min(j0 + strip, tiles);
    const uint16_t* A = reinterpret_cast<const uint16_t*>(d.a);
    const uint16_t* X = reinterpret_cast<const uint16_t*>(d.x[it & 1]);
    Epi ep;
    ep.outF = nullptr;
    ep.out = reinterpret_cast<uint16_t*>(d.x[(it + 1) & 1]);
    ep.ld_out = np;
    ep.outT = nullptr;
    ep.ld_outT = 0;
    ep.E = nullptr;
    ep.ld_e = 0;
    ep.coef_e = 0.f;
    ep.coef_acc = 1.f;
    ep.post = (it == 0) ? gld(d.inv_norm) : 1.f;
    ep.diag = 0.f;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    // the wave's place in the 2 x 2 grid; its product columns are the
    // blocks 64 jj + 32 wn .. + 31 (jj = 0, 1), one in each 64-column slab
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int frow = lane & 31;
    const int khalf = lane >> 5;
    constexpr int KS = C::BK / 16;
    f32x16 acc[C::FM][C::FN];
    f32x16 accg[C::FM][C::FN];
    auto zero = [](f32x16(&t)[C::FM][C::FN]) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj)
#pragma unroll
                for (int r = 0; r < 16; ++r) t[i][jj][r] = 0.f;
    };
    // fragments of k-step kk: rows of sp against rows of sq, or (QKN)
    // against the k-major X slab sq.  SPLIT: the wave's column blocks one per
    // slab (the products written to LDS: B and the tile); else the usual 64
    // contiguous columns (the Gram part, stored by epilogue_bands)
    auto frags = [&](const uint16_t* sp, const uint16_t* sq, int kk, bool qkn, bool split, Frags<C>& f) {
        const int lch = 2 * kk + khalf;
#pragma unroll
        for (int i = 0; i < C::FM; ++i) f.a[i] = read_frag<C>(sp, wm * C::TM + i * 32 + frow, lch);
#pragma unroll
        for (int jj = 0; jj < C::FN; ++jj) {
            const int c0 = split ? 64 * jj + 32 * wn : wn * C::TN + jj * 32;
            f.b[jj] = qkn ? read_frag_kn<C>(sq, 16 * kk, c0, lane) : read_frag<C>(sq, c0 + frow, lch);
        }
    };
    // the products over both slabs (K = 128), software-pipelined: while the
    // MFMAs of one k-step run, the fragments of the next are read into the
    // other register buffer (one wave per SIMD: no other wave hides the LDS
    // latency).  ROWS: the products held in rows (mfma_frags_rows).
    auto product = [&](auto rows, const uint16_t* p0, const uint16_t* p1, const uint16_t* q0,
                       const uint16_t* q1, auto qkn, bool split, f32x16(&a)[C::FM][C::FN])
                       __attribute__((always_inline)) {
        constexpr bool QK = decltype(qkn)::value;
        Frags<C> f[2];
        frags(p0, q0, 0, QK, split, f[0]);
#pragma unroll
        for (int st = 0; st < 2 * KS; ++st) {
            if (st + 1 < 2 * KS) {
                const int u = (st + 1) / KS, kk = (st + 1) % KS;
                frags(u ? p1 : p0, u ? q1 : q0, kk, QK, split, f[(st + 1) & 1]);
            }
            if constexpr (decltype(rows)::value) mfma_frags_rows<C>(a, f[st & 1]);
            else mfma_frags<C>(a, f[st & 1]);
            interleave_reads_mfma<C::FM + (QK ? 2 : 1) * C::FN, C::FM * C::FN, 2>();
        }
    };
    auto copy_x = [&](int j, uint16_t* s0, uint16_t* s1) {
        load_slab_kn<C>(X + (int64_t)j * C::BN, np, s0, wave, lane);
        load_slab_kn<C>(X + (int64_t)C::BK * np + (int64_t)j * C::BN, np, s1, wave, lane);
    };
    if constexpr (NEXT_GRAM) zero(accg);
    // APPLY: W's values under a thread's 16 chunks of 4 columns (SlabQuads:
    // row 16 (k >> 1) + t / 16, columns 64 (k & 1) + 4 (t % 16)), one 16-byte
    // buffer load each (buffer, not flat, accesses: a flat one counts as an
    // LDS access too, and its wait would cover every copy in flight).  The
    // planner keeps the byte offsets below 2 GB.
    const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(APPLY ? d.param : nullptr, 0,
                                                                         0x7fffffff, 0x00020000);
    const int64_t ldw = d.ld_param;
    const float sc = lr * d.scale;
    auto w_off = [&](int j, int k) {
        const int t = threadIdx.x;
        return (uint32_t)(((int64_t)(16 * (k >> 1) + (t >> 4)) * ldw + (int64_t)j * C::BN + 64 * (k & 1) +
                           4 * (t & 15)) * 4);
    };
    auto load_w = [&](int j, f32x4 (&w)[16]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < 16; ++k)
            w[k] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(wr, w_off(j, k), 0, 2));
    };
    // tile j's new W from its values x and its W in w; then (LOADW) tile wj's
    // W is loaded into w, and the new values stored
    auto apply_w = [&](int j, const SlabQuads<C>& x, f32x4 (&w)[16], auto loadw, int wj)
                       __attribute__((always_inline)) {
        f32x4 o[16];
#pragma unroll
        for (int k = 0; k < 16; ++k)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t b = (e >> 1) ? x.v[k].y : x.v[k].x;
                const float xv = __builtin_bit_cast(float, (e & 1) ? (b & 0xffff0000u) : (b << 16));
                o[k][e] = __builtin_fmaf(decay, w[k][e], -(sc * xv));
            }
        if constexpr (decltype(loadw)::value) load_w(wj, w);
#pragma unroll
        for (int k = 0; k < 16; ++k)
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(GWord<16>::T, o[k]), wr, w_off(j, k), 0,
                                                   kStreamStore);
    };
    f32x4 wv[16];

    // A's slabs, then the first three X blocks (a strip shorter than three
    // tiles copies its last block again); A is waited for alone
    constexpr int LX = 2 * ((C::BK / (64 / (C::BN / 8))) / C::NW);  // a thread's copies of one X block
    load_slab<C, C::BM>(A, mp, lp0, wave, lane);
    load_slab<C, C::BM>(A + C::BK, mp, lp1, wave, lane);
    copy_x(j0, la0, la1);
    wait_vmcnt<LX>();
    copy_x(min(j0 + 1, j1 - 1), lb0, lb1);
    copy_x(min(j0 + 2, j1 - 1), lc0, lc1);
    if constexpr (APPLY) load_w(j0, wv);
    lds_barrier();
    // B = a I + b A + c A A (the polynomial's epilogue arithmetic), written
    // over A in place once every wave has read A
    {
        zero(acc);
        product(std::true_type{}, lp0, lp1, lp0, lp1, std::false_type{}, true, acc);
        // The wave's column block jj is columns 32 wn .. + 31 of slab jj; a
        // lane's four columns are half khalf of chunk 4 wn + g of its row.
        // LDS is read and written in whole 16-byte chunks, lanes l and l + 32
        // trading halves with v_permlane32_swap (chunk g of a pair goes
        // through lane l, chunk g + 1 through lane l + 32): paired 8-byte
        // accesses would be merged into one instruction, and a lane exchange
        // through LDS (ds_bpermute) is an LDS access too; the compiler's copy
        // tracking places neither, and would wait for the X copies in flight.
        auto swap2 = [](uint2 p, uint2 q, uint2& p2, uint2& q2) {
            const auto sx = __builtin_amdgcn_permlane32_swap(p.x, q.x, false, false);
            const auto sy = __builtin_amdgcn_permlane32_swap(p.y, q.y, false, false);
            p2 = make_uint2(sx[0], sy[0]);
            q2 = make_uint2(sx[1], sy[1]);
        };
        uint2 e[C::FM][C::FN][4];
        // slab by slab, each from its own array
        auto read_a = [&](const uint16_t* ps, uint2 (&es)[C::FM][4]) {
#pragma unroll
            for (int i = 0; i < C::FM; ++i)
#pragma unroll
                for (int gp = 0; gp < 4; gp += 2) {
                    const int row = wm * C::TM + i * 32 + frow;
                    const int ck = 4 * wn + gp + khalf;
                    const uint4 r = *reinterpret_cast<const uint4*>(ps + row * C::BK + ((ck ^ swz<C::BK>(row)) << 3));
                    // lane l: half 0 of chunks gp (its own) and gp + 1 (lane
                    // l + 32's); lane l + 32: half 1 of both
                    swap2(make_uint2(r.x, r.y), make_uint2(r.z, r.w), es[i][gp], es[i][gp + 1]);
                }
        };
        uint2 e0[C::FM][4], e1[C::FM][4];
        read_a(lp0, e0);
        read_a(lp1, e1);
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                e[i][0][g] = e0[i][g];
                e[i][1][g] = e1[i][g];
            }
        lds_barrier();  // every wave has read A
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int jj = 0; jj < C::FN; ++jj) {
                uint16_t* const ps = jj ? lp1 : lp0;
                const int row = wm * C::TM + i * 32 + frow;
                uint2 o[4];
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int col = 64 * jj + 32 * wn + 8 * g + 4 * khalf;
                    const uint32_t w[2] = {e[i][jj][g].x, e[i][jj][g].y};
                    float v[4];
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const uint32_t h = w[t >> 1];
                        const float av = __builtin_bit_cast(float, (t & 1) ? (h & 0xffff0000u) : (h << 16));
                        v[t] = 1.f * (cc * acc[i][jj][4 * g + t] + cb * av);
                        if (row == col + t) v[t] += ca;
                    }
                    o[g] = __builtin_bit_cast(uint2, __builtin_convertvector(f32x4{v[0], v[1], v[2], v[3]}, bf16x4));
                }
#pragma unroll
                for (int gp = 0; gp < 4; gp += 2) {
                    const int ck = 4 * wn + gp + khalf;
                    uint2 lo, hi;
                    swap2(o[gp], o[gp + 1], lo, hi);
                    *reinterpret_cast<uint4*>(ps + row * C::BK + ((ck ^ swz<C::BK>(row)) << 3)) =
                        make_uint4(lo.x, lo.y, hi.x, hi.y);
                }
            }
    }

    // One tile: its X block is in stage (s0, s1).  Copies of up to two
    // later blocks stay in flight across the wait: loads land in the order
    // issued, so once no more than AHEAD blocks' copies are outstanding, this
    // block's have landed, and every store issued since only makes the count
    // smaller.  FIRST: the strip's first tile (nothing to store yet).  COPY:
    // at the end the tile's stage takes block `next`.
    // Every count and condition is fixed per call site, except in the
    // strip's first tile: the compiler places its own waits by the copies in
    // flight on every path it can see, and a copy that it cannot prove
    // issued would cost a full wait in the tiles after it.
    // APPLY: 16 W loads follow the prologue's copies and precede each copy
    // at a tile's end, so a wait leaving AH blocks' copies in flight may
    // leave WX = 16 more loads (at least 16 more than that were issued after
    // any block a tile waits for; counting fewer only waits longer).
    // LOADW: at its end the tile loads W of tile wj.
    constexpr int WX = APPLY ? 16 : 0;
    SlabRows<C> out;
    SlabQuads<C> outq;
    auto tile = [&](auto ahead, auto first, auto copy, int j, int next, uint16_t* s0, uint16_t* s1,
                    auto loadw, int wj) __attribute__((always_inline)) {
        constexpr int AH = decltype(ahead)::value;
        if constexpr (AH >= 2) wait_vmcnt<2 * LX + WX>();
        else if constexpr (AH == 1) wait_vmcnt<LX + WX>();
        else if constexpr (AH == 0) wait_vmcnt<WX>();
        else {  // the first tile: blocks j0 + 1 and j0 + 2 are copied if they exist
            const int ah = min(2, j1 - 1 - j);
            if (ah >= 2) wait_vmcnt<2 * LX + WX>();
            else if (ah == 1) wait_vmcnt<LX + WX>();
            else wait_vmcnt<WX>();
        }
        lds_barrier();  // X(j) in every wave; B written; the last tile's values read
        if constexpr (!APPLY && !decltype(first)::value) store_slab_rows<C>(out, (int64_t)(j - 1) * C::BN, ep);
        zero(acc);
        product(std::true_type{}, lp0, lp1, s0, s1, std::true_type{}, true, acc);
        lds_barrier();  // every wave is done with X(j)
        rows_to_slab_pair<C>(acc, ep, wm, wn, frow, khalf, s0, s1);
        lds_barrier();
        if constexpr (APPLY) read_slab_quads<C>(s0, s1, outq);
        else read_slab_pair<C>(s0, s1, out);
        if constexpr (NEXT_GRAM) product(std::false_type{}, s0, s1, s0, s1, std::false_type{}, false, accg);
        lds_barrier();  // the tile's values are read: the stage takes the next block
        if constexpr (APPLY) apply_w(j, outq, wv, loadw, wj);
        if constexpr (decltype(copy)::value) copy_x(next, s0, s1);
    };
    using T_ = std::true_type;
    using F_ = std::false_type;
    using Run = std::integral_constant<int, -1>;
    // The first tile (stage a) copies block j0 + 3 into its stage, or the
    // strip's last block again when there is none (never read), so that the
    // same copies are in flight whatever the strip's length.  Then whole
    // rounds of the stages b, c, a while the blocks three tiles on exist, and
    // the R <= 5 tiles left, each count fixed (tail<R>).
    using Two = std::integral_constant<int, 2>;
    // W of the next tile likewise (the strip's last again when there is none).
    tile(Run{}, T_{}, T_{}, j0, min(j0 + 3, j1 - 1), la0, la1, T_{}, min(j0 + 1, j1 - 1));
    int j = j0 + 1;
    for (; j + 5 < j1; j += 3) {
        tile(Two{}, F_{}, T_{}, j, j + 3, lb0, lb1, T_{}, j + 1);
        tile(Two{}, F_{}, T_{}, j + 1, j + 4, lc0, lc1, T_{}, j + 2);
        tile(Two{}, F_{}, T_{}, j + 2, j + 5, la0, la1, T_{}, j + 3);
    }
    auto tail = [&](auto r) __attribute__((always_inline)) {
        constexpr int R = decltype(r)::value;
        // tile t of the tail is block j + t in stage b, c, a, b, c; it copies
        // block j + t + 3 when that exists, and waits for its own block with
        // min(2, R - 1 - t) later blocks in flight
        using A0 = std::integral_constant<int, (R - 1 < 2 ? R - 1 : 2)>;
        using A1 = std::integral_constant<int, (R - 2 < 2 ? R - 2 : 2)>;
        using A2 = std::integral_constant<int, (R - 3 < 2 ? R - 3 : 2)>;
        using A3 = std::integral_constant<int, (R - 4 < 2 ? R - 4 : 2)>;
        if constexpr (R > 0)
            tile(A0{}, F_{}, std::bool_constant<(R > 3)>{}, j, j + 3, lb0, lb1, std::bool_constant<(R > 1)>{}, j + 1);
        if constexpr (R > 1)
            tile(A1{}, F_{}, std::bool_constant<(R > 4)>{}, j + 1, j + 4, lc0, lc1, std::bool_constant<(R > 2)>{},
                 j + 2);
        if constexpr (R > 2) tile(A2{}, F_{}, F_{}, j + 2, 0, la0, la1, std::bool_constant<(R > 3)>{}, j + 3);
        if constexpr (R > 3) tile(A3{}, F_{}, F_{}, j + 3, 0, lb0, lb1, std::bool_constant<(R > 4)>{}, j + 4);
        if constexpr (R > 4) tile(std::integral_constant<int, 0>{}, F_{}, F_{}, j + 4, 0, lc0, lc1, F_{}, 0);
    };
    switch (j1 - j) {
        case 1: tail(std::integral_constant<int, 1>{}); break;
        case 2: tail(std::integral_constant<int, 2>{}); break;
        case 3: tail(std::integral_constant<int, 3>{}); break;
        case 4: tail(std::integral_constant<int, 4>{}); break;
        case 5: tail(std::integral_constant<int, 5>{}); break;
        default: break;  // none left
    }
    // every copy has landed (a strip's first tile always copies, for a strip
    // of one tile its own block again) before the band buffer reuses the
    // first stage and before the workgroup ends (APPLY: every tile has
    // stored its W already)
    wait_vmcnt<0>();
    if constexpr (!APPLY) store_slab_rows<C>(out, (int64_t)(j1 - 1) * C::BN, ep);
    if constexpr (NEXT_GRAM) {
        // this strip's part of the next Gram: raw fp32, as the K-split Gram
        // stores it, through the first stage's first slab (every copy has
        // landed; the band loop's first barrier follows the last reads)
        Epi eg;
        eg.outF = d.gram_part + (int64_t)part * C::BM * C::BN;
        eg.out = nullptr;
        eg.ld_out = 0;
        eg.outT = nullptr;
        eg.ld_outT = 0;
        eg.E = nullptr;
        eg.ld_e = 0;
        eg.coef_e = 0.f;
        eg.coef_acc = 1.f;
        eg.post = 1.f;
        eg.diag = 0.f;
        epilogue_bands<C, false, true, true>(accg, 0, 0, eg, reinterpret_cast<float*>(la0), wm, wn, frow,
                                             khalf);
    }
}

// ---- fp32 operands: the full-precision option on the matrix cores ---------
//
// The fp32 class's three products (X and X^T kept side by side, 64-padded;
// the arithmetic of the FMA kernels in gemm_f32.hip, but the symmetric
// outputs computed on the lower triangle of tiles and mirrored) on the slab
// machinery above: a slab row of 128 bytes holds 32
// fp32 values where it holds 64 bf16, so the copies, the swizzle and the
// fragment reads serve unchanged, with K and the leading dimensions counted
// in 2-byte units.  A 16-byte fragment then holds 4 fp32 k values, and feeds
// four v_mfma_f32_32x32x2f32: in MFMA t, the lanes of k-half h contribute k =
// 8 kk + 4 h + t, so the four sum k-step kk's 8 values.
//
// 64 x 64 tiles (the fp32 padding), four waves of one 32 x 32 block each,
// two 16 KB stages (several workgroups per compute unit); 1 B copied per 16
// flop.

template <class C>
__device__ __forceinline__ void mfma_frags_f32(f32x16 (&acc)[C::FM][C::FN], const Frags<C>& f) {
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j) {
            const f32x4 a = __builtin_bit_cast(f32x4, f.a[i]);
            const f32x4 b = __builtin_bit_cast(f32x4, f.b[j]);
#pragma unroll
            for (int t = 0; t < 4; ++t)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc[i][j], 0, 0, 0);
        }
}

// C tile = sum_k P[i][k] Q[j][k] over fp32 rows (K fp32 values, a multiple of
// 32), the pipeline of gemm_tile with the fp32 products.  Its barriers are
// LDS-only: each wave has waited for its own copies of the stage it reads
// next.
template <class C>
__device__ __forceinline__ void gemm_mainloop_f32(const float* __restrict__ P, int64_t ldp,
                                                  const float* __restrict__ Q, int64_t ldq, int K,
                                                  const Stages& st, f32x16 (&acc)[C::FM][C::FN]) {
    const uint16_t* P0 = reinterpret_cast<const uint16_t*>(P);
    const uint16_t* Q0 = reinterpret_cast<const uint16_t*>(Q);
    ldp *= 2;
    ldq *= 2;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int frow = lane & 31;
    const int khalf = lane >> 5;
#pragma unroll
    for (int i = 0; i < C::FM; ++i)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
    const int KT = (2 * K) / C::BK;
    constexpr int KS = C::BK / 16;
#pragma unroll
    for (int u = 0; u < C::NS; ++u)
        if (u < KT) load_stage<C, false>(P0, ldp, Q0, ldq, (int64_t)u * C::BK, st, u, wave, lane);
    if (KT >= C::NS) wait_vmcnt<(C::NS - 1) * C::LPS>(); else wait_vmcnt<0>();
    lds_barrier();
    Frags<C> f[2];
    read_frags<C, false>(st, 0, 0, wm, wn, frow, khalf, lane, f[0]);
    for (int kt0 = 0; kt0 < KT; kt0 += C::NS) {
#pragma unroll
        for (int u = 0; u < C::NS; ++u) {
            const int kt = kt0 + u;
            if (kt < KT) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    if (kk + 1 < KS) {
                        read_frags<C, false>(st, u, kk + 1, wm, wn, frow, khalf, lane, f[(kk + 1) & 1]);
                    } else {
                        if (kt + C::NS - 1 < KT) wait_vmcnt<(C::NS - 2) * C::LPS>(); else wait_vmcnt<0>();
                        lds_barrier();
                        if (kt + C::NS < KT)
                            load_stage<C, false>(P0, ldp, Q0, ldq, (int64_t)(kt + C::NS) * C::BK, st, u, wave,
                                                 lane);
                        read_frags<C, false>(st, (u + 1) % C::NS, 0, wm, wn, frow, khalf, lane, f[0]);
                    }
                    mfma_frags_f32<C>(acc, f[kk & 1]);
                }
            }
        }
    }
    wait_vmcnt<0>();
}

// Epilogue of an fp32 tile through the band buffer (array 0): v = post *
// (coef_acc * product + coef_e * E), stored to `out` and, if set, transposed
// to `outT`; every access 2 x 16 bytes.
struct EpiF32 {
    float* out;
    int64_t ld_out;
    float* outT;
    int64_t ld_outT;
    const float* E;
    int64_t ld_e;
    float coef_e, coef_acc, post;
};

template <class C>
__device__ __forceinline__ void epilogue_f32(const f32x16 (&acc)[C::FM][C::FN], int64_t row0, int64_t col0,
                                             const EpiF32& ep, float* sb) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int wm = wave / C::WN, wn = wave % C::WN;
    const int frow = lane & 31;
    const int khalf = lane >> 5;
#pragma unroll
    for (int band = 0; band < C::BM / C::RB; ++band) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < C::FM; ++i) {
            if (wm * C::TM + i * 32 == band * C::RB) {
#pragma unroll
                for (int j = 0; j < C::FN; ++j) {
                    const int c = wn * C::TN + j * 32 + frow;
#pragma unroll
                    for (int r = 0; r < 16; ++r) sb[sbi<C>(8 * (r >> 2) + 4 * khalf + (r & 3), c)] = acc[i][j][r];
                }
            }
        }
        __syncthreads();
        const int64_t brow = row0 + (int64_t)band * C::RB;
#pragma unroll
        for (int q = 0; q < (C::RB * C::BN / 8) / C::NT; ++q) {
            const int ch = q * C::NT + threadIdx.x;
            const int rr = ch / (C::BN / 8), c8 = (ch % (C::BN / 8)) * 8;
            const float4 a0 = *reinterpret_cast<const float4*>(sb + sbi<C>(rr, c8));
            const float4 a1 = *reinterpret_cast<const float4*>(sb + sbi<C>(rr, c8) + 4);
            float v[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
            if (ep.E) {
                const float* e = ep.E + (brow + rr) * ep.ld_e + col0 + c8;
                const float4 e0 = gld(reinterpret_cast<const float4*>(e));
                const float4 e1 = gld(reinterpret_cast<const float4*>(e + 4));
                const float ev[8] = {e0.x, e0.y, e0.z, e0.w, e1.x, e1.y, e1.z, e1.w};
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = ep.post * (ep.coef_acc * v[t] + ep.coef_e * ev[t]);
            } else {
#pragma unroll
                for (int t = 0; t < 8; ++t) v[t] = ep.post * (ep.coef_acc * v[t]);
            }
            float* o = ep.out + (brow + rr) * ep.ld_out + col0 + c8;
            gst(reinterpret_cast<float4*>(o), make_float4(v[0], v[1], v[2], v[3]));
            gst(reinterpret_cast<float4*>(o + 4), make_float4(v[4], v[5], v[6], v[7]));
            if (ep.outT) {
                *reinterpret_cast<float4*>(sb + sbi<C>(rr, c8)) = make_float4(v[0], v[1], v[2], v[3]);
                *reinterpret_cast<float4*>(sb + sbi<C>(rr, c8) + 4) = make_float4(v[4], v[5], v[6], v[7]);
            }
        }
        if (ep.outT) {
            __syncthreads();
#pragma unroll
            for (int q = 0; q < (C::BN * C::RB / 8) / C::NT; ++q) {
                const int ch = q * C::NT + threadIdx.x;
                const int c = ch / (C::RB / 8), i8 = (ch % (C::RB / 8)) * 8;
                float v[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) v[e] = sb[sbi<C>(i8 + e, c)];
                float* o = ep.outT + (col0 + c) * ep.ld_outT + brow + i8;
                gst(reinterpret_cast<float4*>(o), make_float4(v[0], v[1], v[2], v[3]));
                gst(reinterpret_cast<float4*>(o + 4), make_float4(v[4], v[5], v[6], v[7]));
            }
        }
    }
}

using F32Cfg = Cfg<64, 64, 2, 2, 64, 2>;

// Operands and epilogue of one fp32 tile in phase PHASE (mirror: an
// off-diagonal tile of a symmetric product, also stored transposed).
template <int PHASE>
__device__ __forceinline__ void f32_operands(const MatDesc& d, int it, float ca, float cb, float cc, bool mirror,
                                             const float*& P, const float*& Q, int64_t& ld, int& K,
                                             EpiF32& ep) {
    const int64_t mp = d.mp, np = d.np;
    ep.outT = nullptr;
    ep.ld_outT = 0;
    ep.E = nullptr;
    ep.ld_e = 0;
    ep.coef_e = 0.f;
    ep.coef_acc = 1.f;
    ep.post = 1.f;
    if (PHASE == GRAM) {
        P = Q = reinterpret_cast<const float*>(d.x[it & 1]);
        ld = np;
        K = (int)np;
        const float s = (it == 0) ? gld(d.inv_norm) : 1.f;
        ep.coef_acc = s * s;
        ep.out = reinterpret_cast<float*>(d.a);
        ep.ld_out = mp;
        ep.outT = mirror ? ep.out : nullptr;
        ep.ld_outT = mp;
    } else if (PHASE == POLY) {
        P = Q = reinterpret_cast<const float*>(d.a);
        ld = mp;
        K = (int)mp;
        ep.E = P;
        ep.ld_e = mp;
        ep.coef_e = cb;
        ep.coef_acc = cc;
        ep.out = reinterpret_cast<float*>(d.b);
        ep.ld_out = mp;
        ep.outT = mirror ? ep.out : nullptr;
        ep.ld_outT = mp;
    } else {
        P = reinterpret_cast<const float*>(d.b);
        Q = reinterpret_cast<const float*>(d.xt[it & 1]);
        ld = mp;
        K = (int)mp;
        ep.E = reinterpret_cast<const float*>(d.x[it & 1]);
        ep.ld_e = np;
        ep.coef_e = ca;
        ep.post = (it == 0) ? gld(d.inv_norm) : 1.f;
        ep.out = reinterpret_cast<float*>(d.x[(it + 1) & 1]);
        ep.ld_out = np;
        ep.outT = reinterpret_cast<float*>(d.xt[(it + 1) & 1]);
        ep.ld_outT = mp;
    }
}


// One fp32 tile per workgroup, over the class's prefix of (full-square or
// update) tiles.
template <int PHASE>
__global__ __launch_bounds__(F32Cfg::NT) void ns_f32_mfma_kernel(const MatDesc* __restrict__ descs, int n,
                                                                 const int32_t* __restrict__ prefix, int it,
                                                                 float ca, float cb, float cc) {
    using C = F32Cfg;
    static_assert(C::BM == kTileF32 && C::BN == kTileF32, "fp32 tiles");
    static_assert(C::NS == 2, "two stages");
    __shared__ __attribute__((aligned(1024))) uint16_t l0[C::STAGE];
    __shared__ __attribute__((aligned(1024))) uint16_t l1[C::STAGE];
    const Stages st{{l0, l1, l1, l1}};
    const int tile = blockIdx.x;
    const int mi = find_matrix(prefix, n, tile);
    const MatDesc& d = descs[mi];
    const int lt = tile - prefix[mi];
    const int64_t mp = d.mp, np = d.np;
    int ti, tj;
    if (PHASE == UPDATE) {
        const int tcols = (int)(np / C::BN);
        ti = lt / tcols;
        tj = lt - ti * tcols;
    } else {
        // the symmetric products: the class's prefix counts every tile of
        // the square; the first T (T + 1) / 2 of a matrix take the lower
        // triangle (each off-diagonal tile also stored mirrored), the rest
        // have nothing to do
        const int T = (int)(mp / C::BM);
        if (lt >= T * (T + 1) / 2) return;
        tri_index(lt, ti, tj);
    }
    const float *P, *Q;
    int64_t ld;
    int K;
    EpiF32 ep;
    f32_operands<PHASE>(d, it, ca, cb, cc, ti != tj, P, Q, ld, K, ep);
    const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
    f32x16 acc[C::FM][C::FN];
    gemm_mainloop_f32<C>(P + r0 * ld, ld, Q + c0 * ld, ld, K, st, acc);
    epilogue_f32<C>(acc, r0, c0, ep, reinterpret_cast<float*>(lds_arr(st, 0)));
}

// fp32 launches of short K (up to KMAX, e.g. one 256 x 256 matrix): a tile of
// 64 leaves most compute units idle and runs its whole K on one.  Here each
// 64-tile of the class's prefix is four workgroups of 32 x 32, and the four
// waves of a workgroup split K: every wave multiplies its quarter of the
// slabs into its own 32 x 32 accumulator, then the four partial tiles are
// summed through LDS in wave order.  The tile's whole K is copied at once.
struct F32SkCopy {  // slab geometry for load_slab / read_frag: 128-byte rows
    static constexpr int BK = 64, CH = 8, RPI = 8, NW = 4;
};

template <int PHASE, int KMAX>
__global__ __launch_bounds__(256) void ns_f32_splitk_kernel(const MatDesc* __restrict__ descs, int n,
                                                            const int32_t* __restrict__ prefix, int it,
                                                            float ca, float cb, float cc) {
    using CP = F32SkCopy;
    constexpr int TB = 32, NSL = KMAX / 32;  // tile edge, fp32 slabs of 32
    static_assert(KMAX % 64 == 0, "whole slab pairs");
    __shared__ __attribute__((aligned(1024))) uint16_t lp[NSL * TB * CP::BK];
    __shared__ __attribute__((aligned(1024))) uint16_t lq[NSL * TB * CP::BK];
    __shared__ __attribute__((aligned(16))) float red[4 * TB * TB];
    const int t64 = blockIdx.x >> 2, q = blockIdx.x & 3;
    const int mi = find_matrix(prefix, n, t64);
    const MatDesc& d = descs[mi];
    const int lt = t64 - prefix[mi];
    int ti, tj;
    if (PHASE == UPDATE) {
        const int tcols = (int)(d.np / kTileF32);
        ti = lt / tcols;
        tj = lt - ti * tcols;
    } else {
        // lower triangle of 64-tiles (the rest of the square's prefix idle),
        // and of a diagonal 64-tile the quarters on and below its diagonal
        const int T = (int)(d.mp / kTileF32);
        if (lt >= T * (T + 1) / 2) return;
        tri_index(lt, ti, tj);
        if (ti == tj && (q >> 1) < (q & 1)) return;
    }
    ti = 2 * ti + (q >> 1);
    tj = 2 * tj + (q & 1);
    const float *P, *Q;
    int64_t ld;
    int K;
    EpiF32 ep;
    f32_operands<PHASE>(d, it, ca, cb, cc, ti != tj, P, Q, ld, K, ep);
    const int64_t r0 = (int64_t)ti * TB, c0 = (int64_t)tj * TB;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int frow = lane & 31, khalf = lane >> 5;
    const int ns = K / 32;  // slabs of this tile (at most NSL)
    {
        const uint16_t* P0 = reinterpret_cast<const uint16_t*>(P + r0 * ld);
        const uint16_t* Q0 = reinterpret_cast<const uint16_t*>(Q + c0 * ld);
        for (int sl = 0; sl < ns; ++sl) {
            load_slab<CP, TB>(P0 + 64 * sl, 2 * ld, lp + sl * TB * CP::BK, wave, lane);
            load_slab<CP, TB>(Q0 + 64 * sl, 2 * ld, lq + sl * TB * CP::BK, wave, lane);
        }
    }
    wait_vmcnt<0>();
    __syncthreads();
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    const int s0 = wave * ns / 4, s1 = (wave + 1) * ns / 4;
    for (int sl = s0; sl < s1; ++sl) {
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
            const f32x4 a = __builtin_bit_cast(f32x4, read_frag<CP>(lp + sl * TB * CP::BK, frow, 2 * kk + khalf));
            const f32x4 b = __builtin_bit_cast(f32x4, read_frag<CP>(lq + sl * TB * CP::BK, frow, 2 * kk + khalf));
#pragma unroll
            for (int t = 0; t < 4; ++t) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[t], b[t], acc, 0, 0, 0);
        }
    }
    // partial tiles to LDS (row 8 (r >> 2) + 4 khalf + (r & 3), column frow), summed in wave order
#pragma unroll
    for (int r = 0; r < 16; ++r) red[wave * TB * TB + (8 * (r >> 2) + 4 * khalf + (r & 3)) * TB + frow] = acc[r];
    __syncthreads();
    const int row = threadIdx.x >> 3, col = (threadIdx.x & 7) * 4;
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int o = row * TB + col + e;
        v[e] = ((red[o] + red[TB * TB + o]) + red[2 * TB * TB + o]) + red[3 * TB * TB + o];
    }
    if (ep.E) {
        const float4 e4 = gld(reinterpret_cast<const float4*>(ep.E + (r0 + row) * ep.ld_e + c0 + col));
        const float ev[4] = {e4.x, e4.y, e4.z, e4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ep.post * (ep.coef_acc * v[e] + ep.coef_e * ev[e]);
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = ep.post * (ep.coef_acc * v[e]);
    }
    gst(reinterpret_cast<float4*>(ep.out + (r0 + row) * ep.ld_out + c0 + col), make_float4(v[0], v[1], v[2], v[3]));
    if (ep.outT) {
        // the transpose through the first partial tile's LDS (read by now:
        // a barrier after every thread's sums)
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) red[(col + e) * (TB + 1) + row] = v[e];
        __syncthreads();
        float w[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = red[row * (TB + 1) + col + e];
        gst(reinterpret_cast<float4*>(ep.outT + (c0 + row) * ep.ld_outT + r0 + col),
            make_float4(w[0], w[1], w[2], w[3]));
    }
}

// single-matrix variants for the test hooks
template <class C, int PHASE>
__global__ __launch_bounds__(C::NT) void ns_sym_single(const uint16_t* __restrict__ src, int64_t ld,
                                                       int K, uint16_t* out, int64_t ld_out,
                                                       float sq, float ca, float cb, float cc,
                                                       XcdSplit xs) {
    constexpr int NA = lds_arrays<C>();
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[kLdsArr];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[NA > 1 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds2[NA > 2 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds3[NA > 3 ? kLdsArr : 8];
    const Stages st{{lds0, lds1, lds2, lds3}};
    int tile, q;
    if (!xcd_task(xs, tile, q)) return;
    int ti, tj;
    tri_index(tile, ti, tj);
    if (q >= 0 && ti == tj && (q >> 1) < (q & 1)) return;
    const bool on_diag = ti == tj && (q < 0 || (q >> 1) == (q & 1));
    Epi ep;
    ep.outF = nullptr;
    ep.out = out;
    ep.ld_out = ld_out;
    ep.outT = on_diag ? nullptr : out;
    ep.ld_outT = ld_out;
    if (PHASE == GRAM) {
        ep.E = nullptr; ep.ld_e = 0; ep.coef_e = 0.f; ep.coef_acc = sq; ep.post = 1.f;
        ep.diag = 0.f;
    } else {
        ep.E = src; ep.ld_e = ld; ep.coef_e = cb; ep.coef_acc = cc; ep.post = 1.f;
        ep.diag = on_diag ? ca : 0.f;
    }
    if (q < 0) {
        const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
        if (on_diag)
            gemm_tile<C, PHASE == POLY, false, false, true>(src + r0 * ld, ld, src + c0 * ld, ld, K, r0, c0,
                                                             ep, st);
        else
            gemm_tile<C, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, K, r0, c0, ep, st);
    } else {
        using Q = QuarterCfg<C>;
        const int64_t r0 = (int64_t)ti * C::BM + (q >> 1) * Q::BM;
        const int64_t c0 = (int64_t)tj * C::BN + (q & 1) * Q::BN;
        if (on_diag)
            gemm_tile<Q, PHASE == POLY, false, false, true>(src + r0 * ld, ld, src + c0 * ld, ld, K, r0, c0,
                                                             ep, st);
        else
            gemm_tile<Q, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, K, r0, c0, ep, st);
    }
}

template <class C>
__global__ __launch_bounds__(C::NT) void ns_update_single(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ B,
                                                          uint16_t* Xo, int m, int n, int64_t ldx,
                                                          int64_t ldb, float s, XcdSplit xs) {
    constexpr int NA = lds_arrays<C>();
    __shared__ __attribute__((aligned(1024))) uint16_t lds0[kLdsArr];
    __shared__ __attribute__((aligned(1024))) uint16_t lds1[NA > 1 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds2[NA > 2 ? kLdsArr : 8];
    __shared__ __attribute__((aligned(1024))) uint16_t lds3[NA > 3 ? kLdsArr : 8];
    const Stages st{{lds0, lds1, lds2, lds3}};
    int tile, q;
    if (!xcd_task(xs, tile, q)) return;
    int ti, tj;
    grouped_index(tile, m / C::BM, n / C::BN, ti, tj);
    Epi ep;
    ep.outF = nullptr;
    ep.out = Xo; ep.ld_out = ldx; ep.outT = nullptr; ep.ld_outT = 0;
    ep.E = nullptr; ep.ld_e = 0; ep.coef_e = 0.f; ep.coef_acc = 1.f; ep.post = s; ep.diag = 0.f;
    if (q < 0) {
        const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
        gemm_tile<C, false, true>(B + r0 * ldb, ldb, X + c0, ldx, m, r0, c0, ep, st);
    } else {
        using Q = QuarterCfg<C>;
        const int64_t r0 = (int64_t)ti * C::BM + (q >> 1) * Q::BM;
        const int64_t c0 = (int64_t)tj * C::BN + (q & 1) * Q::BN;
        gemm_tile<Q, false, true>(B + r0 * ldb, ldb, X + c0, ldx, m, r0, c0, ep, st);
    }
}

inline int xcd_grid(const XcdSplit& xs) { return 8 * (xs.per > 0 ? xs.per : 1); }

using SymCfg = Cfg<256, 256, 2, 4>;
using UpdCfg = Cfg<256, 256, 2, 4>;
// matrices whose short side fits 128 (per-head blocks, small layers)
using SmallCfg = Cfg<128, 128, 2, 2>;

}  // namespace

static_assert(SymCfg::BM == kClassTile[kLarge] && UpdCfg::BM == kClassTile[kLarge] &&
                  UpdCfg::BN == kClassTile[kLarge],
              "256-class tiles");
static_assert(SmallCfg::BM == kClassTile[kSmall] && SmallCfg::BN == kClassTile[kSmall],
              "128-class tiles");

hipError_t launch_gram_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                            int small, int split, hipStream_t st) {
    if (split) {
        if (small)
            ns_gram_split_kernel<SmallCfg><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, p.gram, xs, it);
        else
            ns_gram_split_kernel<SymCfg><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(d, n, p.gram, xs, it);
        return hipGetLastError();
    }
    if (small)
        ns_sym_kernel<SmallCfg, GRAM><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, p.gram, xs, it, 0.f, 0.f, 0.f);
    else
        ns_sym_kernel<SymCfg, GRAM><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(d, n, p.gram, xs, it, 0.f, 0.f, 0.f);
    return hipGetLastError();
}

hipError_t launch_gram_reduce_bf16(const MatDesc* d, int n, Prefix p, int tiles, int it, int small,
                                   hipStream_t st) {
    if (small)
        ns_gram_reduce_kernel<SmallCfg::BM><<<tiles * (SmallCfg::BM / 64) * (SmallCfg::BM / 64), 256, 0, st>>>(
            d, n, p.tri, it);
    else
        ns_gram_reduce_kernel<SymCfg::BM><<<tiles * (SymCfg::BM / 64) * (SymCfg::BM / 64), 256, 0, st>>>(
            d, n, p.tri, it);
    return hipGetLastError();
}

hipError_t launch_poly_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, float a,
                            float b, float c, int small, hipStream_t st) {
    if (small)
        ns_sym_kernel<SmallCfg, POLY><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, p.tri, xs, 0, a, b, c);
    else
        ns_sym_kernel<SymCfg, POLY><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(d, n, p.tri, xs, 0, a, b, c);
    return hipGetLastError();
}

hipError_t launch_update_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                              int small, hipStream_t st) {
    if (small)
        ns_update_kernel<SmallCfg><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, p.upd, xs, it);
    else
        ns_update_kernel<UpdCfg><<<xcd_grid(xs), UpdCfg::NT, 0, st>>>(d, n, p.upd, xs, it);
    return hipGetLastError();
}

hipError_t launch_update_strip_bf16(const MatDesc* d, int n, const int32_t* prefix_strip,
                                   const XcdSplit& xs, int it, int strip, int next_gram, int stream,
                                   int apply, float a, float b, float c, float decay, float lr,
                                   hipStream_t st) {
    if (stream) {
        if (next_gram)
            ns_update_stream_kernel<SmallCfg, true, false><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(
                d, n, prefix_strip, xs, it, strip, a, b, c, decay, lr);
        else if (apply)
            ns_update_stream_kernel<SmallCfg, false, true><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(
                d, n, prefix_strip, xs, it, strip, a, b, c, decay, lr);
        else
            ns_update_stream_kernel<SmallCfg, false, false><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(
                d, n, prefix_strip, xs, it, strip, a, b, c, decay, lr);
        return hipGetLastError();
    }
    if (apply) return hipErrorInvalidValue;  // only streamed strips apply
    if (next_gram)
        ns_update_strip_kernel<SmallCfg, true><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, prefix_strip, xs,
                                                                                      it, strip, a, b, c);
    else
        ns_update_strip_kernel<SmallCfg, false><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(
            d, n, prefix_strip, xs, it, strip, a, b, c);
    return hipGetLastError();
}

hipError_t launch_gram_bf16_single(const void* X, void* A, int m, int n, int64_t ldx, int64_t lda,
                                   float s2, int cus, hipStream_t st) {
    const int T = m / SymCfg::BM;
    const int32_t total = T * (T + 1) / 2;
    const int64_t w = 1;
    const XcdSplit xs = xcd_split(&total, &w, 1, cus, 1);
    ns_sym_single<SymCfg, GRAM><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(
        reinterpret_cast<const uint16_t*>(X), ldx, n, reinterpret_cast<uint16_t*>(A), lda, s2, 0.f,
        0.f, 0.f, xs);
    return hipGetLastError();
}

hipError_t launch_poly_bf16_single(const void* A, void* B, int m, int64_t lda, float a, float b,
                                   float c, int cus, hipStream_t st) {
    const int T = m / SymCfg::BM;
    const int32_t total = T * (T + 1) / 2;
    const int64_t w = 1;
    const XcdSplit xs = xcd_split(&total, &w, 1, cus, 1);
    ns_sym_single<SymCfg, POLY><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(
        reinterpret_cast<const uint16_t*>(A), lda, m, reinterpret_cast<uint16_t*>(B), lda, 1.f, a,
        b, c, xs);
    return hipGetLastError();
}

hipError_t launch_update_bf16_single(const void* X, const void* B, void* Xo, int m, int n,
                                     int64_t ldx, int64_t ldb, float s, int cus, hipStream_t st) {
    const int tiles = (m / UpdCfg::BM) * (n / UpdCfg::BN);
    const int32_t total = tiles;
    const int64_t w = 1;
    const XcdSplit xs = xcd_split(&total, &w, 1, cus, 1);
    ns_update_single<UpdCfg><<<xcd_grid(xs), UpdCfg::NT, 0, st>>>(
        reinterpret_cast<const uint16_t*>(X), reinterpret_cast<const uint16_t*>(B),
        reinterpret_cast<uint16_t*>(Xo), m, n, ldx, ldb, s, xs);
    return hipGetLastError();
}

hipError_t launch_f32_mfma(int phase, const MatDesc* d, int n, const int32_t* prefix, int total, int it,
                           int kmax, float a, float b, float c, hipStream_t st) {
    if (kmax <= 256) {
        if (phase == GRAM)
            ns_f32_splitk_kernel<GRAM, 256><<<4 * total, 256, 0, st>>>(d, n, prefix, it, a, b, c);
        else if (phase == POLY)
            ns_f32_splitk_kernel<POLY, 256><<<4 * total, 256, 0, st>>>(d, n, prefix, it, a, b, c);
        else
            ns_f32_splitk_kernel<UPDATE, 256><<<4 * total, 256, 0, st>>>(d, n, prefix, it, a, b, c);
        return hipGetLastError();
    }
    if (phase == GRAM)
        ns_f32_mfma_kernel<GRAM><<<total, F32Cfg::NT, 0, st>>>(d, n, prefix, it, a, b, c);
    else if (phase == POLY)
        ns_f32_mfma_kernel<POLY><<<total, F32Cfg::NT, 0, st>>>(d, n, prefix, it, a, b, c);
    else
        ns_f32_mfma_kernel<UPDATE><<<total, F32Cfg::NT, 0, st>>>(d, n, prefix, it, a, b, c);
    return hipGetLastError();
}

}  // namespace muon
