// bf16 MFMA kernels of the quintic Newton-Schulz iteration (gfx950).
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

namespace muon {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
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
// BM x BK slab of P, then Q's (BN x BK, or BK x BN k-major).
template <class C, bool QKN>
__device__ __forceinline__ void load_stage(const uint16_t* __restrict__ P0, int64_t ldp,
                                           const uint16_t* __restrict__ Q0, int64_t ldq,
                                           int64_t k0, const Stages& st, int i, int wave, int lane) {
    load_slab<C, C::BM>(P0 + k0, ldp, stage_p<C>(st, i), wave, lane);
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

template <class C, bool QKN>
__device__ __forceinline__ void read_frags(const Stages& st, int i, int kk, int wm, int wn,
                                           int frow, int khalf, int lane, Frags<C>& f) {
    const uint16_t* sp = stage_p<C>(st, i);
    const uint16_t* sq = stage_q<C>(st, i);
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

// C tile = sum_k P[i][k] Q'[k][j] for the BM rows starting at P0 (leading
// dimension ldp) and BN columns of Q' (K a multiple of BK), then the
// epilogue.  Q' is read as Q'[k][j] = Q0[j * ldq + k] (NT) or, with QKN, as
// Q0[k * ldq + j] (k-major).
template <class C, bool HAS_E, bool QKN = false>
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
            load_stage<C, QKN>(P0, ldp, Q0, ldq, (int64_t)u * C::BK, st, u, wave, lane);
        }
    }
    if (KT >= C::NS) wait_vmcnt<(C::NS - 1) * C::LPS>(); else wait_vmcnt<0>();
    __syncthreads();
    Frags<C> f[2];
    read_frags<C, QKN>(st, 0, 0, wm, wn, frow, khalf, lane, f[0]);

    for (int kt0 = 0; kt0 < KT; kt0 += C::NS) {
#pragma unroll
        for (int u = 0; u < C::NS; ++u) {
            const int kt = kt0 + u;
            if (kt < KT) {
#pragma unroll
                for (int kk = 0; kk < KS; ++kk) {
                    if (kk + 1 < KS) {
                        read_frags<C, QKN>(st, u, kk + 1, wm, wn, frow, khalf, lane,
                                           f[(kk + 1) & 1]);
                    } else {
                        // slab kt + 1 has landed once only the copies of the
                        // slabs after it are outstanding; then every wave's.
                        // The last slab takes the same path (its reads of
                        // the next stage are unused) so every slab has one
                        // straight-line sequence of LDS waits.
                        if (kt + C::NS - 1 < KT) wait_vmcnt<(C::NS - 2) * C::LPS>(); else wait_vmcnt<0>();
                        __syncthreads();
                        if (kt + C::NS < KT) {
                            load_stage<C, QKN>(P0, ldp, Q0, ldq, (int64_t)(kt + C::NS) * C::BK,
                                               st, u, wave, lane);
                        }
                        read_frags<C, QKN>(st, (u + 1) % C::NS, 0, wm, wn, frow, khalf, lane, f[0]);
                    }
                    mfma_frags<C>(acc, f[kk & 1]);
                    // two reads with each of the first MFMAs: the reads go out early
                    // (k-major fragments are two reads each)
                    interleave_reads_mfma<C::FM + (QKN ? 2 : 1) * C::FN, C::FM * C::FN, 2>();
                }
            }
        }
    }

    // Epilogue through LDS, in bands of RB rows: the waves holding the band
    // write their fp32 accumulators (MFMA 32x32 layout: lane l, register r is
    // row (r & 3) + 4*(l >> 5) + 8*(r >> 2), column l & 31); then every thread
    // combines 8 consecutive columns with E and stores 16 bytes of the output,
    // and, for the transposed copy, 8 consecutive rows of one column.
    //
    // The band loop is unrolled so the compiler can count outstanding memory
    // operations exactly: no wait ever covers the stores of earlier bands, and
    // E is loaded one band ahead so its latency hides behind the LDS work.
    float* sb = reinterpret_cast<float*>(lds_arr(st, 0));
    constexpr int QN = (C::RB * C::BN / 8) / C::NT;  // 16-byte chunks per thread per band
    uint4 ecur[QN], enxt[QN];
    wait_vmcnt<0>();  // every slab copy has landed: the band buffer is free
    if (HAS_E) load_e_band<C, QN>(ep, row0, col0, 0, ecur);
#pragma unroll
    for (int band = 0; band < C::BM / C::RB; ++band) {
        if (HAS_E && band + 1 < C::BM / C::RB) load_e_band<C, QN>(ep, row0, col0, band + 1, enxt);
        __syncthreads();
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
        __syncthreads();
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
        if (ep.outT) {
            __syncthreads();
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

// Task of this workgroup under an XcdSplit: a whole tile (quarter = -1) or
// quarter q of a tile (rows (q >> 1), columns (q & 1) of its 2 x 2 split).
// False: no task, exit.
__device__ __forceinline__ bool xcd_task(const XcdSplit& xs, int& tile, int& quarter) {
    const int b = (int)blockIdx.x;
    const int x = b & 7;
    const int t = b >> 3;
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
    tri_index(tile - prefix[mi], ti, tj);
    // a quarter above the diagonal of a diagonal tile is the mirror of the
    // quarter below it
    if (q >= 0 && ti == tj && (q >> 1) < (q & 1)) return;
    // the tile (or quarter) holds part of the diagonal: stored once, no mirror
    const bool on_diag = ti == tj && (q < 0 || (q >> 1) == (q & 1));
    const int64_t mp = d.mp, np = d.np;
    Epi ep;
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
    if (q < 0) {
        const int64_t r0 = (int64_t)ti * C::BM, c0 = (int64_t)tj * C::BN;
        gemm_tile<C, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, (int)ld, r0, c0, ep, st);
    } else if constexpr (C::BM == 256) {
        using Q = QuarterCfg<C>;
        const int64_t r0 = (int64_t)ti * C::BM + (q >> 1) * Q::BM;
        const int64_t c0 = (int64_t)tj * C::BN + (q & 1) * Q::BN;
        gemm_tile<Q, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, (int)ld, r0, c0, ep, st);
    }
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
        gemm_tile<C, PHASE == POLY>(src + r0 * ld, ld, src + c0 * ld, ld, K, r0, c0, ep, st);
    } else {
        using Q = QuarterCfg<C>;
        const int64_t r0 = (int64_t)ti * C::BM + (q >> 1) * Q::BM;
        const int64_t c0 = (int64_t)tj * C::BN + (q & 1) * Q::BN;
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

int gemm_tile_bf16(int small) { return small ? SmallCfg::BM : SymCfg::BM; }
int upd_tile_m_bf16(int small) { return small ? SmallCfg::BM : UpdCfg::BM; }
int upd_tile_n_bf16(int small) { return small ? SmallCfg::BN : UpdCfg::BN; }

XcdSplit xcd_split(const int32_t* ntiles, const int64_t* weight, int n, int cus, int quarters) {
    XcdSplit xs;
    int64_t total_w = 0, total_t = 0;
    for (int k = 0; k < n; ++k) {
        total_w += (int64_t)ntiles[k] * weight[k];
        total_t += ntiles[k];
    }
    // boundary x: first tile whose preceding work reaches x/8 of the total
    xs.b[0] = 0;
    int x = 1;
    int64_t cum_w = 0, cum_t = 0;
    for (int k = 0; k < n && x < 8; ++k) {
        const int64_t w = weight[k] > 0 ? weight[k] : 1;
        const int64_t end_w = cum_w + (int64_t)ntiles[k] * w;
        while (x < 8 && end_w * 8 >= (int64_t)x * total_w) {
            // smallest t in [0, ntiles] with (cum_w + t*w) * 8 >= x * total_w
            const int64_t need = (int64_t)x * total_w - cum_w * 8;
            int64_t t = need <= 0 ? 0 : (need + 8 * w - 1) / (8 * w);
            if (t > ntiles[k]) t = ntiles[k];
            xs.b[x++] = (int32_t)(cum_t + t);
        }
        cum_w = end_w;
        cum_t += ntiles[k];
    }
    while (x < 9) xs.b[x++] = (int32_t)total_t;
    xs.b[8] = (int32_t)total_t;
    xs.per = 0;
    for (int i = 0; i < 8; ++i) {
        if (xs.b[i + 1] < xs.b[i]) xs.b[i + 1] = xs.b[i];
        const int T = xs.b[i + 1] - xs.b[i];
        // last round of R tiles on `cus` CUs: as 4R quarter tiles when R <= cus/2
        const int R = cus > 0 ? T % cus : 0;
        xs.sub[i] = (quarters && R > 0 && 2 * R <= cus) ? R : 0;
        const int tasks = T + 3 * xs.sub[i];
        if (tasks > xs.per) xs.per = tasks;
    }
    return xs;
}

hipError_t launch_gram_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                            int small, hipStream_t st) {
    if (small)
        ns_sym_kernel<SmallCfg, GRAM><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, p.gram, xs, it, 0.f, 0.f, 0.f);
    else
        ns_sym_kernel<SymCfg, GRAM><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(d, n, p.gram, xs, it, 0.f, 0.f, 0.f);
    return hipGetLastError();
}

hipError_t launch_poly_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, float a,
                            float b, float c, int small, hipStream_t st) {
    if (small)
        ns_sym_kernel<SmallCfg, POLY><<<xcd_grid(xs), SmallCfg::NT, 0, st>>>(d, n, p.gram, xs, 0, a, b, c);
    else
        ns_sym_kernel<SymCfg, POLY><<<xcd_grid(xs), SymCfg::NT, 0, st>>>(d, n, p.gram, xs, 0, a, b, c);
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

}  // namespace muon
