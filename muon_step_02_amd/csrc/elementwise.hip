// Memory-bound kernels of the Muon step and the AdamW fallback (gfx950).
//
//   momentum_kernel  M <- mu M + (1-mu) G; Y <- Nesterov blend; per-tile
//                    sum of Y^2; Y written (unnormalised) into the padded
//                    Newton-Schulz buffer in the canonical orientation (Y or,
//                    for rows > cols, Y^T through LDS; the fp32 iteration
//                    keeps both), with zeros in the padding.
//   norm_finalize    ||Y||_F from the per-tile partial sums (fixed order, so
//                    every run gives the same bits) and s = 1/(||Y||_F + eps).
//   table_upload     the host-built descriptor table, carried in kernel
//                    arguments.
//   apply_kernel     W <- (1 - lr wd) W - lr scale O, then the optional
//                    QK-Clip row scaling ("The Optimizer Wars ...", section
//                    "What is MuonClip?").
//   adamw_kernel     fused AdamW over a group of tensors.
//
// "About Muon: Why Not Adam" (kiungsong.github.io), section "The whole thing,
// in about forty lines": the momentum buffer is interpolated towards the
// gradient by 1 - mu, the Nesterov input interpolates the gradient towards
// the updated buffer by mu, the iteration starts from Y / (||Y||_F + eps),
// and the weight is decayed by (1 - lr wd) before the scaled update is
// subtracted.  AdamW: "Por qué AdamW para entrenar modelos de lenguaje, y qué
// está cambiando" (gustavoai.dev), sections "Adam: las dos ideas juntas" and
// "La W: un error de regularización que duró tres años".
//
// Each workgroup of the Muon kernels owns one tile of one weight (see
// EwTile for the shapes); the AdamW kernels take chunks of kAdamwChunk
// elements of one tensor.
#include <string.h>

#include "muon_internal.h"

namespace muon {

namespace {

struct Vals4 {
    float v[4];
};

typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// Streaming accesses: every element of the optimizer's tensors is touched
// once per kernel, so loads and stores bypass cache retention.
__device__ __forceinline__ float4 ld_nt(const float* p) {
    const f32x4v t = __builtin_nontemporal_load((const MUON_GLOBAL f32x4v*)p);
    return make_float4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void st_nt(float* p, float4 v) {
    const f32x4v t = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(t, (MUON_GLOBAL f32x4v*)p);
}
__device__ __forceinline__ uint2 ld_nt(const uint16_t* p) {
    const u32x2v t = __builtin_nontemporal_load((const MUON_GLOBAL u32x2v*)p);
    return make_uint2(t.x, t.y);
}
__device__ __forceinline__ void st_nt(uint16_t* p, uint2 v) {
    const u32x2v t = {v.x, v.y};
    __builtin_nontemporal_store(t, (MUON_GLOBAL u32x2v*)p);
}

template <bool VEC>
__device__ __forceinline__ Vals4 load4(const void* base, int dtype_bf16, int64_t off, int valid) {
    Vals4 r;
    if (VEC) {
        if (dtype_bf16) {
            uint2 u = ld_nt(reinterpret_cast<const uint16_t*>(base) + off);
            r.v[0] = __builtin_bit_cast(float, u.x << 16);
            r.v[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
            r.v[2] = __builtin_bit_cast(float, u.y << 16);
            r.v[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
        } else {
            float4 f = ld_nt(reinterpret_cast<const float*>(base) + off);
            r.v[0] = f.x; r.v[1] = f.y; r.v[2] = f.z; r.v[3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < valid) {
                r.v[e] = dtype_bf16
                    ? bf16_bits_to_f32(gld(reinterpret_cast<const uint16_t*>(base) + off + e))
                    : gld(reinterpret_cast<const float*>(base) + off + e);
            } else {
                r.v[e] = 0.f;
            }
        }
    }
    return r;
}

template <bool VEC>
__device__ __forceinline__ void store4(void* base, int dtype_bf16, int64_t off, const Vals4& r,
                                       int valid) {
    if (VEC) {
        if (dtype_bf16) {
            uint2 u;
            u.x = (uint32_t)f32_to_bf16_bits(r.v[0]) | ((uint32_t)f32_to_bf16_bits(r.v[1]) << 16);
            u.y = (uint32_t)f32_to_bf16_bits(r.v[2]) | ((uint32_t)f32_to_bf16_bits(r.v[3]) << 16);
            st_nt(reinterpret_cast<uint16_t*>(base) + off, u);
        } else {
            st_nt(reinterpret_cast<float*>(base) + off, make_float4(r.v[0], r.v[1], r.v[2], r.v[3]));
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if (e < valid) {
                if (dtype_bf16)
                    gst(reinterpret_cast<uint16_t*>(base) + off + e, f32_to_bf16_bits(r.v[e]));
                else
                    gst(reinterpret_cast<float*>(base) + off + e, r.v[e]);
            }
        }
    }
}

// Store four values into a Newton-Schulz buffer (bf16 or f32), 4-aligned.
template <bool NS_F32>
__device__ __forceinline__ void store_ns4(void* base, int64_t off, const float* v) {
    if (NS_F32) {
        gst(reinterpret_cast<float4*>(reinterpret_cast<float*>(base) + off),
            make_float4(v[0], v[1], v[2], v[3]));
    } else {
        uint2 u;
        u.x = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
        u.y = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
        gst(reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(base) + off), u);
    }
}

template <bool NS_F32>
__device__ __forceinline__ void load_ns4(const void* base, int64_t off, float* v) {
    if (NS_F32) {
        float4 f = ld_nt(reinterpret_cast<const float*>(base) + off);
        v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
    } else {
        uint2 u = ld_nt(reinterpret_cast<const uint16_t*>(base) + off);
        v[0] = __builtin_bit_cast(float, u.x << 16);
        v[1] = __builtin_bit_cast(float, u.x & 0xffff0000u);
        v[2] = __builtin_bit_cast(float, u.y << 16);
        v[3] = __builtin_bit_cast(float, u.y & 0xffff0000u);
    }
}

__device__ __forceinline__ float block_sum_256(float v, float* red) {
    v = wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float t = 0.f;
    if (threadIdx.x == 0) t = (red[0] + red[1]) + (red[2] + red[3]);
    return t;
}

// Elementwise tiles: TH x TW elements of the weight, 256 threads, each four
// consecutive columns of NP rows (rr + RPP q).  Three shapes:
//  - 16 x 256 streaming tiles where the bf16 iteration input is Y itself:
//    every wave instruction is one contiguous 1 KB (fp32) row segment;
//  - kTrTH x kTrTW tiles where the bf16 iteration runs on Y^T (rows > cols):
//    the tile goes through LDS; momentum stores Y transposed, apply reads X
//    transposed.  The tile is wide so the fp32 row segments are 512 B long;
//    that matters more than the length of the transposed bf16 rows (TH);
//  - 64 x 64 tiles for the fp32 iteration, which keeps both Y and Y^T.
template <int TH_, int TW_>
struct EwTile {
    static constexpr int TH = TH_, TW = TW_;
    static constexpr int TPR = TW / 4;     // threads per row
    static constexpr int RPP = 256 / TPR;  // rows per pass
    static constexpr int NP = TH / RPP;    // passes
    // the transposed tile (TW x TH), four consecutive entries per thread
    static constexpr int TPRT = TH / 4;
    static constexpr int RPPT = 256 / TPRT;
    static constexpr int NPT = TW / RPPT;
    static_assert(TPR * RPP == 256 && RPP * NP == TH, "passes cover the tile");
    static_assert(TPRT * RPPT == 256 && RPPT * NPT == TW, "transposed passes cover the tile");
};

// LDS tile for the transposing shapes: TW rows of TH + 1 floats (the +1 keeps
// both the column writes and the row reads on distinct banks).
constexpr int lds_tile(int th, int tw) { return tw * (th + 1); }

template <bool VEC, bool NS_F32, int TH, int TW, bool GBF>
__device__ __forceinline__ void momentum_tile(const MatDesc& d, int lt, float mu, int nesterov,
                                              float* tileT, float* red) {
    using T = EwTile<TH, TW>;
    constexpr bool TRN = TH != 16;  // the tile goes through LDS
    const int tr = lt / d.ew_tiles_c, tc = lt - tr * d.ew_tiles_c;
    const int64_t r0 = (int64_t)tr * TH, c0 = (int64_t)tc * TW;
    const int t = threadIdx.x;
    const int cg = (t % T::TPR) * 4;
    const int rr = t / T::TPR;
    const int64_t rows = d.rows, cols = d.cols;
    // natural orientation (rows_pad x cols_pad, ld cols_pad) and transposed
    // orientation (cols_pad x rows_pad, ld rows_pad) of Y.  The fp32
    // iteration keeps both X and X^T; the bf16 one only the canonical X
    // (short side first), which is Y itself or Y^T.
    void* nat = d.transposed ? d.xt[0] : d.x[0];
    void* trn = d.transposed ? d.x[0] : d.xt[0];
    const bool write_nat = NS_F32 || !d.transposed;
    const bool write_trn = TRN && (NS_F32 || d.transposed);
    const int64_t ld_nat = d.cols_pad, ld_trn = d.rows_pad;
    const float omm = 1.f - mu;
    float ss = 0.f;
    // all loads of the thread's rows first, so they are in flight together
    Vals4 g[T::NP], m[T::NP];
    int valid[T::NP];
#pragma unroll
    for (int q = 0; q < T::NP; ++q) {
        const int64_t r = r0 + rr + T::RPP * q;
        const int64_t cv = cols - (c0 + cg);
        valid[q] = (r < rows && cv > 0) ? (cv >= 4 ? 4 : (int)cv) : 0;
        if (valid[q] > 0) {
            g[q] = load4<VEC>(d.grad, GBF, r * d.ld_grad + c0 + cg, valid[q]);
            m[q] = load4<VEC>(d.mom, 0, r * d.ld_mom + c0 + cg, valid[q]);
        }
    }
#pragma unroll
    for (int q = 0; q < T::NP; ++q) {
        const int lr = rr + T::RPP * q;
        const int64_t r = r0 + lr;
        const int64_t c = c0 + cg;
        float y[4] = {0.f, 0.f, 0.f, 0.f};
        if (valid[q] > 0) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const float mn = mu * m[q].v[e] + omm * g[q].v[e];
                m[q].v[e] = mn;
                const float yy = nesterov ? (omm * g[q].v[e] + mu * mn) : mn;
                y[e] = (e < valid[q]) ? yy : 0.f;
                ss += y[e] * y[e];
            }
            store4<VEC>(d.mom, 0, r * d.ld_mom + c, m[q], valid[q]);
        }
        if (write_nat) store_ns4<NS_F32>(nat, r * ld_nat + c, y);
        if (TRN) {
#pragma unroll
            for (int e = 0; e < 4; ++e) tileT[(cg + e) * (TH + 1) + lr] = y[e];
        }
    }
    if (write_trn) {
        __syncthreads();
        const int cgt = (t % T::TPRT) * 4;  // weight row within the tile
        const int rrt = t / T::TPRT;
#pragma unroll
        for (int q = 0; q < T::NPT; ++q) {
            const int lc = rrt + T::RPPT * q;  // weight column = row of Y^T
            float v[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = tileT[lc * (TH + 1) + cgt + e];
            store_ns4<NS_F32>(trn, (c0 + lc) * ld_trn + r0 + cgt, v);
        }
    }
    const float tot = block_sum_256(ss, red);
    if (threadIdx.x == 0) gst(d.partials + lt, tot);
}

// The dtype and alignment of a matrix are uniform over the workgroup: branch
// once here, so the tile's loads are straight-line code that can all be in
// flight together.
template <bool NS_F32, int TH, int TW>
__device__ __forceinline__ void momentum_dispatch(const MatDesc& d, int lt, float mu, int nesterov,
                                                  float* tileT, float* red) {
    const bool gbf = d.grad_dtype == MUON_BF16;
    if (d.vec4) {
        if (gbf) momentum_tile<true, NS_F32, TH, TW, true>(d, lt, mu, nesterov, tileT, red);
        else momentum_tile<true, NS_F32, TH, TW, false>(d, lt, mu, nesterov, tileT, red);
    } else {
        if (gbf) momentum_tile<false, NS_F32, TH, TW, true>(d, lt, mu, nesterov, tileT, red);
        else momentum_tile<false, NS_F32, TH, TW, false>(d, lt, mu, nesterov, tileT, red);
    }
}

// LDS: tiles of the fp32 iteration (64 x 64) or the transposing bf16 shape.
template <bool NS_F32, bool LDS>
constexpr int ew_lds_floats() {
    return !LDS ? 1 : NS_F32 ? lds_tile(kEwTile, kEwTile) : lds_tile(kTrTH, kTrTW);
}

template <bool NS_F32, bool LDS>
__global__ __launch_bounds__(256) void momentum_kernel(const MatDesc* __restrict__ descs, int n,
                                                       const int32_t* __restrict__ prefix,
                                                       float mu, int nesterov) {
    __shared__ float tileT[ew_lds_floats<NS_F32, LDS>()];
    __shared__ float red[4];
    const int tile = blockIdx.x;
    const int mi = find_matrix(prefix, n, tile);
    const MatDesc& d = descs[mi];
    const int lt = tile - prefix[mi];
    if (NS_F32)
        momentum_dispatch<true, kEwTile, kEwTile>(d, lt, mu, nesterov, tileT, red);
    else if (!LDS)
        momentum_dispatch<false, 16, 256>(d, lt, mu, nesterov, tileT, red);
    else
        momentum_dispatch<false, kTrTH, kTrTW>(d, lt, mu, nesterov, tileT, red);
}

__global__ __launch_bounds__(256) void norm_finalize_kernel(const MatDesc* __restrict__ descs,
                                                            float eps) {
    const MatDesc& d = descs[blockIdx.x];
    __shared__ double red[4];
    double s = 0.0;
    for (int i = threadIdx.x; i < d.ew_tiles; i += 256) s += (double)gld(d.partials + i);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double tot = (red[0] + red[1]) + (red[2] + red[3]);
        const double nu = sqrt(tot);
        gst(d.inv_norm, (float)(1.0 / (nu + (double)eps)));
        if (d.norm_out) gst(d.norm_out, (float)nu);
    }
}

template <bool VEC, bool NS_F32, int TH, int TW, bool PBF>
__device__ __forceinline__ void apply_tile(const MatDesc& d, int lt, int parity, float decay,
                                           float step, float qk_tau, float* tileT) {
    using T = EwTile<TH, TW>;
    const int tr = lt / d.ew_tiles_c, tc = lt - tr * d.ew_tiles_c;
    const int64_t r0 = (int64_t)tr * TH, c0 = (int64_t)tc * TW;
    const int t = threadIdx.x;
    const int cg = (t % T::TPR) * 4;
    const int rr = t / T::TPR;
    const int64_t rows = d.rows, cols = d.cols;
    // O in the weight's orientation (rows_pad x cols_pad, ld cols_pad): X
    // when not transposed, else X^T, which the fp32 iteration keeps and the
    // bf16 one gets by transposing X (cols_pad x rows_pad) through LDS.
    const bool via_lds = TH != 16 && !NS_F32 && d.transposed;
    const void* O = d.transposed ? (NS_F32 ? d.xt[parity] : d.x[parity]) : d.x[parity];
    const int64_t ld_o = d.cols_pad;
    const float sc = step * d.scale;
    float o[T::NP][4];
    Vals4 w[T::NP];
    int valid[T::NP];
    if (via_lds) {
        // X rows c0.. (weight columns), columns r0.. (weight rows); all inside
        // the zero-padded buffer
        const int cgt = (t % T::TPRT) * 4;
        const int rrt = t / T::TPRT;
#pragma unroll
        for (int q = 0; q < T::NPT; ++q) {
            const int lc = rrt + T::RPPT * q;
            float v[4];
            load_ns4<NS_F32>(O, (c0 + lc) * d.rows_pad + r0 + cgt, v);
#pragma unroll
            for (int e = 0; e < 4; ++e) tileT[lc * (TH + 1) + cgt + e] = v[e];
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < T::NP; ++q) {
        const int64_t r = r0 + rr + T::RPP * q;
        const int64_t cv = cols - (c0 + cg);
        valid[q] = (r < rows && cv > 0) ? (cv >= 4 ? 4 : (int)cv) : 0;
        if (valid[q] > 0) {
            if (via_lds) {
#pragma unroll
                for (int e = 0; e < 4; ++e) o[q][e] = tileT[(cg + e) * (TH + 1) + rr + T::RPP * q];
            } else {
                load_ns4<NS_F32>(O, r * ld_o + c0 + cg, o[q]);
            }
            w[q] = load4<VEC>(d.param, PBF, r * d.ld_param + c0 + cg, valid[q]);
        }
    }
#pragma unroll
    for (int q = 0; q < T::NP; ++q) {
        if (valid[q] == 0) continue;
        const int64_t r = r0 + rr + T::RPP * q;
        const int64_t c = c0 + cg;
        // QK-Clip: rows of head h scaled by sqrt(tau / S_max^h) when S_max^h > tau
        float clip = 1.f;
        if (d.qk_smax) {
            const float sm = gld(d.qk_smax + r / d.qk_block_rows);
            clip = sm > qk_tau ? sqrtf(qk_tau / sm) : 1.f;
        }
#pragma unroll
        // one explicit fma, so that the streamed update that applies the
        // step itself rounds the same way
        for (int e = 0; e < 4; ++e) w[q].v[e] = clip * __builtin_fmaf(decay, w[q].v[e], -(sc * o[q][e]));
        store4<VEC>(d.param, PBF, r * d.ld_param + c, w[q], valid[q]);
        if (d.update_out) {
            Vals4 ov;
#pragma unroll
            for (int e = 0; e < 4; ++e) ov.v[e] = o[q][e];
            store4<false>(d.update_out, 0, r * cols + c, ov, valid[q]);
        }
    }
}

template <bool NS_F32, int TH, int TW>
__device__ __forceinline__ void apply_dispatch(const MatDesc& d, int lt, int parity, float decay,
                                               float step, float qk_tau, float* tileT) {
    const bool pbf = d.param_dtype == MUON_BF16;
    if (d.vec4) {
        if (pbf) apply_tile<true, NS_F32, TH, TW, true>(d, lt, parity, decay, step, qk_tau, tileT);
        else apply_tile<true, NS_F32, TH, TW, false>(d, lt, parity, decay, step, qk_tau, tileT);
    } else {
        if (pbf) apply_tile<false, NS_F32, TH, TW, true>(d, lt, parity, decay, step, qk_tau, tileT);
        else apply_tile<false, NS_F32, TH, TW, false>(d, lt, parity, decay, step, qk_tau, tileT);
    }
}

template <bool NS_F32, bool LDS>
__global__ __launch_bounds__(256) void apply_kernel(const MatDesc* __restrict__ descs, int n,
                                                    const int32_t* __restrict__ prefix,
                                                    int parity, float decay, float step,
                                                    float qk_tau) {
    // the fp32 iteration keeps X^T: no transposing through LDS
    __shared__ float tileT[NS_F32 ? 1 : ew_lds_floats<false, LDS>()];
    const int tile = blockIdx.x;
    const int mi = find_matrix(prefix, n, tile);
    const MatDesc& d = descs[mi];
    const int lt = tile - prefix[mi];
    if (NS_F32)
        apply_dispatch<true, kEwTile, kEwTile>(d, lt, parity, decay, step, qk_tau, tileT);
    else if (!LDS)
        apply_dispatch<false, 16, 256>(d, lt, parity, decay, step, qk_tau, tileT);
    else
        apply_dispatch<false, kTrTH, kTrTW>(d, lt, parity, decay, step, qk_tau, tileT);
}

// ------------------------------------------------------ table upload ----

struct TableChunk {
    uint32_t w[kTableChunkWords];
};

__global__ __launch_bounds__(256) void table_upload_kernel(TableChunk c, uint32_t* dst, int nwords) {
    for (int i = threadIdx.x; i < nwords; i += 256) gst(dst + i, c.w[i]);
}

// ---------------------------------------------------------------- AdamW ----

__device__ __forceinline__ void adamw_elem(float& th, float g, float& m, float& v, float lr,
                                           float b1, float b2, float eps, float wd, float inv_bc1,
                                           float inv_bc2) {
    m = b1 * m + (1.f - b1) * g;
    v = b2 * v + (1.f - b2) * (g * g);
    const float mhat = m * inv_bc1;
    const float vhat = v * inv_bc2;
    th = th - lr * (mhat / (sqrtf(vhat) + eps) + wd * th);
}

__device__ __forceinline__ int adamw_tensor_of(const AdamwGroup& grp, int blk) {
    int lo = 0, hi = grp.count - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (grp.block_prefix[mid] <= blk) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// One whole chunk on the vector path.  Every load of the chunk is issued
// before the first store: the compiler cannot move a load above a store to a
// pointer it may alias, so a load/compute/store loop would keep only one
// quarter of the chunk in flight per thread.
template <bool PBF, bool GBF>
__device__ __forceinline__ void adamw_chunk_vec(void* P, const void* G, float* M, float* V,
                                                int64_t start, float gs, float lr, float b1,
                                                float b2, float eps, float wd, float inv_bc1,
                                                float inv_bc2) {
    constexpr int Q = kAdamwChunk / 1024;
    Vals4 th[Q], g[Q];
    float4 m[Q], v[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t off = start + q * 1024 + threadIdx.x * 4;
        th[q] = load4<true>(P, PBF, off, 4);
        g[q] = load4<true>(G, GBF, off, 4);
        m[q] = ld_nt(M + off);
        v[q] = ld_nt(V + off);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t off = start + q * 1024 + threadIdx.x * 4;
        adamw_elem(th[q].v[0], gs * g[q].v[0], m[q].x, v[q].x, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
        adamw_elem(th[q].v[1], gs * g[q].v[1], m[q].y, v[q].y, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
        adamw_elem(th[q].v[2], gs * g[q].v[2], m[q].z, v[q].z, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
        adamw_elem(th[q].v[3], gs * g[q].v[3], m[q].w, v[q].w, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
        store4<true>(P, PBF, off, th[q], 4);
        st_nt(M + off, m[q]);
        st_nt(V + off, v[q]);
    }
}

// gscale: null, or a device scalar every gradient is multiplied by first
// (global-norm clipping).
__global__ __launch_bounds__(256) void adamw_kernel(AdamwGroup grp, float lr, float b1, float b2,
                                                    float eps, float wd, float inv_bc1,
                                                    float inv_bc2, const float* gscale) {
    const int blk = blockIdx.x;
    const int ti = adamw_tensor_of(grp, blk);
    const float gs = gscale ? gld(gscale) : 1.f;
    const int64_t start = (int64_t)(blk - grp.block_prefix[ti]) * kAdamwChunk;
    const int64_t numel = grp.numel[ti];
    const int64_t end = start + kAdamwChunk < numel ? start + kAdamwChunk : numel;
    void* P = grp.param[ti];
    const void* G = grp.grad[ti];
    float* M = grp.m[ti];
    float* V = grp.v[ti];
    const int pbf = grp.param_bf16[ti], gbf = grp.grad_bf16[ti];
    if (grp.vec4[ti] && end - start == kAdamwChunk) {
        // the dtypes are uniform over the workgroup: branch once, outside the chunk
        if (pbf) {
            if (gbf)
                adamw_chunk_vec<true, true>(P, G, M, V, start, gs, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
            else
                adamw_chunk_vec<true, false>(P, G, M, V, start, gs, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
        } else {
            if (gbf)
                adamw_chunk_vec<false, true>(P, G, M, V, start, gs, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
            else
                adamw_chunk_vec<false, false>(P, G, M, V, start, gs, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
        }
    } else {
        for (int64_t i = start + threadIdx.x; i < end; i += 256) {
            float th = pbf ? bf16_bits_to_f32(gld(reinterpret_cast<const uint16_t*>(P) + i))
                           : gld(reinterpret_cast<const float*>(P) + i);
            const float g = gs * (gbf ? bf16_bits_to_f32(gld(reinterpret_cast<const uint16_t*>(G) + i))
                                      : gld(reinterpret_cast<const float*>(G) + i));
            float m = gld(M + i), v = gld(V + i);
            adamw_elem(th, g, m, v, lr, b1, b2, eps, wd, inv_bc1, inv_bc2);
            if (pbf)
                gst(reinterpret_cast<uint16_t*>(P) + i, f32_to_bf16_bits(th));
            else
                gst(reinterpret_cast<float*>(P) + i, th);
            gst(M + i, m);
            gst(V + i, v);
        }
    }
}

// Sum of squares of the gradients of one group, one partial per block of
// kAdamwChunk elements, written at partials[block_offset + block].  Every
// thread issues its four loads before the first product.  (Two or more
// chunks per workgroup, with all of their loads issued at once, measured
// slower: the many small workgroups keep more of the chip busy.)
__global__ __launch_bounds__(256) void adamw_sumsq_kernel(AdamwGroup grp, float* partials,
                                                          int block_offset) {
    __shared__ float red[4];
    const int blk = blockIdx.x;
    const int ti = adamw_tensor_of(grp, blk);
    const int64_t start = (int64_t)(blk - grp.block_prefix[ti]) * kAdamwChunk;
    const int64_t numel = grp.numel[ti];
    const int64_t end = start + kAdamwChunk < numel ? start + kAdamwChunk : numel;
    const void* G = grp.grad[ti];
    const int gbf = grp.grad_bf16[ti];
    float ss = 0.f;
    if (grp.vec4[ti] && end - start == kAdamwChunk) {
        constexpr int Q = kAdamwChunk / 1024;
        Vals4 g[Q];
        if (gbf) {
#pragma unroll
            for (int q = 0; q < Q; ++q) g[q] = load4<true>(G, 1, start + q * 1024 + threadIdx.x * 4, 4);
        } else {
#pragma unroll
            for (int q = 0; q < Q; ++q) g[q] = load4<true>(G, 0, start + q * 1024 + threadIdx.x * 4, 4);
        }
#pragma unroll
        for (int q = 0; q < Q; ++q)
#pragma unroll
            for (int e = 0; e < 4; ++e) ss += g[q].v[e] * g[q].v[e];
    } else {
        for (int64_t i = start + threadIdx.x; i < end; i += 256) {
            const float g = gbf ? bf16_bits_to_f32(gld(reinterpret_cast<const uint16_t*>(G) + i))
                                : gld(reinterpret_cast<const float*>(G) + i);
            ss += g * g;
        }
    }
    const float tot = block_sum_256(ss, red);
    if (threadIdx.x == 0) gst(partials + block_offset + blk, tot);
}

// norm = sqrt(sum of partials) in a fixed order; scale = max_norm / norm if
// norm > max_norm, else 1.
__global__ __launch_bounds__(256) void clip_finalize_kernel(const float* partials, int nblocks,
                                                            float max_norm, float* scale,
                                                            float* norm_out) {
    __shared__ double red[4];
    double s = 0.0;
    for (int i = threadIdx.x; i < nblocks; i += 256) s += (double)gld(partials + i);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off, 64);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) red[wave] = s;
    __syncthreads();
    if (threadIdx.x == 0) {
        const double norm = sqrt((red[0] + red[1]) + (red[2] + red[3]));
        gst(scale, norm > (double)max_norm ? (float)((double)max_norm / norm) : 1.f);
        if (norm_out) gst(norm_out, (float)norm);
    }
}

}  // namespace

hipError_t launch_adamw_sumsq(const AdamwGroup& g, int total_blocks, float* partials,
                              int block_offset, hipStream_t st) {
    adamw_sumsq_kernel<<<total_blocks, 256, 0, st>>>(g, partials, block_offset);
    return hipGetLastError();
}

hipError_t launch_clip_finalize(const float* partials, int nblocks, float max_norm, float* scale,
                                float* norm_out, hipStream_t st) {
    clip_finalize_kernel<<<1, 256, 0, st>>>(partials, nblocks, max_norm, scale, norm_out);
    return hipGetLastError();
}

hipError_t launch_momentum(const MatDesc* d, int n, const EwGroups& g, float mu, int nesterov,
                           hipStream_t st) {
    if (g.tiles[kEwStream] > 0)
        momentum_kernel<false, false><<<g.tiles[kEwStream], 256, 0, st>>>(d, n, g.prefix[kEwStream], mu, nesterov);
    if (g.tiles[kEwTrans] > 0)
        momentum_kernel<false, true><<<g.tiles[kEwTrans], 256, 0, st>>>(d, n, g.prefix[kEwTrans], mu, nesterov);
    if (g.tiles[kEwF32] > 0)
        momentum_kernel<true, true><<<g.tiles[kEwF32], 256, 0, st>>>(d, n, g.prefix[kEwF32], mu, nesterov);
    return hipGetLastError();
}

hipError_t launch_norm_finalize(const MatDesc* d, int n, float eps, hipStream_t st) {
    norm_finalize_kernel<<<n, 256, 0, st>>>(d, eps);
    return hipGetLastError();
}

hipError_t launch_apply(const MatDesc* d, int n, const EwGroups& g, int final_parity, float lr,
                        float wd, float qk_tau, hipStream_t st) {
    const float decay = 1.f - lr * wd;
    if (g.tiles[kEwStream] > 0)
        apply_kernel<false, false><<<g.tiles[kEwStream], 256, 0, st>>>(d, n, g.prefix[kEwStream],
                                                                      final_parity, decay, lr, qk_tau);
    if (g.tiles[kEwTrans] > 0)
        apply_kernel<false, true><<<g.tiles[kEwTrans], 256, 0, st>>>(d, n, g.prefix[kEwTrans],
                                                                    final_parity, decay, lr, qk_tau);
    if (g.tiles[kEwF32] > 0)
        apply_kernel<true, true><<<g.tiles[kEwF32], 256, 0, st>>>(d, n, g.prefix[kEwF32],
                                                                 final_parity, decay, lr, qk_tau);
    return hipGetLastError();
}

hipError_t launch_table_upload(const void* host, size_t bytes, void* dst, hipStream_t st) {
    const uint32_t* src = static_cast<const uint32_t*>(host);
    const size_t words = bytes / 4;
    for (size_t w0 = 0; w0 < words; w0 += kTableChunkWords) {
        const int nw = (int)(words - w0 < (size_t)kTableChunkWords ? words - w0 : kTableChunkWords);
        TableChunk c;
        memcpy(c.w, src + w0, (size_t)nw * 4);
        if (nw < kTableChunkWords) memset(c.w + nw, 0, (size_t)(kTableChunkWords - nw) * 4);
        table_upload_kernel<<<1, 256, 0, st>>>(c, static_cast<uint32_t*>(dst) + w0, nw);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

hipError_t launch_adamw(const AdamwGroup& g, int total_blocks, float lr, float beta1, float beta2,
                        float eps, float wd, float bc1, float bc2, const float* gscale,
                        hipStream_t st) {
    adamw_kernel<<<total_blocks, 256, 0, st>>>(g, lr, beta1, beta2, eps, wd, 1.f / bc1, 1.f / bc2,
                                               gscale);
    return hipGetLastError();
}

}  // namespace muon
