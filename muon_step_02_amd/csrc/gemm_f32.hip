// fp32 Newton-Schulz phases (the full-precision option of the Muon step).
//
// Same three products and the same buffer layout as the bf16 kernels (X and
// X^T kept side by side, padded to multiples of 64, zero padding).  A launch
// whose K exceeds 64 runs on the matrix cores (launch_f32_mfma, with the bf16
// kernels' slab machinery).  A launch of tiny matrices only (K at most 64,
// e.g. thousands of at most 32 x 32 blocks) runs here, with fp32 FMAs on
// 64 x 64 tiles: 256 threads, 4 x 4 outputs each, the tile's whole K extent
// staged in LDS at once, every tile of the symmetric outputs computed.
//
//   gram:   A = s^2 X X^T        (s = 1/(||Y||+eps) on the first iteration)
//   poly:   B = b A + c A A
//   update: X <- s (a X + B X), X^T alongside
//
// ("About Muon: Why Not Adam", kiungsong.github.io, sections "Making It
// Actually Run" and "The whole thing, in about forty lines".)
#include "muon_internal.h"

namespace muon {

namespace {

enum { GRAM = 0, POLY = 1, UPDATE = 2 };
constexpr int T = kTileF32;  // 64
constexpr int KS = 16;

// Tile of phase PHASE: operands, their leading dimensions and the K extent.
template <int PHASE>
struct F32Tile {
    const MatDesc* d;
    const float* P;
    const float* Q;
    int64_t ldp, ldq;
    int K;
    int ti, tj;
};

template <int PHASE>
__device__ __forceinline__ F32Tile<PHASE> f32_tile(const MatDesc* __restrict__ descs, int n,
                                                   const int32_t* __restrict__ prefix, int it) {
    F32Tile<PHASE> t;
    const int tile = blockIdx.x;
    const int mi = find_matrix(prefix, n, tile);
    t.d = &descs[mi];
    const MatDesc& d = *t.d;
    const int lt = tile - prefix[mi];
    const int tcols = (int)((PHASE == UPDATE ? d.np : d.mp) / T);
    t.ti = lt / tcols;
    t.tj = lt - t.ti * tcols;
    if (PHASE == GRAM) {
        t.P = t.Q = reinterpret_cast<const float*>(d.x[it & 1]);
        t.ldp = t.ldq = d.np;
        t.K = (int)d.np;
    } else if (PHASE == POLY) {
        t.P = t.Q = reinterpret_cast<const float*>(d.a);
        t.ldp = t.ldq = d.mp;
        t.K = (int)d.mp;
    } else {
        t.P = reinterpret_cast<const float*>(d.b);
        t.Q = reinterpret_cast<const float*>(d.xt[it & 1]);
        t.ldp = t.ldq = d.mp;
        t.K = (int)d.mp;
    }
    return t;
}

// Epilogue of a 64 x 64 tile: thread (ty, tx) holds rows 4 ty .. 4 ty + 3,
// columns 4 tx .. 4 tx + 3 of the product.
template <int PHASE>
__device__ __forceinline__ void f32_epilogue(const F32Tile<PHASE>& t, const float (&acc)[4][4], int it,
                                             float ca, float cb, float cc) {
    const MatDesc& d = *t.d;
    const int ty = threadIdx.x >> 4, tx = threadIdx.x & 15;
    const int64_t mp = d.mp, np = d.np;
    const int64_t i0 = (int64_t)t.ti * T + ty * 4;
    const int64_t j0 = (int64_t)t.tj * T + tx * 4;
    if (PHASE == GRAM) {
        const float s = (it == 0) ? gld(d.inv_norm) : 1.f;
        const float s2 = s * s;
        float* A = reinterpret_cast<float*>(d.a);
#pragma unroll
        for (int r = 0; r < 4; ++r)
            gst(reinterpret_cast<float4*>(A + (i0 + r) * mp + j0),
                make_float4(s2 * acc[r][0], s2 * acc[r][1], s2 * acc[r][2], s2 * acc[r][3]));
    } else if (PHASE == POLY) {
        const float* A = reinterpret_cast<const float*>(d.a);
        float* B = reinterpret_cast<float*>(d.b);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 e = gld(reinterpret_cast<const float4*>(A + (i0 + r) * mp + j0));
            gst(reinterpret_cast<float4*>(B + (i0 + r) * mp + j0),
                make_float4(cb * e.x + cc * acc[r][0], cb * e.y + cc * acc[r][1],
                            cb * e.z + cc * acc[r][2], cb * e.w + cc * acc[r][3]));
        }
    } else {
        const float post = (it == 0) ? gld(d.inv_norm) : 1.f;
        const float* X = reinterpret_cast<const float*>(d.x[it & 1]);
        float* Xo = reinterpret_cast<float*>(d.x[(it + 1) & 1]);
        float* XoT = reinterpret_cast<float*>(d.xt[(it + 1) & 1]);
        float v[4][4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float4 e = gld(reinterpret_cast<const float4*>(X + (i0 + r) * np + j0));
            v[r][0] = post * (ca * e.x + acc[r][0]);
            v[r][1] = post * (ca * e.y + acc[r][1]);
            v[r][2] = post * (ca * e.z + acc[r][2]);
            v[r][3] = post * (ca * e.w + acc[r][3]);
            gst(reinterpret_cast<float4*>(Xo + (i0 + r) * np + j0),
                make_float4(v[r][0], v[r][1], v[r][2], v[r][3]));
        }
#pragma unroll
        for (int c = 0; c < 4; ++c)
            gst(reinterpret_cast<float4*>(XoT + (j0 + c) * mp + i0),
                make_float4(v[0][c], v[1][c], v[2][c], v[3][c]));
    }
}

// K of at most KMAX: every thread issues the loads of the tile's whole K
// extent at once, they go to LDS transposed, and after one barrier the
// product runs from LDS (on a tiny matrix the load latency, not the
// arithmetic, sets the launch time).
template <int PHASE, int KMAX>
__global__ __launch_bounds__(256) void ns_f32_shortk_kernel(const MatDesc* __restrict__ descs, int n,
                                                            const int32_t* __restrict__ prefix, int it,
                                                            float ca, float cb, float cc) {
    static_assert(KMAX % KS == 0, "whole slabs");
    __shared__ float Ps[KMAX][T + 4];
    __shared__ float Qs[KMAX][T + 4];
    const F32Tile<PHASE> tl = f32_tile<PHASE>(descs, n, prefix, it);
    const int t = threadIdx.x;
    const int ty = t >> 4, tx = t & 15;
    const int lrow = t >> 2, lk = (t & 3) * 4;
    const float* Pr = tl.P + (int64_t)(tl.ti * T + lrow) * tl.ldp + lk;
    const float* Qr = tl.Q + (int64_t)(tl.tj * T + lrow) * tl.ldq + lk;
    constexpr int NSL = KMAX / KS;
    float4 pv[NSL], qv[NSL];
#pragma unroll
    for (int s = 0; s < NSL; ++s) {
        if (s * KS < tl.K) {
            pv[s] = gld(reinterpret_cast<const float4*>(Pr + s * KS));
            qv[s] = gld(reinterpret_cast<const float4*>(Qr + s * KS));
        }
    }
#pragma unroll
    for (int s = 0; s < NSL; ++s) {
        if (s * KS < tl.K) {
            const int k = s * KS + lk;
            Ps[k + 0][lrow] = pv[s].x; Ps[k + 1][lrow] = pv[s].y; Ps[k + 2][lrow] = pv[s].z; Ps[k + 3][lrow] = pv[s].w;
            Qs[k + 0][lrow] = qv[s].x; Qs[k + 1][lrow] = qv[s].y; Qs[k + 2][lrow] = qv[s].z; Qs[k + 3][lrow] = qv[s].w;
        }
    }
    __syncthreads();
    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;
    for (int k0 = 0; k0 < tl.K; k0 += KS) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = Ps[k0 + kk][ty * 4 + r];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = Qs[k0 + kk][tx * 4 + c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
        }
    }
    f32_epilogue<PHASE>(tl, acc, it, ca, cb, cc);
}

}  // namespace

// The kernel for a launch whose largest K is kmax (the planner's largest n'
// or m' of the class): the FMA kernel staging the whole K up to 64 (a launch
// of tiny matrices only), else the matrix-core kernels.  Measured: the
// 256 x 256 matrix's launches 16.2-17.0 us with the FMA kernels, 5.1-5.4 us
// on the matrix cores (K split four ways); 2500 matrices of at most 32 x 32,
// the step 0.73-0.77 ms with the FMA kernel, 0.78-0.80 ms on the matrix
// cores.
template <int PHASE>
hipError_t launch_f32(const MatDesc* d, int n, const int32_t* prefix, int total, int it, int kmax,
                      float a, float b, float c, hipStream_t st) {
    if (kmax <= 64) {
        ns_f32_shortk_kernel<PHASE, 64><<<total, 256, 0, st>>>(d, n, prefix, it, a, b, c);
        return hipGetLastError();
    }
    return launch_f32_mfma(PHASE, d, n, prefix, total, it, kmax, a, b, c, st);
}

hipError_t launch_gram_f32(const MatDesc* d, int n, Prefix p, int total, int it, int kmax, hipStream_t st) {
    return launch_f32<GRAM>(d, n, p.gram, total, it, kmax, 0.f, 0.f, 0.f, st);
}

hipError_t launch_poly_f32(const MatDesc* d, int n, Prefix p, int total, int kmax, float b, float c,
                           hipStream_t st) {
    return launch_f32<POLY>(d, n, p.tri, total, 0, kmax, 0.f, b, c, st);
}

hipError_t launch_update_f32(const MatDesc* d, int n, Prefix p, int total, int it, int kmax, float a,
                             hipStream_t st) {
    return launch_f32<UPDATE>(d, n, p.upd, total, it, kmax, a, 0.f, 0.f, st);
}

}  // namespace muon
