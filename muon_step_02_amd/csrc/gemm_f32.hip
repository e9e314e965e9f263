// fp32 Newton-Schulz phases (the full-precision option of the Muon step).
//
// Same three products and the same buffer layout as the bf16 kernels (X and
// X^T kept side by side, padded to multiples of 64, zero padding), computed
// with fp32 FMAs on 64 x 64 tiles: 256 threads, 4 x 4 outputs each, K in
// slabs of 16 staged through LDS.  This path serves small matrices where
// accuracy matters more than throughput, so every tile of the symmetric
// outputs is computed (no triangle skipping).
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

template <int PHASE>
__global__ __launch_bounds__(256) void ns_f32_kernel(const MatDesc* __restrict__ descs, int n,
                                                     const int32_t* __restrict__ prefix, int it,
                                                     float ca, float cb, float cc) {
    __shared__ float Ps[KS][T + 4];
    __shared__ float Qs[KS][T + 4];
    const int tile = blockIdx.x;
    const int mi = find_matrix(prefix, n, tile);
    const MatDesc& d = descs[mi];
    const int lt = tile - prefix[mi];
    const int64_t mp = d.mp, np = d.np;
    const int tcols = (int)((PHASE == UPDATE ? np : mp) / T);
    const int ti = lt / tcols, tj = lt - ti * tcols;

    const float* P;
    const float* Q;
    int64_t ldp, ldq;
    int K;
    if (PHASE == GRAM) {
        P = Q = reinterpret_cast<const float*>(d.x[it & 1]);
        ldp = ldq = np;
        K = (int)np;
    } else if (PHASE == POLY) {
        P = Q = reinterpret_cast<const float*>(d.a);
        ldp = ldq = mp;
        K = (int)mp;
    } else {
        P = reinterpret_cast<const float*>(d.b);
        Q = reinterpret_cast<const float*>(d.xt[it & 1]);
        ldp = ldq = mp;
        K = (int)mp;
    }
    const int t = threadIdx.x;
    const int ty = t >> 4, tx = t & 15;
    const int lrow = t >> 2, lk = (t & 3) * 4;
    const float* Pr = P + (int64_t)(ti * T + lrow) * ldp + lk;
    const float* Qr = Q + (int64_t)(tj * T + lrow) * ldq + lk;

    float acc[4][4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[r][c] = 0.f;

    for (int k0 = 0; k0 < K; k0 += KS) {
        const float4 pv = gld(reinterpret_cast<const float4*>(Pr + k0));
        const float4 qv = gld(reinterpret_cast<const float4*>(Qr + k0));
        __syncthreads();
        Ps[lk + 0][lrow] = pv.x; Ps[lk + 1][lrow] = pv.y; Ps[lk + 2][lrow] = pv.z; Ps[lk + 3][lrow] = pv.w;
        Qs[lk + 0][lrow] = qv.x; Qs[lk + 1][lrow] = qv.y; Qs[lk + 2][lrow] = qv.z; Qs[lk + 3][lrow] = qv.w;
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
            float a[4], b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] = Ps[kk][ty * 4 + r];
#pragma unroll
            for (int c = 0; c < 4; ++c) b[c] = Qs[kk][tx * 4 + c];
#pragma unroll
            for (int r = 0; r < 4; ++r)
#pragma unroll
                for (int c = 0; c < 4; ++c) acc[r][c] = fmaf(a[r], b[c], acc[r][c]);
        }
    }

    const int64_t i0 = (int64_t)ti * T + ty * 4;
    const int64_t j0 = (int64_t)tj * T + tx * 4;
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

}  // namespace

hipError_t launch_gram_f32(const MatDesc* d, int n, Prefix p, int total, int it, hipStream_t st) {
    ns_f32_kernel<GRAM><<<total, 256, 0, st>>>(d, n, p.gram, it, 0.f, 0.f, 0.f);
    return hipGetLastError();
}

hipError_t launch_poly_f32(const MatDesc* d, int n, Prefix p, int total, float b, float c,
                           hipStream_t st) {
    ns_f32_kernel<POLY><<<total, 256, 0, st>>>(d, n, p.tri, 0, 0.f, b, c);
    return hipGetLastError();
}

hipError_t launch_update_f32(const MatDesc* d, int n, Prefix p, int total, int it, float a,
                             hipStream_t st) {
    ns_f32_kernel<UPDATE><<<total, 256, 0, st>>>(d, n, p.upd, it, a, 0.f, 0.f);
    return hipGetLastError();
}

}  // namespace muon
