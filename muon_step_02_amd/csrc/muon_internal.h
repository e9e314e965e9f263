// Internal declarations shared by the HIP sources of libmuon (gfx950 only).
//
// Device-side view of one Muon matrix, the workspace layout and the launch
// wrappers of every kernel.  Nothing here is part of the public ABI
// (include/muon.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/muon.h"
#include "layout.h"

namespace muon {

// ---- global-memory accessors ----------------------------------------------
// Pointers that reach a kernel through a descriptor are generic, and a plain
// dereference compiles to a flat_* instruction.  Flat accesses count against
// the LDS wait counter as well as the vector-memory one, so every wait for an
// LDS read would also wait for all outstanding global stores.  Casting to the
// global address space makes the compiler emit global_* instructions.
#define MUON_GLOBAL __attribute__((address_space(1)))
template <int BYTES> struct GWord;
template <> struct GWord<2> { using T = uint16_t; };
template <> struct GWord<4> { using T = uint32_t; };
template <> struct GWord<8> { using T = uint32_t __attribute__((ext_vector_type(2))); };
template <> struct GWord<16> { using T = uint32_t __attribute__((ext_vector_type(4))); };
template <class T>
__device__ __forceinline__ T gld(const T* p) {
    using W = typename GWord<sizeof(T)>::T;
    return __builtin_bit_cast(T, *(const MUON_GLOBAL W*)p);
}
template <class T>
__device__ __forceinline__ void gst(T* p, const T& v) {
    using W = typename GWord<sizeof(T)>::T;
    *(MUON_GLOBAL W*)p = __builtin_bit_cast(W, v);
}

__device__ __forceinline__ int find_matrix(const int32_t* prefix, int n, int32_t tile) {
    // largest i with prefix[i] <= tile (prefix[0] = 0, prefix[n] = total)
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (gld(prefix + mid) <= tile) lo = mid; else hi = mid - 1;
    }
    // uniform across the workgroup: descriptor fields then come through
    // scalar loads into scalar registers
    return __builtin_amdgcn_readfirstlane(lo);
}

// ---- bf16 helpers (round to nearest even, as a hardware conversion) -------
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    __bf16 h = (__bf16)f;
    return __builtin_bit_cast(uint16_t, h);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// ---- launch wrappers ------------------------------------------------------
// All return hipGetLastError() after the launch.

// Copy `bytes` (a multiple of 4) of host data to device memory `dst` in
// kernel arguments, kTableChunkWords words (16 KB) per launch.  Measured on
// the MI355X: a 2 KB argument block takes 3.4 us a launch, 16 KB 7.5 us.
constexpr int kTableChunkWords = 4096;
hipError_t launch_table_upload(const void* host, size_t bytes, void* dst, hipStream_t st);
hipError_t launch_momentum(const MatDesc* d, int n, const EwGroups& g, float mu, int nesterov,
                           hipStream_t st);
hipError_t launch_norm_finalize(const MatDesc* d, int n, float eps, hipStream_t st);
hipError_t launch_apply(const MatDesc* d, int n, const EwGroups& g, int final_parity, float lr,
                        float wd, float qk_tau, hipStream_t st);

// bf16 Newton-Schulz phases over all matrices of one size class (kLarge or
// kSmall).  `it` is the iteration index (0-based): it selects the ping-pong
// buffers and, for it == 0, folds the normalisation s = 1/(||Y||+eps) into
// the epilogues.  Tiles are dealt to XCDs by `xs` (see XcdSplit).
// split: the class's Gram launch is K-split (p.gram counts tasks); the reduce
// launch (over p.tri's `tiles` triangle tiles) then forms A
hipError_t launch_gram_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                            int small, int split, hipStream_t st);
hipError_t launch_gram_reduce_bf16(const MatDesc* d, int n, Prefix p, int tiles, int it, int small,
                                   hipStream_t st);
// poly writes B = a I + b A + c A A, so the update is the plain product B X
// small: 128-tiles (the small class, or a large-class launch with few
// 256-tiles), else 256-tiles
hipError_t launch_poly_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, float a,
                            float b, float c, int small, hipStream_t st);
hipError_t launch_update_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                              int small, hipStream_t st);
// the small class's update in strips of `strip` consecutive column tiles per
// workgroup; prefix_strip: strips per matrix, prefix-summed.  Each strip
// forms B = a I + b A + c A A from A itself (no polynomial launch for the
// class).  next_gram: each strip also stores its part of the next
// iteration's K-split Gram (the strip count per matrix equals its gram_split).
// stream: one workgroup per compute unit streaming its tiles (the class runs
// alone in the call), else two per compute unit.  apply (last iteration,
// stream only, every matrix eligible: ClassPlan::fuse_apply): the strips
// update W in place, W <- decay W - lr scale X, in place of the apply launch
hipError_t launch_update_strip_bf16(const MatDesc* d, int n, const int32_t* prefix_strip,
                                   const XcdSplit& xs, int it, int strip, int next_gram, int stream,
                                   int apply, float a, float b, float c, float decay, float lr,
                                   hipStream_t st);

// fp32 class (p.gram == p.tri: the prefix counts every tile of the square).
// kmax: the largest K of the launch's matrices (n' for the Gram, m' for the
// polynomial and the update); up to 64 an FMA kernel stages a tile's whole K
// extent in LDS at once, above that the launch runs on the matrix cores
hipError_t launch_gram_f32(const MatDesc* d, int n, Prefix p, int total, int it, int kmax,
                           hipStream_t st);
hipError_t launch_poly_f32(const MatDesc* d, int n, Prefix p, int total, int kmax, float b, float c,
                           hipStream_t st);
hipError_t launch_update_f32(const MatDesc* d, int n, Prefix p, int total, int it, int kmax, float a,
                             hipStream_t st);
// the fp32 products on the matrix cores, for launches whose K exceeds what
// the FMA kernel stages whole; phase: 0 Gram, 1 polynomial, 2 update; prefix
// and total as for the FMA launches (64-tiles); kmax as above: up to 256 each
// 64-tile is four workgroups of 32 x 32 that split K over their waves, above
// that one workgroup per 64-tile pipelines its K
hipError_t launch_f32_mfma(int phase, const MatDesc* d, int n, const int32_t* prefix, int total, int it,
                           int kmax, float a, float b, float c, hipStream_t st);

// single-phase test hooks (one matrix, caller buffers)
hipError_t launch_gram_bf16_single(const void* X, void* A, int m, int n, int64_t ldx, int64_t lda,
                                   float s2, int cus, hipStream_t st);
hipError_t launch_poly_bf16_single(const void* A, void* B, int m, int64_t lda, float a, float b,
                                   float c, int cus, hipStream_t st);
hipError_t launch_update_bf16_single(const void* X, const void* B, void* Xo, int m, int n,
                                     int64_t ldx, int64_t ldb, float s, int cus, hipStream_t st);

// AdamW: tensors travel in kernel arguments, kAdamwGroup per launch (about
// 12 KB of arguments), so a model's many small norm and bias tensors share a
// launch: each extra launch costs about 16 us, launch gap included.
constexpr int kAdamwGroup = 256;
struct AdamwGroup {
    void* param[kAdamwGroup];
    const void* grad[kAdamwGroup];
    float* m[kAdamwGroup];
    float* v[kAdamwGroup];
    int64_t numel[kAdamwGroup];
    int32_t block_prefix[kAdamwGroup + 1];
    uint8_t param_bf16[kAdamwGroup];
    uint8_t grad_bf16[kAdamwGroup];
    uint8_t vec4[kAdamwGroup];
    int32_t count;
};
static_assert(sizeof(AdamwGroup) <= 16384, "AdamW group must fit a 16 KB argument block");
constexpr int kAdamwChunk = 4096;  // elements per workgroup
hipError_t launch_adamw(const AdamwGroup& g, int total_blocks, float lr, float beta1, float beta2,
                        float eps, float wd, float bc1, float bc2, const float* gscale,
                        hipStream_t st);
hipError_t launch_adamw_sumsq(const AdamwGroup& g, int total_blocks, float* partials,
                              int block_offset, hipStream_t st);
hipError_t launch_clip_finalize(const float* partials, int nblocks, float max_norm, float* scale,
                                float* norm_out, hipStream_t st);

}  // namespace muon
