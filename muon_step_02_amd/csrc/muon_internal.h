// Internal declarations shared by the HIP sources of libmuon (gfx950 only).
//
// Device-side view of one Muon matrix, the workspace layout and the launch
// wrappers of every kernel.  Nothing here is part of the public ABI
// (include/muon.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/muon.h"

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

// Canonical Newton-Schulz buffers are padded to these multiples so the GEMM
// kernels run on whole tiles with no bounds checks.  The padding is zero and
// the iteration keeps it zero: zero rows/cols of X give zero rows/cols of
// A = X X^T, B = a I + b A + c A A is a I on the padded block, and B X maps
// the zero padded rows of X to zero.  bf16 matrices whose short side is at most
// kSmallBf16 use 128-wide tiles and padding ("small" class), the others 256.
constexpr int kPadBf16 = 256;
constexpr int kSmallBf16 = 128;
constexpr int kPadF32 = 64;
// Elementwise kernels (momentum, apply) work on tiles of the weight:
// 16 x 256 where the bf16 iteration reads Y as it is; kTrTH x kTrTW, through
// LDS, where it reads Y^T (or the padded width is not a multiple of 256);
// kEwTile x kEwTile for the fp32 iteration.  Padded dimensions are multiples
// of every tile edge used on them.
constexpr int kEwTile = 64;
constexpr int kTrTH = 64, kTrTW = 128;

// One matrix as the kernels see it.  Built on the host, copied into the
// workspace once per call.
struct MatDesc {
    // caller tensors
    void* param;
    const void* grad;
    float* mom;
    float* update_out;
    float* norm_out;
    const float* qk_smax;   // optional: max attention logit per block of qk_block_rows rows
    int64_t qk_block_rows;
    int64_t rows, cols;
    int64_t ld_param, ld_grad, ld_mom;
    int32_t param_dtype, grad_dtype;
    int32_t transposed;  // rows > cols: the iteration runs on W^T
    int32_t mp, np;      // padded canonical dims: m' = min, n' = max
    int32_t rows_pad, cols_pad;
    int32_t ew_th, ew_tw;  // elementwise tile: 16 x 256, kTrTH x kTrTW or kEwTile x kEwTile
    int32_t ew_tiles_c;    // elementwise tiles along cols_pad
    int32_t ew_tiles;      // elementwise tiles of this matrix (one norm partial each)
    int32_t vec4;        // 1: every row start of param/grad/mom is 16B aligned and cols % 4 == 0
    float scale;         // shape multiplier * extra_scale
    // workspace buffers (bf16 or f32 elements by ns dtype)
    void* x[2];   // canonical X, mp x np, ld np (ping-pong)
    void* xt[2];  // X^T, np x mp, ld mp (ping-pong; fp32 iteration only, else null)
    void* a;      // A = X X^T, mp x mp
    void* b;      // B = b A + c A A, mp x mp
    float* partials;  // one sum of squares per elementwise tile
    float* inv_norm;  // s = 1/(||Y||_F + eps)
};

// Grouped launches: workgroup -> (matrix, local tile) through prefix sums of
// tiles per matrix (int32 entries, n+1 of them).
struct Prefix {
    const int32_t* gram;  // triangle tiles (Gram and polynomial)
    const int32_t* upd;   // full tiles of the update
};

// Elementwise tiles by kind: 0 streaming (16 x 256), 1 through LDS (the
// transposing and the fp32 shapes).  Each kind is its own launch, so the
// streaming kernel keeps the occupancy of its small register and LDS
// footprint; its prefix runs over all matrices, those of the other kind
// having no tiles in it.
struct EwGroups {
    const int32_t* prefix[2];
    int tiles[2];
};

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
// kernel arguments, kTableChunkWords words per launch.
constexpr int kTableChunkWords = 512;
hipError_t launch_table_upload(const void* host, size_t bytes, void* dst, hipStream_t st);
hipError_t launch_momentum(const MatDesc* d, int n, const EwGroups& g, float mu, int nesterov,
                           int ns_f32, hipStream_t st);
hipError_t launch_norm_finalize(const MatDesc* d, int n, float eps, hipStream_t st);
hipError_t launch_apply(const MatDesc* d, int n, const EwGroups& g, int final_parity, float lr,
                        float wd, float qk_tau, int ns_f32, hipStream_t st);

// bf16 Newton-Schulz phases over all matrices.  `it` is the iteration index
// (0-based): it selects the ping-pong buffers and, for it == 0, folds the
// normalisation s = 1/(||Y||+eps) into the epilogues.
// `small` selects the 128-tile kernels for the small class.
//
// Workgroups are dealt to the 8 XCDs round-robin (workgroup b runs on XCD
// b % 8).  XcdSplit gives XCD x the contiguous tile range [b[x], b[x+1]):
// tiles that share operand slabs then share one L2, and the ranges are cut
// at equal work (tiles weighted by their K), not equal tile counts.
//
// An XCD runs its tiles in rounds of one tile per CU.  When the last round
// would leave at least half of the CUs idle, its sub[x] tiles are run as
// four quarter tiles each instead (task order: whole tiles, then the quarters
// of the remaining tiles, four consecutive tasks per tile).  The grid is
// 8 * per workgroups, per = the largest task count of an XCD.
struct XcdSplit {
    int32_t b[9];
    int32_t per;
    int32_t sub[8];
};
// Split `ntiles[k]` tiles of weight `weight[k]` (matrix order) into 8 ranges;
// with `quarters`, the short last round of each range is split as above
// (cus = compute units per XCD).
XcdSplit xcd_split(const int32_t* ntiles, const int64_t* weight, int n, int cus, int quarters);

hipError_t launch_gram_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                            int small, hipStream_t st);
// poly writes B = a I + b A + c A A, so the update is the plain product B X
hipError_t launch_poly_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, float a,
                            float b, float c, int small, hipStream_t st);
hipError_t launch_update_bf16(const MatDesc* d, int n, Prefix p, const XcdSplit& xs, int it,
                              int small, hipStream_t st);
int gemm_tile_bf16(int small);  // square tile edge of the Gram/polynomial kernels
int upd_tile_m_bf16(int small);
int upd_tile_n_bf16(int small);

hipError_t launch_gram_f32(const MatDesc* d, int n, Prefix p, int total, int it, hipStream_t st);
hipError_t launch_poly_f32(const MatDesc* d, int n, Prefix p, int total, float b, float c,
                           hipStream_t st);
hipError_t launch_update_f32(const MatDesc* d, int n, Prefix p, int total, int it, float a,
                             hipStream_t st);
constexpr int kTileF32 = 64;

// single-phase test hooks (one matrix, caller buffers)
hipError_t launch_gram_bf16_single(const void* X, void* A, int m, int n, int64_t ldx, int64_t lda,
                                   float s2, int cus, hipStream_t st);
hipError_t launch_poly_bf16_single(const void* A, void* B, int m, int64_t lda, float a, float b,
                                   float c, int cus, hipStream_t st);
hipError_t launch_update_bf16_single(const void* X, const void* B, void* Xo, int m, int n,
                                     int64_t ldx, int64_t ldb, float s, int cus, hipStream_t st);

// AdamW: tensors travel in kernel arguments, kAdamwGroup per launch.
constexpr int kAdamwGroup = 32;
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
constexpr int kAdamwChunk = 4096;  // elements per workgroup
hipError_t launch_adamw(const AdamwGroup& g, int total_blocks, float lr, float beta1, float beta2,
                        float eps, float wd, float bc1, float bc2, const float* gscale,
                        hipStream_t st);
hipError_t launch_adamw_sumsq(const AdamwGroup& g, int total_blocks, float* partials,
                              int block_offset, hipStream_t st);
hipError_t launch_clip_finalize(const float* partials, int nblocks, float max_norm, float* scale,
                                float* norm_out, hipStream_t st);

}  // namespace muon
