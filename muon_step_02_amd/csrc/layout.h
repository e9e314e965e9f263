// Data layout shared by the host planner and the kernels of libmuon.
//
// Plain C++ (no HIP headers): the planner in plan.cpp is also built on its
// own with host sanitizers.  Nothing here is part of the public ABI
// (include/muon.h is).
#pragma once

#include <stdint.h>

namespace muon {

// Size classes of the Newton-Schulz iteration.  Each class has its own GEMM
// kernels, tile edge and buffer padding, and its own grouped launches.
//   kLarge: bf16 operands, 256 x 256 tiles, padding 256;
//   kSmall: bf16 operands, short side <= kSmallBf16: 128 x 128 tiles, padding 128;
//   kF32:   fp32 operands, 64 x 64 tiles, padding 64.  Every matrix when the
//           caller asks for the fp32 iteration; with the bf16 iteration, the
//           matrices whose short side is at most kTinyF32 (a bf16 iteration
//           on a handful of singular values misses the bf16 tolerance on some
//           inputs: its rounding errors do not average out).
enum SizeClass { kLarge = 0, kSmall = 1, kF32 = 2, kNumClasses = 3 };
constexpr int kSmallBf16 = 128;
constexpr int kTinyF32 = 32;
constexpr int kClassPad[kNumClasses] = {256, 128, 64};
constexpr int kClassTile[kNumClasses] = {256, 128, 64};  // square tiles, all three phases
constexpr int kTileF32 = 64;
// Split-K of tile-starved Gram launches: a part covers at least kMinSplitSlabs
// 64-wide K slabs, and a tile has at most kMaxSplit parts.
constexpr int kGemmBK = 64;
constexpr int kMinSplitSlabs = 8;
constexpr int kMaxSplit = 16;

// Elementwise kernels (momentum, apply) work on tiles of the weight, one
// kind per launch:
//   kEwStream: 16 x 256 where the bf16 iteration reads Y as it is;
//   kEwTrans:  kTrTH x kTrTW through LDS where the bf16 iteration reads Y^T
//              (or the padded width is not a multiple of 256);
//   kEwF32:    kEwTile x kEwTile for the fp32 iteration, which keeps X and X^T.
// Padded dimensions are multiples of every tile edge used on them.
enum EwKind { kEwStream = 0, kEwTrans = 1, kEwF32 = 2, kNumEwKinds = 3 };
constexpr int kEwTile = 64;
constexpr int kTrTH = 64, kTrTW = 128;
static_assert(kClassPad[kSmall] % kTrTH == 0 && kClassPad[kSmall] % kTrTW == 0,
              "transposing elementwise tiles must divide every bf16 padding");
static_assert(kClassPad[kF32] % kEwTile == 0, "fp32 elementwise tiles must divide the fp32 padding");
static_assert(kClassTile[kF32] == kTileF32, "fp32 GEMM tile");

// One matrix as the kernels see it.  Built on the host, carried into the
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
    int32_t ew_th, ew_tw;  // elementwise tile (see EwKind)
    int32_t ew_tiles_c;    // elementwise tiles along cols_pad
    int32_t ew_tiles;      // elementwise tiles of this matrix (one norm partial each)
    int32_t vec4;        // 1: every row start of param/grad/mom is 16B aligned and cols % 4 == 0
    int32_t cls;         // SizeClass
    int32_t gram_split;  // K-parts of each Gram tile (1: unsplit; see Prefix)
    float scale;         // shape multiplier * extra_scale
    // workspace buffers (bf16, or f32 elements for the kF32 class)
    void* x[2];   // canonical X, mp x np, ld np (ping-pong)
    void* xt[2];  // X^T, np x mp, ld mp (ping-pong; kF32 class only, else null)
    void* a;      // A = X X^T, mp x mp
    void* b;      // B = a I + b A + c A A, mp x mp
    float* partials;  // one sum of squares per elementwise tile
    float* inv_norm;  // s = 1/(||Y||_F + eps)
    float* gram_part; // split Gram: fp32 partial tiles [part][tile][BM][BN] (task order)
};

// Grouped launches: workgroup -> (matrix, local task) through prefix sums of
// tasks per matrix (int32 entries, n+1 of them).
//
// A Gram launch with too few tiles to fill the chip (less than one tile per
// compute unit) is split along K: matrix k's Gram tiles are computed in
// gram_split parts of its K range each, as fp32 partial tiles, and a reduce
// launch sums the parts in a fixed order and writes A (scaled, rounded,
// mirrored).  Its Gram launch then runs tiles * gram_split tasks (part-major:
// task t is part t / tiles of tile t % tiles).
struct Prefix {
    const int32_t* gram;  // Gram tasks (tiles, or tiles * gram_split when split)
    const int32_t* tri;   // triangle tiles: the reduce of a split Gram, and the
                          // polynomial (of a large-class launch that runs on
                          // 128-tiles, the triangle of those)
    const int32_t* upd;   // update tiles
};

// Elementwise tiles by kind: each kind is its own launch over all matrices
// (matrices of another kind have no tiles in it), so each kernel keeps the
// occupancy of its own register and LDS footprint.
struct EwGroups {
    const int32_t* prefix[kNumEwKinds];
    int tiles[kNumEwKinds];
};

// Workgroups of a grouped GEMM launch are dealt to the 8 XCDs round-robin
// (workgroup b runs on XCD b % 8, as its task b / 8).  An XCD runs its tasks
// in rounds of one tile per compute unit (`cus` of them).  Two ways of
// dealing tiles to XCDs:
//
//   ranges (interleaved == 0): XCD x takes the contiguous tile range
//     [b[x], b[x+1]), cut at equal work (tiles weighted by their K), so the
//     tiles that share operand slabs share one L2;
//   interleaved rounds (interleaved == 1): the first `rounds` rounds deal
//     chunks of `cus` consecutive tiles to the XCDs in turn (XCD x, round r:
//     chunk 8 r + x), so in each round the 8 XCDs work on neighbouring tiles
//     of the same matrices and the operand panels they share come from the
//     memory-side cache instead of HBM; the remaining tiles are split into 8
//     contiguous parts [b[x], b[x+1]).
//
// In both, when the last round of an XCD would leave at least half of its
// compute units idle, its sub[x] tiles are run as four quarter tiles each
// (task order: whole tiles, then the quarters of the remaining tiles, four
// consecutive tasks per tile).  The grid is 8 * per workgroups, per = the
// largest task count of an XCD.
struct XcdSplit {
    int32_t b[9];
    int32_t per;
    int32_t sub[8];
    int32_t interleaved;
    int32_t rounds;  // interleaved: full rounds dealt chunk by chunk
    int32_t cus;     // compute units per XCD (chunk length)
};
// Deal `ntiles[k]` tiles of weight `weight[k]` (matrix order) to the 8 XCDs
// as above; `quarters` allows the quarter tiles of a short last round.
XcdSplit xcd_split(const int32_t* ntiles, const int64_t* weight, int n, int cus, int quarters,
                   int interleaved = 0);

}  // namespace muon
