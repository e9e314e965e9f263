// Host-side planning of one Muon step: validation, size classes, the order
// of the descriptor table, tile prefixes, per-XCD tile ranges and the
// workspace layout.  Plain C++ (no HIP), so that it is also built and checked
// on its own under host sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "../../include/muon.h"
#include "layout.h"

namespace muon {

// Tiles and launch ranges of one size class.
struct ClassPlan {
    int first = 0, count = 0;           // descriptor range [first, first + count)
    std::vector<int32_t> pgram, ptri, ppoly, pupd;  // count + 1 entries each (see Prefix)
    size_t off_pgram = 0, off_ptri = 0, off_ppoly = 0, off_pupd = 0;  // their workspace offsets
    int total_gram = 0, total_tri = 0, total_poly = 0, total_upd = 0;
    bool gram_split = false;            // the Gram launch runs K-split (bf16 classes)
    bool poly_small = false;            // large class: the polynomial runs on 128-tiles
    // small class: the update in strips of `strip` consecutive column tiles
    // per workgroup (0: one tile per workgroup, the ordinary update launch)
    int strip = 0;
    std::vector<int32_t> pstrip;        // strips per matrix, count + 1 entries
    size_t off_pstrip = 0;
    int total_strips = 0;
    XcdSplit xs_strip{};
    // small class, K-split Gram and strips with as many strips per matrix as
    // Gram parts: from the second iteration on, the update's strips store the
    // Gram parts and the split Gram launch is skipped
    bool fuse_gram = false;
    // small class alone in the call: strips for one workgroup per compute
    // unit, streamed (and a K-split Gram cut into as many parts as strips);
    // else strips for two workgroups per compute unit
    bool stream = false;
    // streamed, and every matrix an fp32 weight of exactly 128 rows and a
    // multiple of 128 columns (not transposed, no padding), rows 16-byte
    // aligned, without QK-Clip or an update output: the last update applies
    // the step to W itself and no apply launch runs
    bool fuse_apply = false;
    int kmax_n = 0, kmax_m = 0;         // largest padded n' and m' of the class
    XcdSplit xs_gram{}, xs_poly{}, xs_upd{};  // bf16 classes: per-XCD tile ranges of equal work
};

struct Plan {
    std::vector<MatDesc> d;          // descriptor table, in launch order
    std::vector<int> order;          // d[k] describes the caller's matrix order[k]
    std::vector<int32_t> pew;        // elementwise tiles of all kinds (norm partial offsets)
    std::vector<int32_t> pek[kNumEwKinds];  // elementwise tiles by kind (launch prefixes)
    ClassPlan cls[kNumClasses];
    size_t off_pek[kNumEwKinds] = {};
    size_t table_bytes = 0;          // descriptor table + prefixes, at the workspace start
    size_t off_partials = 0, off_invnorm = 0, total = 0;
    int total_ek[kNumEwKinds] = {};
};

// Everything about one call that does not touch the device.  `ws` is the
// workspace address the descriptors point into (0 to size the workspace
// only); `need_ptrs` checks the tensor pointers too (alignment, overlap);
// `cus` is the number of compute units per XCD.  Any status other than
// MUON_OK leaves P unspecified.
muon_status make_plan(const muon_matrix* mats, int n, const muon_hparams* hp, bool need_ptrs,
                      uintptr_t ws, int cus, Plan& P);

// K-parts per matrix for a Gram launch over `tiles[k]` tiles of `slabs[k]`
// 64-wide K slabs each, with `cus_total` workgroup slots: all 1 unless the
// tiles fill at most a quarter of the slots; then, for the shortest part
// length L (at least kMinSplitSlabs, and at least the total work over
// cus_total) at which the tasks still fit one round, floor(slabs / L) parts
// (between 1 and kMaxSplit), so every part holds at least L slabs.
std::vector<int32_t> gram_splits(const std::vector<int32_t>& tiles,
                                 const std::vector<int32_t>& slabs, int cus_total);

// Host image of the workspace's first P.table_bytes bytes: the descriptors
// and every prefix array.
void table_image(const Plan& P, std::vector<char>& out);

// Caller indices (ascending, no repeats) of the matrices that hold a tile at
// the start or end of a per-XCD range of a bf16 GEMM launch, or quarter tiles.
std::vector<int> split_matrices(const Plan& P);

// Per-matrix multiplier of the orthogonalised update (muon_scale_mode).
double shape_multiplier(int mode, int64_t rows, int64_t cols);

constexpr int64_t kMaxDim = 1 << 20;

}  // namespace muon
