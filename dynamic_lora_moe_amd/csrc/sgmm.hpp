// Structures shared between the host API (api.hip) and the SGMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dlm {

// ---- SGMM -----------------------------------------------------------------

struct SgDesc {
    const void* x;
    const void* A;
    const void* Ap;     // packed copy of A ([E][d_in / 8][r][8]), or nullptr
    const void* B;
    void* y;
    int32_t d_in, d_out;
    int32_t n_cb;       // column groups of the expand (kSgmmExpandCols each)
    int32_t n_ks;       // kSgmmKSlice-wide K slices of the shrink
    int64_t ks0;        // first K slice of this problem (prefix sum of n_ks)
    int64_t unit0;      // first column block of this problem (prefix sum of n_cb)
};

// Workspace sections (byte offsets, each 256-aligned).
struct SgLayout {
    // perm: row at each sorted position (-1 = padding); epk: its expert pair
    // (slot 0 in the low 16 bits, slot 1 in the high, -1 = empty); gpk: its two
    // gates; hist, cerr: each segmentation chunk's key counts and bad-set flag;
    // v: the shrink's results
    // dep, xcd: the one-launch shrink + expand's per-(problem, tile) counts of
    // finished shrink items and its per-XCD work ranges
    size_t hdr, perm, epk, gpk, hist, cerr, v, dep, xcd, total;
    int64_t T, T_pad, tiles_max, n_chunks;
    int r_pad;
    int max_ks;  // K slices of the widest problem
};
// Width of one shrink K slice (one work item; its fp32 partial v is summed
// with the other slices' afterwards).
constexpr int kSgmmKSlice = 2048;
// Up to this rank the expand adds a tile's K-slice partials itself; above it a
// K-slice sum launch runs between the shrink and the expand.
constexpr int kSgmmFoldRank = 64;
SgLayout sgmm_layout(int64_t T, int64_t d_in_max, int E, int r, int n_prob);

// Rows per segmentation chunk (one workgroup of the segmentation kernels).
constexpr int kSgmmSegRows = 1024;
// Up to this many rows the segmentation is one launch (each workgroup counts
// every chunk's rows); above it a count launch runs first.
constexpr int kSgmmSegFewRows = 8192;

// Output columns one SGMM expand work item covers (4 waves x 4 x 64).
constexpr int kSgmmExpandCols = 1024;

// Single-problem calls with at most this many rows (bf16) take one launch:
// each column group computes the rank vectors itself instead of a
// segmentation, a shrink and a K-slice sum running first.
constexpr int kSgmmSmallT = 4;

// Up to this many rows (one wave's lanes) the shrink and expand workgroups
// order the rows themselves (the segmentation's order, computed by one wave),
// so there is no segmentation launch; batches that need the K-slice sum launch
// keep it.
constexpr int kSgmmInlineRows = 64;

// Header words of the workspace.
enum { SG_ERR = 0, SG_NPOS = 1, SG_NTILES = 2 };
// Words per XCD of the one-launch shrink + expand's work ranges.
constexpr int kSgmmXcdWords = 16;
// One-launch shrink + expand after the segmentation (bf16, ranks up to
// kSgmmFoldRank): 0 off, 1 for segmented batches, 2 also for batches of up to
// kSgmmInlineRows rows (segmented first instead of ordered in the kernels).
#ifndef DLM_SGMM_FUSED
#define DLM_SGMM_FUSED 2
#endif
constexpr int kSgmmFused = DLM_SGMM_FUSED;
// Its counts hold K slices in 16 bits and K slices x (XCD id + 1) in 15: up to
// this many K slices per problem.
constexpr int kSgmmFusedMaxKs = 4095;
// It pays from this many (problem, tile) pairs on (32 per XCD); smaller batches,
// whose few items would mostly wait on each other, keep two launches.
constexpr int64_t kSgmmFusedMinPairs = 256;

struct SgmmArgs {
    const SgDesc* descs;    // device table, or nullptr to use `single`
    const SgDesc* ks_desc;  // the owning problem's descriptor per K slice (device; with descs)
    const SgDesc* cb_desc;  // the owning problem's descriptor per expand column group (device; with descs)
    SgDesc single;
    int32_t n_prob;
    int64_t n_expand_units;  // tiles_max * total_cb
    int64_t total_cb;        // sum over problems of their expand column groups
    int64_t total_ks;        // sum over problems of their shrink K slices
    int64_t d_out_max;       // largest d_out over the problems
    int32_t packed;          // 1: the shrink reads every problem's packed A (Ap)
    const int32_t* idx;
    const float* g;
    int64_t T;
    int32_t E, r;
    float scale;
    char* ws;
    SgLayout L;
    int32_t* status_out;   // device word that also receives the set-validity flag, or nullptr
    int32_t inline_seg;    // 1: the shrink and expand order the rows themselves (launch_sgmm sets it)
    int32_t w_max;         // largest K slices + column groups of one problem
};

hipError_t launch_sgmm(const SgmmArgs& a, int dtype, hipStream_t s);
// Ap[e][k / 8][rho][0..8) = A[e][rho][k..k+8) for k = 0, 8, ..., d_in - 8 (bf16).
hipError_t launch_sgmm_pack_a(const void* A, void* Ap, int E, int r, int64_t d_in, hipStream_t s);

}  // namespace dlm
