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
    // gates; tmask: the experts each 32-row tile uses; v: the shrink's results
    size_t hdr, perm, epk, gpk, tmask, v, total;
    int64_t T, T_pad, tiles_max;
    int r_pad;
    int max_ks;  // K slices of the widest problem
};
// Width of one shrink K slice.
constexpr int kSgmmKSlice = 512;
SgLayout sgmm_layout(int64_t T, int64_t d_in_max, int E, int r, int n_prob);

// Output columns one SGMM expand work item covers (4 waves x 4 x 64).
constexpr int kSgmmExpandCols = 1024;

// Header words of the workspace.
enum { SG_ERR = 0, SG_NPOS = 1, SG_NTILES = 2 };

struct SgmmArgs {
    const SgDesc* descs;   // device table, or nullptr to use `single`
    const int32_t* ks_owner;  // problem of each K slice (device; with descs)
    const int32_t* cb_owner;  // problem of each expand column group (device; with descs)
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
};

hipError_t launch_sgmm(const SgmmArgs& a, int dtype, hipStream_t s);
// Ap[e][k / 8][rho][0..8) = A[e][rho][k..k+8) for k = 0, 8, ..., d_in - 8 (bf16).
hipError_t launch_sgmm_pack_a(const void* A, void* Ap, int E, int r, int64_t d_in, hipStream_t s);

}  // namespace dlm
