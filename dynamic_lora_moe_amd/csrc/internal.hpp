// Structures shared between the host API (api.hip) and the switch and router
// kernels (the SGMM's are in sgmm.hpp).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dlm {

// A launch covers at most 2^32 - 1 work-items along x (the dispatch packet's
// grid size is 32 bits).  Launchers check their grid with this before they
// launch anything and refuse one past it with hipErrorInvalidConfiguration,
// rather than letting the block count wrap when it is narrowed.
inline bool grid_fits(int64_t blocks, int64_t threads_per_block) {
    return blocks >= 0 && blocks <= (int64_t)0xffffffffLL / threads_per_block;
}

// ---- fused switch ---------------------------------------------------------

// One adapted weight in the device table of a dlm_layers handle.
struct SwDesc {
    void* W;            // [d_out][d_in]
    const void* A;      // [E][r][d_in]
    const void* B;      // [E][d_out][r]
    int32_t d_out, d_in;
    int32_t n_rt, n_ct; // row tiles x column tiles of this weight
    int64_t tile0;      // index of its first tile in the launch (prefix sum)
    int64_t elem0;      // index of its first element (generic path)
    const void* Ap;     // packed A images of the wide tiles (ranks 17..64), else null
    // merged-weight products (dlm_gemv / dlm_switch_gemv), once vectors are bound
    const void* xv;     // [d_in], the weight's input
    float* yv;          // [d_out] fp32, its output
    float* part;        // [n_ct][d_out] fp32 per-column-tile partial products (fused path)
    int64_t rb0;        // index of its first kGemvRows-row block in a product launch
    int64_t rt0;        // index of its first 256-row band in a partial-sum launch
    int64_t ks0;        // index of its first kLoraKSlice-wide K slice (unmerged product)
    int32_t n_ks;       // its K slices
};

struct SwitchArgs {
    const SwDesc* descs;
    int32_t n_desc;
    int32_t E, r;
    float scale;
    int64_t n_units;    // tiles (MFMA path) or elements (generic path)
    int64_t per_xcd;    // units per XCD chunk (MFMA path)
    const int32_t* old_idx;
    const float* old_g;
    const int32_t* new_idx;
    const float* new_g;
    int32_t* err;
    const void* zimg;   // one all-zero A image (inactive slots of the wide tiles)
    float* vpart;       // unmerged product: per K slice the partial rank vectors [2][r]
};

// Tile geometry of the bf16 MFMA switch for a padded rank.
struct SwTile {
    int r16;   // padded rank / 16
    int ct;    // columns per tile
    int rt;    // rows per tile
};
SwTile switch_tile_for_rank(int r);

// Once per handle, on the handle's device, before its first launch: raises the
// dynamic-LDS limit of the kernel instance the tile uses where it needs more
// than 64 KB (no stream work; launches then only launch).
hipError_t prepare_switch_bf16(const SwTile& t);
hipError_t launch_switch_bf16(const SwitchArgs& a, const SwTile& t, hipStream_t s);

// Rows per block of the product kernel (one row per wave).
constexpr int kGemvRows = 4;

// y = W x for every weight of a.descs (bound vectors), one launch: n_blocks
// kGemvRows-row blocks over all weights.  With sets in a (after a switch), sets the
// switch rejects leave y alone.
hipError_t launch_gemv(const SwitchArgs& a, int64_t n_blocks, int dtype, hipStream_t s);
// Whether the fused switch + product kernel serves this configuration (bf16,
// ranks up to 16); it writes per-column-tile partial products, which
// launch_gemv_reduce then adds up in a fixed order (n_bands 256-row bands;
// it writes nothing for sets the switch rejects).
bool switch_gemv_fused(const SwTile& t, int dtype);
hipError_t launch_switch_gemv_bf16(const SwitchArgs& a, hipStream_t s);
hipError_t launch_gemv_reduce(const SwitchArgs& a, int64_t n_bands, hipStream_t s);

// The product with one set's adapters unmerged (W untouched):
//   y = W x + sum_k c_k B_{e_k} (A_{e_k} x),  c = s g,
// in two launches: the rank vectors A_e x per (weight, kLoraKSlice-wide K
// slice, group of 8 rank vectors) into a.vpart (n_ks_total slices), then the
// product, each row adding its adapters' B row times the slices' sum.  Sets
// the switch rejects write nothing (the first launch sets the error word).
// a.new_idx / a.new_g must be non-null and a.old_idx null.
constexpr int kLoraKSlice = 2048;
hipError_t launch_gemv_unmerged(const SwitchArgs& a, int64_t n_ks_total, int64_t n_blocks, int dtype,
                                hipStream_t s);

// Packed A images used by the wide tiles (ranks 17..64, bf16): for expert e and
// 64-column block cb of a weight, one contiguous image of the block's A slice
// in the LDS layout the MFMAs read ([half][MFMA row][rank], chunk-swizzled), so
// a tile stages it with direct global->LDS copies.  Zero past d_in.
bool switch_packs_a(const SwTile& t);
size_t switch_packed_a_elems(int64_t d_in, int E, const SwTile& t);  // per weight
size_t switch_zero_image_elems(const SwTile& t);
hipError_t launch_switch_pack_a(const void* A, void* Ap, int64_t d_in, int E, int r, const SwTile& t,
                                hipStream_t s);
hipError_t launch_switch_generic(const SwitchArgs& a, int dtype, hipStream_t s);

// ---- router ---------------------------------------------------------------

hipError_t launch_pregate(const void* x, const void* Wr, int64_t T, int64_t d, int E,
                          int dtype, int32_t* idx, float* g, hipStream_t s);
hipError_t launch_pregate_centroid(const void* x, const void* C, int64_t T, int64_t d, int E, int J, int dtype,
                                   int32_t* idx, float* g, hipStream_t s);

}  // namespace dlm
