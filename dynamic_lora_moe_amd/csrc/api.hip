// Host side of the C ABI declared in include/dlm.h: argument validation (no GPU
// call before it passes), device descriptor tables, launches and status words.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <new>
#include <utility>
#include <vector>

#include "dlm.h"
#include "internal.hpp"
#include "sgmm.hpp"

using namespace dlm;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return code;
}

int ok() {
    g_err[0] = 0;
    return DLM_OK;
}

int hip_fail(hipError_t e, const char* what) {
    if (e == hipErrorInvalidConfiguration)  // the launchers' own refusal (grid_fits)
        return fail(DLM_ESHAPE, "%s: the sizes need a launch grid of more than 2^32 - 1 work-items", what);
    return fail(DLM_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t esize(int dtype) { return dtype == DLM_F32 ? 4 : 2; }

bool valid_dtype(int dtype) { return dtype == DLM_F32 || dtype == DLM_BF16; }

constexpr int64_t kMaxDim = (int64_t)1 << 30;

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
    const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
    return a0 < b0 + nb && b0 < a0 + na;
}

// A byte range a launch reads or writes.  The kernels update buffers in place
// from many workgroups, so a written range that overlaps any other range of the
// same call gives a silent race: such calls are refused.
struct Span {
    uintptr_t lo, hi;  // [lo, hi)
    bool write;
    const char* what;
    int who;
};

Span span(const void* p, size_t bytes, bool write, const char* what, int who) {
    return Span{(uintptr_t)p, (uintptr_t)p + bytes, write, what, who};
}

// First pair of overlapping spans of which at least one is written, or false.
// Sorted by start; for each span, the span reaching furthest so far and the
// written span reaching furthest so far are the only candidates that can
// overlap it while some earlier written span overlaps it, so one pass finds a
// conflict whenever there is one.
bool write_conflict(std::vector<Span> v, Span* a, Span* b) {
    std::sort(v.begin(), v.end(), [](const Span& x, const Span& y) { return x.lo < y.lo; });
    int far = -1, farw = -1;
    for (int k = 0; k < (int)v.size(); ++k) {
        if (v[k].hi <= v[k].lo) continue;
        if (far >= 0 && v[far].hi > v[k].lo && (v[k].write || v[far].write)) {
            *a = v[far];
            *b = v[k];
            return true;
        }
        if (farw >= 0 && v[farw].hi > v[k].lo) {
            *a = v[farw];
            *b = v[k];
            return true;
        }
        if (far < 0 || v[k].hi > v[far].hi) far = k;
        if (v[k].write && (farw < 0 || v[k].hi > v[farw].hi)) farw = k;
    }
    return false;
}

int conflict_fail(const char* call, const Span& a, const Span& b) {
    return fail(DLM_EINVAL, "%s: %s %d overlaps %s %d, and one of them is written in place", call, a.what, a.who,
                b.what, b.who);
}

}  // namespace

// --------------------------------------------------------------- handles ----

struct dlm_layers {
    SwDesc* d_descs = nullptr;
    int32_t* d_err = nullptr;
    void* d_pack = nullptr;       // packed A images of every weight, then the zero image (wide tiles)
    void* d_zimg = nullptr;
    float* d_part = nullptr;      // partial products of the fused switch + product (bound vectors)
    float* d_vpart = nullptr;     // rank-vector partials of the unmerged product (bound vectors)
    int64_t n_ks = 0;             // their K slices over all weights
    bool bound = false;           // dlm_layers_bind_vectors has been called
    int64_t n_blocks = 0, n_bands = 0;  // product blocks (kGemvRows rows) and 256-row bands over all weights
    std::vector<SwDesc> h_descs;
    int32_t n = 0;
    int32_t E = 0, r = 0;
    float scale = 1.f;
    int32_t dtype = 0;
    SwTile tile{};
    int64_t n_tiles = 0, n_elems = 0, per_xcd = 0;
    std::vector<std::pair<uintptr_t, uintptr_t>> w_spans;  // every W, sorted, disjoint
};

// Whether [p, p + bytes) touches any weight the handle writes.
static bool hits_weights(const dlm_layers* h, const void* p, size_t bytes) {
    if (!p) return false;
    const uintptr_t lo = (uintptr_t)p, hi = lo + bytes;
    auto it = std::upper_bound(h->w_spans.begin(), h->w_spans.end(), std::make_pair(lo, UINTPTR_MAX));
    if (it != h->w_spans.begin() && std::prev(it)->second > lo) return true;
    return it != h->w_spans.end() && it->first < hi;
}

static int check_sets(const dlm_layers* h, const int32_t* old_idx, const float* old_g, const int32_t* new_idx,
                      const float* new_g, const char* call) {
    if ((old_idx && !old_g) || (new_idx && !new_g)) return fail(DLM_EINVAL, "%s: a set has indices but no gates", call);
    if (hits_weights(h, old_idx, 8) || hits_weights(h, old_g, 8) || hits_weights(h, new_idx, 8) ||
        hits_weights(h, new_g, 8))
        return fail(DLM_EINVAL, "%s: a set lies inside a weight the switch writes", call);
    return DLM_OK;
}

struct dlm_sgmm_group {
    SgDesc* d_descs = nullptr;          // device block: descriptors, then their per-unit copies
    const SgDesc* d_ks_desc = nullptr;
    const SgDesc* d_cb_desc = nullptr;
    std::vector<SgDesc> h_descs;
    int32_t n = 0;
    int32_t E = 0, r = 0;
    float scale = 1.f;
    int32_t dtype = 0;
    int64_t total_cb = 0, total_ks = 0, d_out_max = 0, d_in_max = 0;
    int32_t w_max = 0;  // largest K slices + column groups of one problem
    // packed copies of the distinct A banks (bf16 groups), owned by the handle
    struct Pack {
        const void* A;
        void* Ap;
        int64_t d_in;
    };
    std::vector<Pack> packs;
    int64_t checked_T = 0;  // largest row count whose buffers were checked for overlaps
};

// Scratch memory of dlm_sgmm_noalloc: one file-scope device array, which each
// device that loads the library holds until the process ends.  In host code
// its name stands for a host-side shadow, not for device memory: the device
// address is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that address is ever handed to a kernel.
constexpr size_t kNoAllocScratchBytes = DLM_SGMM_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

extern "C" {

const char* dlm_last_error(void) { return g_err; }

const char* dlm_version(void) { return "dlm 0.1.0 (gfx950)"; }

// ---------------------------------------------------------------- router ----

int dlm_pregate(const void* x, const void* Wr, int64_t T, int64_t d, int32_t E, int32_t dtype,
                int32_t* idx, float* g, void* stream) {
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(DLM_ESHAPE, "pregate: T=%lld out of range", (long long)T);
    if (d < 1 || d > kMaxDim) return fail(DLM_ESHAPE, "pregate: d=%lld out of range", (long long)d);
    if (E < 2 || E > DLM_MAX_EXPERTS) return fail(DLM_ESHAPE, "pregate: E=%d not in [2, %d]", E, DLM_MAX_EXPERTS);
    if (!valid_dtype(dtype)) return fail(DLM_EDTYPE, "pregate: unknown dtype %d", dtype);
    if (T == 0) return ok();
    if (!x || !Wr || !idx || !g) return fail(DLM_EINVAL, "pregate: null pointer");
    hipError_t e = launch_pregate(x, Wr, T, d, E, dtype, idx, g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "pregate launch");
    return ok();
}

int dlm_pregate_centroid(const void* x, const void* C, int64_t T, int64_t d, int32_t E, int32_t J, int32_t dtype,
                         int32_t* idx, float* g, void* stream) {
    if (T < 0 || T >= ((int64_t)1 << 31)) return fail(DLM_ESHAPE, "pregate_centroid: T=%lld out of range", (long long)T);
    if (d < 1 || d > kMaxDim) return fail(DLM_ESHAPE, "pregate_centroid: d=%lld out of range", (long long)d);
    if (E < 1 || E > DLM_MAX_EXPERTS)
        return fail(DLM_ESHAPE, "pregate_centroid: E=%d not in [1, %d]", E, DLM_MAX_EXPERTS);
    if (J < 1 || J > DLM_MAX_CENTROIDS)
        return fail(DLM_ESHAPE, "pregate_centroid: J=%d not in [1, %d]", J, DLM_MAX_CENTROIDS);
    if (!valid_dtype(dtype)) return fail(DLM_EDTYPE, "pregate_centroid: unknown dtype %d", dtype);
    if (T == 0) return ok();
    if (!x || !C || !idx || !g) return fail(DLM_EINVAL, "pregate_centroid: null pointer");
    hipError_t e = launch_pregate_centroid(x, C, T, d, E, J, dtype, idx, g, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "pregate_centroid launch");
    return ok();
}

// ---------------------------------------------------------------- switch ----

int dlm_layers_create(const dlm_proj* projs, int32_t n, int32_t E, int32_t r, float scale,
                      int32_t dtype, dlm_layers** out) {
    if (!out) return fail(DLM_EINVAL, "layers_create: out is null");
    *out = nullptr;
    if (!projs) return fail(DLM_EINVAL, "layers_create: projs is null");
    if (n < 1) return fail(DLM_EINVAL, "layers_create: n=%d", n);
    if (E < 1 || E > DLM_MAX_EXPERTS) return fail(DLM_ESHAPE, "layers_create: E=%d not in [1, %d]", E, DLM_MAX_EXPERTS);
    if (r < 1 || r > DLM_MAX_RANK) return fail(DLM_ESHAPE, "layers_create: r=%d not in [1, %d]", r, DLM_MAX_RANK);
    if (!valid_dtype(dtype)) return fail(DLM_EDTYPE, "layers_create: unknown dtype %d", dtype);
    if (!std::isfinite(scale)) return fail(DLM_EINVAL, "layers_create: scale is not finite");
    const SwTile tile = switch_tile_for_rank(r);
    std::vector<SwDesc> h(n);
    int64_t tiles = 0, elems = 0, blocks = 0, bands = 0;
    for (int i = 0; i < n; ++i) {
        const dlm_proj& p = projs[i];
        if (!p.W || !p.A || !p.B) return fail(DLM_EINVAL, "layers_create: proj %d has a null pointer", i);
        if (p.d_out < 1 || p.d_in < 1 || p.d_out > kMaxDim || p.d_in > kMaxDim)
            return fail(DLM_ESHAPE, "layers_create: proj %d shape %lldx%lld out of range", i,
                        (long long)p.d_out, (long long)p.d_in);
        if (dtype == DLM_BF16) {
            if (!aligned16(p.W) || !aligned16(p.A) || !aligned16(p.B))
                return fail(DLM_EALIGN, "layers_create: proj %d pointer not 16-byte aligned", i);
            if (p.d_in % 8 != 0)
                return fail(DLM_EALIGN, "layers_create: proj %d d_in=%lld not a multiple of 8", i, (long long)p.d_in);
        }
        SwDesc& d = h[i];
        d.W = p.W;
        d.A = p.A;
        d.B = p.B;
        d.d_out = (int32_t)p.d_out;
        d.d_in = (int32_t)p.d_in;
        d.n_rt = (int32_t)((p.d_out + tile.rt - 1) / tile.rt);
        d.n_ct = (int32_t)((p.d_in + tile.ct - 1) / tile.ct);
        d.tile0 = tiles;
        d.elem0 = elems;
        d.Ap = nullptr;
        d.xv = nullptr;
        d.yv = nullptr;
        d.part = nullptr;
        d.rb0 = blocks;
        d.rt0 = bands;
        blocks += (p.d_out + kGemvRows - 1) / kGemvRows;
        bands += (p.d_out + 255) / 256;
        tiles += (int64_t)d.n_rt * d.n_ct;
        elems += p.d_out * p.d_in;
    }
    {
        std::vector<Span> v;
        const size_t es = esize(dtype);
        for (int i = 0; i < n; ++i) {
            const dlm_proj& p = projs[i];
            v.push_back(span(p.W, (size_t)p.d_out * p.d_in * es, true, "weight W", i));
            v.push_back(span(p.A, (size_t)E * r * p.d_in * es, false, "bank A", i));
            v.push_back(span(p.B, (size_t)E * p.d_out * r * es, false, "bank B", i));
        }
        Span a, b;
        if (write_conflict(std::move(v), &a, &b)) return conflict_fail("layers_create", a, b);
    }
    dlm_layers* hd = new (std::nothrow) dlm_layers();
    if (!hd) return fail(DLM_ENOMEM, "layers_create: host allocation failed");
    hd->n = n;
    hd->E = E;
    hd->r = r;
    hd->scale = scale;
    hd->dtype = dtype;
    hd->tile = tile;
    hd->n_tiles = tiles;
    hd->n_elems = elems;
    hd->per_xcd = (tiles + 7) / 8;
    hd->n_blocks = blocks;
    hd->n_bands = bands;
    hipError_t e = dtype == DLM_BF16 ? prepare_switch_bf16(tile) : hipSuccess;
    if (e == hipSuccess && dtype == DLM_BF16 && switch_packs_a(tile)) {
        // ranks 17..64: packed A images for the copy-staged tiles, one block
        size_t elems_total = 0;
        std::vector<size_t> off(n);
        for (int i = 0; i < n; ++i) {
            off[i] = elems_total;
            elems_total += switch_packed_a_elems(h[i].d_in, E, tile);
        }
        const size_t zero_off = elems_total;
        elems_total += switch_zero_image_elems(tile);
        e = hipMalloc(&hd->d_pack, elems_total * 2);
        if (e == hipSuccess) {
            uint16_t* base = (uint16_t*)hd->d_pack;
            hd->d_zimg = base + zero_off;
            e = hipMemset(hd->d_zimg, 0, switch_zero_image_elems(tile) * 2);
            for (int i = 0; i < n && e == hipSuccess; ++i) {
                h[i].Ap = base + off[i];
                e = launch_switch_pack_a(h[i].A, base + off[i], h[i].d_in, E, r, tile, nullptr);
            }
            if (e == hipSuccess) e = hipDeviceSynchronize();
        }
    }
    if (e == hipSuccess) e = hipMalloc((void**)&hd->d_descs, sizeof(SwDesc) * n);
    if (e == hipSuccess) e = hipMalloc((void**)&hd->d_err, 256);
    if (e == hipSuccess) e = hipMemcpy(hd->d_descs, h.data(), sizeof(SwDesc) * n, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipMemset(hd->d_err, 0, 256);
    if (e != hipSuccess) {
        if (hd->d_descs) (void)hipFree(hd->d_descs);
        if (hd->d_err) (void)hipFree(hd->d_err);
        if (hd->d_pack) (void)hipFree(hd->d_pack);
        delete hd;
        return hip_fail(e, "layers_create");
    }
    for (const SwDesc& q : h)
        hd->w_spans.emplace_back((uintptr_t)q.W, (uintptr_t)q.W + (size_t)q.d_out * q.d_in * esize(dtype));
    std::sort(hd->w_spans.begin(), hd->w_spans.end());
    hd->h_descs = std::move(h);
    *out = hd;
    return ok();
}

int dlm_layers_repack(dlm_layers* h, void* stream) {
    if (!h) return fail(DLM_EINVAL, "layers_repack: null handle");
    if (!h->d_pack) return ok();
    for (const SwDesc& d : h->h_descs) {
        hipError_t e = launch_switch_pack_a(d.A, (void*)d.Ap, d.d_in, h->E, h->r, h->tile, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "layers_repack launch");
    }
    return ok();
}

int dlm_layers_destroy(dlm_layers* h) {
    if (!h) return fail(DLM_EINVAL, "layers_destroy: null handle");
    hipError_t e = hipDeviceSynchronize();
    if (h->d_descs) (void)hipFree(h->d_descs);
    if (h->d_err) (void)hipFree(h->d_err);
    if (h->d_pack) (void)hipFree(h->d_pack);
    if (h->d_part) (void)hipFree(h->d_part);
    if (h->d_vpart) (void)hipFree(h->d_vpart);
    delete h;
    if (e != hipSuccess) return hip_fail(e, "layers_destroy");
    return ok();
}

static SwitchArgs switch_args(const dlm_layers* h, const int32_t* old_idx, const float* old_g,
                              const int32_t* new_idx, const float* new_g) {
    SwitchArgs a;
    a.descs = h->d_descs;
    a.n_desc = h->n;
    a.E = h->E;
    a.r = h->r;
    a.scale = h->scale;
    a.old_idx = old_idx;
    a.old_g = old_g;
    a.new_idx = new_idx;
    a.new_g = new_g;
    a.err = h->d_err;
    a.zimg = h->d_zimg;
    a.vpart = h->d_vpart;
    if (h->dtype == DLM_BF16) {
        a.n_units = h->n_tiles;
        a.per_xcd = h->per_xcd;
    } else {
        a.n_units = h->n_elems;
        a.per_xcd = 0;
    }
    return a;
}

int dlm_switch(dlm_layers* h, const int32_t* old_idx, const float* old_g, const int32_t* new_idx,
               const float* new_g, void* stream) {
    if (!h) return fail(DLM_EINVAL, "switch: null handle");
    const int rc = check_sets(h, old_idx, old_g, new_idx, new_g, "switch");
    if (rc != DLM_OK) return rc;
    const SwitchArgs a = switch_args(h, old_idx, old_g, new_idx, new_g);
    const hipError_t e = h->dtype == DLM_BF16 ? launch_switch_bf16(a, h->tile, (hipStream_t)stream)
                                              : launch_switch_generic(a, h->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "switch launch");
    return ok();
}

int dlm_switch_launches(const dlm_layers* h) { return h ? 1 : 0; }

// ------------------------------------------------- merged-weight products ----

int dlm_layers_bind_vectors(dlm_layers* h, const void* const* x, float* const* y) {
    if (!h || !x || !y) return fail(DLM_EINVAL, "bind_vectors: null argument");
    std::vector<SwDesc> d = h->h_descs;
    for (int i = 0; i < h->n; ++i) {
        if (!x[i] || !y[i]) return fail(DLM_EINVAL, "bind_vectors: vector %d is null", i);
        if (h->dtype == DLM_BF16 && !aligned16(x[i]))
            return fail(DLM_EALIGN, "bind_vectors: x %d not 16-byte aligned", i);
        if (((uintptr_t)y[i] & 3u) != 0) return fail(DLM_EALIGN, "bind_vectors: y %d not 4-byte aligned", i);
        d[i].xv = x[i];
        d[i].yv = y[i];
    }
    {
        // the product reads W, x (and the switch + product also writes W and
        // reads A, B); y is written
        std::vector<Span> v;
        const size_t es = esize(h->dtype);
        for (int i = 0; i < h->n; ++i) {
            v.push_back(span(d[i].W, (size_t)d[i].d_out * d[i].d_in * es, true, "weight W", i));
            v.push_back(span(d[i].A, (size_t)h->E * h->r * d[i].d_in * es, false, "bank A", i));
            v.push_back(span(d[i].B, (size_t)h->E * d[i].d_out * h->r * es, false, "bank B", i));
            v.push_back(span(x[i], (size_t)d[i].d_in * es, false, "vector x", i));
            v.push_back(span(y[i], (size_t)d[i].d_out * 4, true, "vector y", i));
        }
        Span a, b;
        if (write_conflict(std::move(v), &a, &b)) return conflict_fail("bind_vectors", a, b);
    }
    float* part = nullptr;
    float* vpart = nullptr;
    // the unmerged product's K slices: per weight a prefix and a count
    int64_t n_ks = 0;
    for (int i = 0; i < h->n; ++i) {
        d[i].ks0 = n_ks;
        d[i].n_ks = (int32_t)((d[i].d_in + kLoraKSlice - 1) / kLoraKSlice);
        n_ks += d[i].n_ks;
    }
    // launches still in flight on any stream read the current table and
    // partial buffers: let them finish before any is replaced
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = hipMalloc((void**)&vpart, (size_t)n_ks * 2 * h->r * sizeof(float));
    if (e == hipSuccess && switch_gemv_fused(h->tile, h->dtype)) {
        size_t total = 0;
        for (const SwDesc& q : d) total += (size_t)q.n_ct * q.d_out;
        e = hipMalloc((void**)&part, total * sizeof(float));
        size_t off = 0;
        for (int i = 0; i < h->n && e == hipSuccess; ++i) {
            d[i].part = part + off;
            off += (size_t)d[i].n_ct * d[i].d_out;
        }
    }
    if (e == hipSuccess) e = hipMemcpy(h->d_descs, d.data(), sizeof(SwDesc) * h->n, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (part) (void)hipFree(part);
        if (vpart) (void)hipFree(vpart);
        return hip_fail(e, "bind_vectors");
    }
    if (h->d_part) (void)hipFree(h->d_part);
    if (h->d_vpart) (void)hipFree(h->d_vpart);
    h->d_part = part;
    h->d_vpart = vpart;
    h->n_ks = n_ks;
    h->h_descs = std::move(d);
    h->bound = true;
    return ok();
}

int dlm_gemv(dlm_layers* h, void* stream) {
    if (!h) return fail(DLM_EINVAL, "gemv: null handle");
    if (!h->bound) return fail(DLM_EINVAL, "gemv: no vectors bound (dlm_layers_bind_vectors)");
    const SwitchArgs a = switch_args(h, nullptr, nullptr, nullptr, nullptr);
    hipError_t e = launch_gemv(a, h->n_blocks, h->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gemv launch");
    return ok();
}

int dlm_switch_gemv(dlm_layers* h, const int32_t* old_idx, const float* old_g, const int32_t* new_idx,
                    const float* new_g, void* stream) {
    if (!h) return fail(DLM_EINVAL, "switch_gemv: null handle");
    if (!h->bound) return fail(DLM_EINVAL, "switch_gemv: no vectors bound (dlm_layers_bind_vectors)");
    const int rc = check_sets(h, old_idx, old_g, new_idx, new_g, "switch_gemv");
    if (rc != DLM_OK) return rc;
    const SwitchArgs a = switch_args(h, old_idx, old_g, new_idx, new_g);
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (switch_gemv_fused(h->tile, h->dtype)) {
        e = launch_switch_gemv_bf16(a, s);
        if (e == hipSuccess) e = launch_gemv_reduce(a, h->n_bands, s);
    } else {
        e = h->dtype == DLM_BF16 ? launch_switch_bf16(a, h->tile, s) : launch_switch_generic(a, h->dtype, s);
        if (e == hipSuccess) e = launch_gemv(a, h->n_blocks, h->dtype, s);
    }
    if (e != hipSuccess) return hip_fail(e, "switch_gemv launch");
    return ok();
}

int dlm_switch_gemv_launches(const dlm_layers* h) { return h ? 2 : 0; }

int dlm_gemv_unmerged(dlm_layers* h, const int32_t* idx, const float* g, void* stream) {
    if (!h) return fail(DLM_EINVAL, "gemv_unmerged: null handle");
    if (!h->bound) return fail(DLM_EINVAL, "gemv_unmerged: no vectors bound (dlm_layers_bind_vectors)");
    if (!idx || !g) return fail(DLM_EINVAL, "gemv_unmerged: idx or g is null");
    const int rc = check_sets(h, nullptr, nullptr, idx, g, "gemv_unmerged");
    if (rc != DLM_OK) return rc;
    const SwitchArgs a = switch_args(h, nullptr, nullptr, idx, g);
    const hipError_t e = launch_gemv_unmerged(a, h->n_ks, h->n_blocks, h->dtype, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "gemv_unmerged launch");
    return ok();
}

int dlm_gemv_unmerged_launches(const dlm_layers* h) { return h ? 2 : 0; }

int dlm_layers_status(dlm_layers* h, int32_t* code, void* stream) {
    if (!h || !code) return fail(DLM_EINVAL, "layers_status: null argument");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    int32_t v = 0;
    if (e == hipSuccess) e = hipMemcpy(&v, h->d_err, sizeof v, hipMemcpyDeviceToHost);
    if (e == hipSuccess && v != 0) e = hipMemset(h->d_err, 0, sizeof v);
    if (e != hipSuccess) return hip_fail(e, "layers_status");
    *code = v ? DLM_EDEVICE : DLM_OK;
    return ok();
}

// ------------------------------------------------------------------ SGMM ----

int dlm_sgmm_workspace_size(int64_t T, int64_t d_in_max, int32_t E, int32_t r, int32_t n_problems,
                            size_t* bytes) {
    if (!bytes) return fail(DLM_EINVAL, "sgmm_workspace_size: bytes is null");
    if (T < 0 || T > ((int64_t)1 << 30)) return fail(DLM_ESHAPE, "sgmm_workspace_size: T=%lld", (long long)T);
    if (d_in_max < 1 || d_in_max > kMaxDim)
        return fail(DLM_ESHAPE, "sgmm_workspace_size: d_in_max=%lld", (long long)d_in_max);
    if (E < 1 || E > DLM_MAX_EXPERTS) return fail(DLM_ESHAPE, "sgmm_workspace_size: E=%d", E);
    if (r < 1 || r > DLM_MAX_RANK) return fail(DLM_ESHAPE, "sgmm_workspace_size: r=%d", r);
    if (n_problems < 1) return fail(DLM_EINVAL, "sgmm_workspace_size: n_problems=%d", n_problems);
    *bytes = sgmm_layout(T, d_in_max, E, r, n_problems).total;
    return ok();
}

namespace {

int check_problem(const dlm_sgmm_problem& p, int dtype, int i) {
    if (!p.x || !p.A || !p.B || !p.y) return fail(DLM_EINVAL, "sgmm: problem %d has a null pointer", i);
    if (p.d_in < 1 || p.d_out < 1 || p.d_in > kMaxDim || p.d_out > kMaxDim)
        return fail(DLM_ESHAPE, "sgmm: problem %d shape d_in=%lld d_out=%lld", i, (long long)p.d_in,
                    (long long)p.d_out);
    if (dtype == DLM_BF16) {
        if (!aligned16(p.x) || !aligned16(p.A) || !aligned16(p.B) || !aligned16(p.y))
            return fail(DLM_EALIGN, "sgmm: problem %d pointer not 16-byte aligned", i);
        if (p.d_in % 8 != 0 || p.d_out % 8 != 0)
            return fail(DLM_EALIGN, "sgmm: problem %d d_in/d_out not multiples of 8", i);
    }
    return DLM_OK;
}

int check_ws(void* ws, size_t ws_bytes, const SgLayout& L) {
    if (!ws) return fail(DLM_EWORKSPACE, "sgmm: workspace is null");
    if (((uintptr_t)ws & 255u) != 0) return fail(DLM_EALIGN, "sgmm: workspace not 256-byte aligned");
    if (ws_bytes < L.total)
        return fail(DLM_EWORKSPACE, "sgmm: workspace %zu bytes < %zu needed", ws_bytes, L.total);
    return DLM_OK;
}

int run_sgmm(const SgDesc* d_descs, const SgDesc* ks_desc, const SgDesc* cb_desc,
             const SgDesc& single, int n_prob, int64_t total_cb,
             int64_t total_ks, int64_t d_out_max, int32_t w_max, const int32_t* idx, const float* g, int64_t T,
             int E, int r, float scale, int dtype, int packed, void* ws, const SgLayout& L, hipStream_t s,
             int32_t* status_out = nullptr) {
    SgmmArgs a;
    a.w_max = w_max;
    a.status_out = status_out;
    a.inline_seg = 0;  // launch_sgmm decides
    a.descs = d_descs;
    a.ks_desc = ks_desc;
    a.cb_desc = cb_desc;
    a.packed = packed;
    a.single = single;
    a.n_prob = n_prob;
    a.n_expand_units = L.tiles_max * total_cb;
    a.total_cb = total_cb;
    a.total_ks = total_ks;
    a.d_out_max = d_out_max;
    a.idx = idx;
    a.g = g;
    a.T = T;
    a.E = E;
    a.r = r;
    a.scale = scale;
    a.ws = (char*)ws;
    a.L = L;
    hipError_t e = launch_sgmm(a, dtype, s);
    if (e != hipSuccess) return hip_fail(e, "sgmm launch");
    return ok();
}

// Host checks shared by dlm_sgmm and dlm_sgmm_noalloc (everything but the
// workspace).  *done = true: T == 0, nothing to enqueue.
int check_sgmm_args(const void* x, const int32_t* idx, const float* g, const void* A, const void* B, void* y,
                    int64_t T, int64_t d_in, int64_t d_out, int32_t E, int32_t r, float scale, int32_t dtype,
                    const void* ws, size_t ws_bytes, bool* done) {
    *done = false;
    if (T < 0 || T > ((int64_t)1 << 30)) return fail(DLM_ESHAPE, "sgmm: T=%lld out of range", (long long)T);
    if (E < 1 || E > DLM_MAX_EXPERTS) return fail(DLM_ESHAPE, "sgmm: E=%d not in [1, %d]", E, DLM_MAX_EXPERTS);
    if (r < 1 || r > DLM_MAX_RANK) return fail(DLM_ESHAPE, "sgmm: r=%d not in [1, %d]", r, DLM_MAX_RANK);
    if (!valid_dtype(dtype)) return fail(DLM_EDTYPE, "sgmm: unknown dtype %d", dtype);
    if (!std::isfinite(scale)) return fail(DLM_EINVAL, "sgmm: scale is not finite");
    if (T == 0) {  // nothing to do; the (possibly empty) buffers are not looked at
        if (d_in < 1 || d_out < 1 || d_in > kMaxDim || d_out > kMaxDim)
            return fail(DLM_ESHAPE, "sgmm: shape d_in=%lld d_out=%lld", (long long)d_in, (long long)d_out);
        *done = true;
        return DLM_OK;
    }
    dlm_sgmm_problem p{x, A, B, y, d_in, d_out};
    int rc = check_problem(p, dtype, 0);
    if (rc != DLM_OK) return rc;
    if (!idx || !g) return fail(DLM_EINVAL, "sgmm: idx or g is null");
    const size_t es = esize(dtype);
    std::vector<Span> v = {span(x, (size_t)T * d_in * es, false, "x", 0), span(y, (size_t)T * d_out * es, true, "y", 0),
                           span(A, (size_t)E * r * d_in * es, false, "A", 0), span(B, (size_t)E * d_out * r * es, false, "B", 0),
                           span(idx, (size_t)T * 8, false, "idx", 0), span(g, (size_t)T * 8, false, "g", 0)};
    if (ws) v.push_back(span(ws, ws_bytes, true, "workspace", 0));
    Span a, b;
    if (write_conflict(std::move(v), &a, &b)) return conflict_fail("sgmm", a, b);
    return DLM_OK;
}

SgDesc single_desc(const void* x, const void* A, const void* B, void* y, int64_t d_in, int64_t d_out) {
    SgDesc d{};
    d.x = x;
    d.A = A;
    d.B = B;
    d.y = y;
    d.d_in = (int32_t)d_in;
    d.d_out = (int32_t)d_out;
    d.n_cb = (int32_t)((d_out + kSgmmExpandCols - 1) / kSgmmExpandCols);
    d.unit0 = 0;
    d.n_ks = (int32_t)((d_in + kSgmmKSlice - 1) / kSgmmKSlice);
    d.ks0 = 0;
    return d;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on its first use there).
int scratch_on_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "sgmm_noalloc: hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(DLM_EDEVICE, "sgmm_noalloc: device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "sgmm_noalloc: hipGetSymbolAddress(scratch)");
        if (!p) return fail(DLM_EHIP, "sgmm_noalloc: scratch has no device address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DLM_OK;
}

}  // namespace

int dlm_sgmm(const void* x, const int32_t* idx, const float* g, const void* A, const void* B,
             void* y, int64_t T, int64_t d_in, int64_t d_out, int32_t E, int32_t r, float scale,
             int32_t dtype, void* workspace, size_t ws_bytes, void* stream) {
    bool done = false;
    int rc = check_sgmm_args(x, idx, g, A, B, y, T, d_in, d_out, E, r, scale, dtype, workspace, ws_bytes, &done);
    if (rc != DLM_OK) return rc;
    if (done) return ok();
    const SgLayout L = sgmm_layout(T, d_in, E, r, 1);
    rc = check_ws(workspace, ws_bytes, L);
    if (rc != DLM_OK) return rc;
    const SgDesc d = single_desc(x, A, B, y, d_in, d_out);
    return run_sgmm(nullptr, nullptr, nullptr, d, 1, d.n_cb, d.n_ks, d_out, d.n_cb + d.n_ks, idx, g, T, E, r, scale,
                    dtype, 0, workspace, L,
                    (hipStream_t)stream);
}

int dlm_sgmm_noalloc(const void* x, const int32_t* idx, const float* g, const void* A, const void* B,
                     void* y, int64_t T, int64_t d_in, int64_t d_out, int32_t E, int32_t r, float scale,
                     int32_t dtype, int32_t* status, void* stream) {
    bool done = false;
    int rc = check_sgmm_args(x, idx, g, A, B, y, T, d_in, d_out, E, r, scale, dtype, status, status ? 4 : 0, &done);
    if (rc != DLM_OK) return rc;
    if (done) return ok();
    const SgLayout L = sgmm_layout(T, d_in, E, r, 1);
    if (L.total > kNoAllocScratchBytes)
        return fail(DLM_EWORKSPACE, "sgmm_noalloc: needs %zu bytes of scratch, the library's maximum is %zu "
                    "(use dlm_sgmm with a caller workspace)", L.total, kNoAllocScratchBytes);
    int sdev = -1, cdev = -1;
    hipError_t e = hipStreamGetDevice((hipStream_t)stream, &sdev);
    if (e == hipSuccess) e = hipGetDevice(&cdev);
    if (e != hipSuccess) return hip_fail(e, "sgmm_noalloc: stream device");
    if (sdev != cdev) return fail(DLM_EINVAL, "sgmm_noalloc: the stream belongs to device %d, not the current %d", sdev, cdev);
    void* ws = nullptr;
    rc = scratch_on_current_device(&ws);
    if (rc != DLM_OK) return rc;
    const SgDesc d = single_desc(x, A, B, y, d_in, d_out);
    return run_sgmm(nullptr, nullptr, nullptr, d, 1, d.n_cb, d.n_ks, d_out, d.n_cb + d.n_ks, idx, g, T, E, r, scale,
                    dtype, 0, ws, L,
                    (hipStream_t)stream, status);
}

int dlm_sgmm_group_create(const dlm_sgmm_problem* probs, int32_t n, int32_t E, int32_t r,
                          float scale, int32_t dtype, dlm_sgmm_group** out) {
    if (!out) return fail(DLM_EINVAL, "sgmm_group_create: out is null");
    *out = nullptr;
    if (!probs || n < 1 || n > 65535) return fail(DLM_EINVAL, "sgmm_group_create: bad problem list (n=%d)", n);
    if (E < 1 || E > DLM_MAX_EXPERTS) return fail(DLM_ESHAPE, "sgmm_group_create: E=%d", E);
    if (r < 1 || r > DLM_MAX_RANK) return fail(DLM_ESHAPE, "sgmm_group_create: r=%d", r);
    if (!valid_dtype(dtype)) return fail(DLM_EDTYPE, "sgmm_group_create: unknown dtype %d", dtype);
    if (!std::isfinite(scale)) return fail(DLM_EINVAL, "sgmm_group_create: scale is not finite");
    dlm_sgmm_group* h = new (std::nothrow) dlm_sgmm_group();
    if (!h) return fail(DLM_ENOMEM, "sgmm_group_create: host allocation failed");
    h->h_descs.resize(n);
    int64_t cb = 0, ks = 0, dmax = 0, dimax = 0;
    for (int i = 0; i < n; ++i) {
        const int rc = check_problem(probs[i], dtype, i);
        if (rc != DLM_OK) {
            delete h;
            return rc;
        }
        SgDesc& d = h->h_descs[i];
        d = SgDesc{};
        d.x = probs[i].x;
        d.A = probs[i].A;
        d.B = probs[i].B;
        d.y = probs[i].y;
        d.d_in = (int32_t)probs[i].d_in;
        d.d_out = (int32_t)probs[i].d_out;
        d.n_cb = (int32_t)((probs[i].d_out + kSgmmExpandCols - 1) / kSgmmExpandCols);
        d.unit0 = cb;
        cb += d.n_cb;
        d.n_ks = (int32_t)((probs[i].d_in + kSgmmKSlice - 1) / kSgmmKSlice);
        d.ks0 = ks;
        ks += d.n_ks;
        if (probs[i].d_out > dmax) dmax = probs[i].d_out;
        if (probs[i].d_in > dimax) dimax = probs[i].d_in;
        if (d.n_ks + d.n_cb > h->w_max) h->w_max = d.n_ks + d.n_cb;
    }
    h->n = n;
    h->E = E;
    h->r = r;
    h->scale = scale;
    h->dtype = dtype;
    h->total_cb = cb;
    h->total_ks = ks;
    h->d_out_max = dmax;
    h->d_in_max = dimax;
    hipError_t e = hipSuccess;
    if (dtype == DLM_BF16) {
        // one packed copy per distinct (A, d_in); problems sharing a bank share it
        std::map<std::pair<const void*, int64_t>, void*> seen;
        for (int i = 0; i < n && e == hipSuccess; ++i) {
            SgDesc& d = h->h_descs[i];
            const auto key = std::make_pair(d.A, (int64_t)d.d_in);
            auto it = seen.find(key);
            if (it == seen.end()) {
                void* ap = nullptr;
                e = hipMalloc(&ap, (size_t)E * r * d.d_in * 2);
                if (e != hipSuccess) break;
                h->packs.push_back({d.A, ap, d.d_in});
                e = launch_sgmm_pack_a(d.A, ap, E, r, d.d_in, nullptr);
                it = seen.emplace(key, ap).first;
            }
            d.Ap = it->second;
        }
        if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
    }
    // one device block: the descriptors, then a copy of the owning problem's
    // descriptor for every K slice and every expand column group (a work item
    // reads its problem with one load, not an owner index and then the table)
    const size_t desc_bytes = (sizeof(SgDesc) * n + 255) & ~(size_t)255;
    const size_t ks_bytes = (sizeof(SgDesc) * (size_t)ks + 255) & ~(size_t)255;
    std::vector<char> blob(desc_bytes + ks_bytes + sizeof(SgDesc) * (size_t)cb);
    std::memcpy(blob.data(), h->h_descs.data(), sizeof(SgDesc) * n);
    SgDesc* ks_desc = (SgDesc*)(blob.data() + desc_bytes);
    SgDesc* cb_desc = (SgDesc*)(blob.data() + desc_bytes + ks_bytes);
    for (int i = 0; i < n; ++i) {
        const SgDesc& d = h->h_descs[i];
        for (int k = 0; k < d.n_ks; ++k) ks_desc[d.ks0 + k] = d;
        for (int k = 0; k < d.n_cb; ++k) cb_desc[d.unit0 + k] = d;
    }
    if (e == hipSuccess) e = hipMalloc((void**)&h->d_descs, blob.size());
    if (e == hipSuccess) e = hipMemcpy(h->d_descs, blob.data(), blob.size(), hipMemcpyHostToDevice);
    if (e != hipSuccess) {
        if (h->d_descs) (void)hipFree(h->d_descs);
        for (auto& pk : h->packs) (void)hipFree(pk.Ap);
        delete h;
        return hip_fail(e, "sgmm_group_create");
    }
    h->d_ks_desc = (const SgDesc*)((const char*)h->d_descs + desc_bytes);
    h->d_cb_desc = (const SgDesc*)((const char*)h->d_descs + desc_bytes + ks_bytes);
    *out = h;
    return ok();
}

int dlm_sgmm_group_destroy(dlm_sgmm_group* h) {
    if (!h) return fail(DLM_EINVAL, "sgmm_group_destroy: null handle");
    hipError_t e = hipDeviceSynchronize();
    if (h->d_descs) (void)hipFree(h->d_descs);
    for (auto& pk : h->packs) (void)hipFree(pk.Ap);
    delete h;
    if (e != hipSuccess) return hip_fail(e, "sgmm_group_destroy");
    return ok();
}

int dlm_sgmm_group_repack(dlm_sgmm_group* h, void* stream) {
    if (!h) return fail(DLM_EINVAL, "sgmm_group_repack: null handle");
    for (auto& pk : h->packs) {
        const hipError_t e = launch_sgmm_pack_a(pk.A, pk.Ap, h->E, h->r, pk.d_in, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "sgmm_group_repack");
    }
    return ok();
}

int dlm_sgmm_group_run(dlm_sgmm_group* h, const int32_t* idx, const float* g, int64_t T,
                       void* workspace, size_t ws_bytes, void* stream) {
    if (!h) return fail(DLM_EINVAL, "sgmm_group_run: null handle");
    if (T < 0 || T > ((int64_t)1 << 30)) return fail(DLM_ESHAPE, "sgmm_group_run: T=%lld", (long long)T);
    if (T == 0) return ok();
    if (!idx || !g) return fail(DLM_EINVAL, "sgmm_group_run: idx or g is null");
    const size_t es = esize(h->dtype);
    const SgLayout L = sgmm_layout(T, h->d_in_max, h->E, h->r, h->n);
    const int rc = check_ws(workspace, ws_bytes, L);
    if (rc != DLM_OK) return rc;
    {
        // every problem's ranges, the sets and the workspace: a written one (y,
        // workspace) may overlap nothing else.  The problems' extents grow with
        // T, so a row count up to one already checked needs only the per-call
        // pointers (sets, workspace) checked again.
        std::vector<Span> v;
        const int64_t Tc = T > h->checked_T ? T : h->checked_T;
        for (int i = 0; i < h->n; ++i) {
            const SgDesc& d = h->h_descs[i];
            v.push_back(span(d.x, (size_t)Tc * d.d_in * es, false, "problem x", i));
            v.push_back(span(d.y, (size_t)Tc * d.d_out * es, true, "problem y", i));
            v.push_back(span(d.A, (size_t)h->E * h->r * d.d_in * es, false, "problem A", i));
            v.push_back(span(d.B, (size_t)h->E * d.d_out * h->r * es, false, "problem B", i));
        }
        if (T > h->checked_T) {
            Span a, b;
            if (write_conflict(v, &a, &b)) return conflict_fail("sgmm_group_run", a, b);
            h->checked_T = T;
        }
        const Span call[3] = {span(idx, (size_t)T * 8, false, "idx", 0), span(g, (size_t)T * 8, false, "g", 0),
                              span(workspace, ws_bytes, true, "workspace", 0)};
        for (const Span& c : call)
            for (const Span& q : v)
                if (c.hi > q.lo && q.hi > c.lo && (c.write || q.write)) return conflict_fail("sgmm_group_run", c, q);
        if (overlap(workspace, ws_bytes, idx, (size_t)T * 8) || overlap(workspace, ws_bytes, g, (size_t)T * 8))
            return fail(DLM_EINVAL, "sgmm_group_run: the workspace overlaps the sets");
    }
    return run_sgmm(h->d_descs, h->d_ks_desc, h->d_cb_desc, h->h_descs[0], h->n, h->total_cb, h->total_ks, h->d_out_max,
                    h->w_max, idx, g, T, h->E,
                    h->r, h->scale, h->dtype, h->packs.empty() ? 0 : 1, workspace, L, (hipStream_t)stream);
}

int dlm_sgmm_status(void* workspace, int32_t* code, void* stream) {
    if (!workspace || !code) return fail(DLM_EINVAL, "sgmm_status: null argument");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    int32_t v = 0;
    if (e == hipSuccess) e = hipMemcpy(&v, (char*)workspace + SG_ERR * 4, sizeof v, hipMemcpyDeviceToHost);
    if (e == hipSuccess && v != 0) e = hipMemset((char*)workspace + SG_ERR * 4, 0, sizeof v);
    if (e != hipSuccess) return hip_fail(e, "sgmm_status");
    *code = v ? DLM_EDEVICE : DLM_OK;
    return ok();
}

int dlm_sgmm_launches(int64_t T, int64_t d_in_max, int32_t r, int32_t n_problems, int32_t dtype) {
    if (T < 0 || d_in_max < 1 || r < 1 || r > DLM_MAX_RANK || n_problems < 1 ||
        (dtype != DLM_F32 && dtype != DLM_BF16)) {
        fail(DLM_EINVAL, "sgmm_launches: T < 0, d_in_max < 1, r outside [1, DLM_MAX_RANK], n_problems < 1 or unknown dtype");
        return -1;
    }
    if (T == 0) return 0;
    if (dtype == DLM_BF16 && T <= kSgmmSmallT) return n_problems == 1 ? 1 : 2;
    const int seg = T > kSgmmSegFewRows ? 2 : 1;
    if (dtype == DLM_F32) return seg + 2;
    const int vsum = d_in_max > kSgmmKSlice && r > kSgmmFoldRank ? 1 : 0;
    const bool fold = (r + 15) / 16 * 16 <= kSgmmFoldRank;
    const bool fused_ks = (d_in_max + kSgmmKSlice - 1) / kSgmmKSlice <= kSgmmFusedMaxKs;
    const bool fused_pairs = (int64_t)n_problems * ((T + 31) / 32) >= kSgmmFusedMinPairs;
    if (fold && fused_ks && fused_pairs && kSgmmFused > 0 && (kSgmmFused > 1 || T > kSgmmInlineRows))
        return seg + 1;  // one launch after the segmentation
    if (T <= kSgmmInlineRows && !vsum) return 2;  // the rows ordered inside the shrink and expand
    return seg + 2 + vsum;
}

}  // extern "C"
