// SGMM: batched unmerged adapters for rows carrying different expert sets,
//     y[t] <- round( y[t] + sum_k s*g[t][k] * B_{e_k} (A_{e_k} x[t]) ).
// The AdaFuse digest (section 2-na) names its core kernel SGMM, "segmented
// gather matrix multiplication"; this is the batched form of the same adapters.
//
// Launches:
//   segment  (one workgroup per 1024 rows; a count launch first when there
//            are several) every row gets the key of its unordered expert
//            pair; a stable counting sort lists the rows by key (perm, with
//            each position's pair and gates beside it), so rows sharing
//            experts sit next to each other.  The sorted list is cut into
//            32-row tiles; the later kernels take each tile's expert union
//            from its positions' pairs.  Rows with two empty slots are left
//            out.  The same segmentation serves every problem of a grouped
//            call (one routing decision per token for all layers).
//   shrink   per (problem, 2048-wide K slice, live tile): the slice's partial
//            v = x_rows A_U^T for the tile's experts U, bf16 MFMA 32x32x16 with
//            M = tile rows (gathered through perm, staged in LDS 512 columns at
//            a time), N = (expert, rank); each row keeps the fp32 partial v of
//            its own two slots.
//   sum      (ranks above 64, problems with d_in > 2048) the slices' partials
//            added in slice order.
//   expand   per (problem, 1024 output columns, live tile): y_rows += u B_U^T with
//            u = s*g*v per (row, expert, rank); up to rank 64 it first adds
//            the K slices' partials of its tile in slice order into LDS (the
//            sum launch's order, so the result is the same bit for bit).  u
//            stays fp32-accurate by
//            entering the MFMA as two bf16 terms (hi + lo); B slices are
//            k-contiguous and load straight into operand registers; lane l
//            ends with 16 consecutive outputs of one row (two 128-bit y
//            accesses), y is rounded to bf16 once.
// A tile whose rows share one pair contracts over 2r (x2 for hi/lo); a tile
// mixing many pairs contracts over every expert it touches, so skewed prefill
// batches get segment-sized work and small mixed decode batches read each
// expert's A and B once per tile instead of once per pair.
#include "gfx950.hpp"
#include "internal.hpp"
#include "sgmm.hpp"

namespace dlm {

static size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

SgLayout sgmm_layout(int64_t T, int64_t d_in_max, int E, int r, int n_prob) {
    SgLayout L;
    L.T = T;
    L.T_pad = ((T > 0 ? T : 1) + 31) / 32 * 32;
    L.tiles_max = L.T_pad / 32;
    L.r_pad = (r + 15) / 16 * 16;
    L.max_ks = (int)((d_in_max + kSgmmKSlice - 1) / kSgmmKSlice);
    size_t o = 0;
    L.hdr = o;   o += 256;
    L.perm = o;  o += a256((size_t)L.T_pad * 4);
    L.epk = o;   o += a256((size_t)L.T_pad * 4);
    L.gpk = o;   o += a256((size_t)L.T_pad * 8);
    L.n_chunks = (L.T + kSgmmSegRows - 1) / kSgmmSegRows;
    L.hist = o;  o += a256((size_t)L.n_chunks * (E + 1) * (E + 1) * 4);
    L.cerr = o;  o += a256((size_t)L.n_chunks * 4);
    L.v = o;     o += a256((size_t)n_prob * L.max_ks * L.T_pad * 2 * L.r_pad * 4);
    L.dep = o;   o += a256((size_t)n_prob * L.max_ks * L.tiles_max * 4);
    L.xcd = o;   o += a256((size_t)8 * kSgmmXcdWords * 4);
    L.total = o;
    return L;
}

namespace {

constexpr int kSegThreads = 1024;  // rows per segmentation chunk
// Up to this many chunks every placing workgroup counts all rows itself, so the
// segmentation is one launch; more chunks get a count launch first.
constexpr int kSegFewChunks = kSgmmSegFewRows / kSgmmSegRows;
constexpr int kSegWaves = kSegThreads / kWave;
constexpr int kMaxKeys = (32 + 1) * (32 + 1);

// ---- segment ---------------------------------------------------------------

// A row's set as loaded once: slots, gates and key.  key = the unordered pair
// (a <= b, -1 = empty slot) as (a + 1) (E + 1) + (b + 1); -1 for a row with
// two empty slots, a bad set or t >= T.
struct SegRow {
    int e0, e1, key;
    float g0, g1;
    bool bad;
};
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
// Raw set of row t.  The loads are not guarded (t past the end reads row
// T - 1, T >= 1, and is marked empty later), so several rows' loads can be in
// flight at once.
struct SegRaw {
    i32x2 e;
    f32x2 g;
};
__device__ __forceinline__ SegRaw seg_load(const int32_t* idx, const float* g, int64_t t, int64_t T) {
    const int64_t tc = t < T ? t : T - 1;
    return SegRaw{gld((const i32x2*)idx + tc), gld((const f32x2*)g + tc)};
}
__device__ __forceinline__ SegRow seg_row(const SegRaw& r, bool in, int E) {
    SegRow q;
    q.e0 = in ? r.e.x : -1;
    q.e1 = in ? r.e.y : -1;
    q.g0 = r.g.x;
    q.g1 = r.g.y;
    q.bad = q.e0 < -1 || q.e0 >= E || q.e1 < -1 || q.e1 >= E;
    if (q.e0 >= 0 && !__builtin_isfinite(q.g0)) q.bad = true;
    if (q.e1 >= 0 && !__builtin_isfinite(q.g1)) q.bad = true;
    const int a = q.e0 < q.e1 ? q.e0 : q.e1, b = q.e0 < q.e1 ? q.e1 : q.e0;
    q.key = (!q.bad && b >= 0) ? (a + 1) * (E + 1) + (b + 1) : -1;
    return q;
}

// Lanes of the wave whose key equals this lane's (keys in [0, 2^nbits); a
// negative key matches nothing): one ballot per key bit.
__device__ __forceinline__ uint64_t wave_match(int k, int nbits) {
    uint64_t same = __ballot(k >= 0);
    for (int b = 0; b < nbits; ++b) {
        const uint64_t set = __ballot((k >> b) & 1);
        same &= ((k >> b) & 1) ? set : ~set;
    }
    return k >= 0 ? same : 0ull;
}

// Exclusive scan over the workgroup (one value per thread, thread order).
__device__ __forceinline__ int block_exscan(int v, int* s_tot, int& total) {
    const int lane = lane_id(), w = wave_id();
    int inc = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int y = __shfl_up(inc, o, kWave);
        if (lane >= o) inc += y;
    }
    if (lane == kWave - 1) s_tot[w] = inc;
    __syncthreads();
    int before = 0;
    total = 0;
    for (int i = 0; i < kSegWaves; ++i) {
        const int x = s_tot[i];
        before += i < w ? x : 0;
        total += x;
    }
    __syncthreads();
    return before + inc - v;
}

// Work ranges of the one-launch shrink + expand (one workgroup, all threads;
// run by the segmentation once the live tile count nt is known).  The
// (problem, tile) pairs, problem-major, are split into 8 contiguous ranges of
// about equal weight, one per XCD, a pair weighing its problem's K slices +
// column groups (its shrink + expand items): the pair whose weight interval
// holds x/8 of the total starts XCD x's range.  Per XCD it writes
//   [0] p_a  [1] t_a  [2] p_b  [3] t_b     first pair, last problem and its tiles
//   [4] shrink items of p_a  [5] of the problems between  [6] all its shrink items
//   [7] ks0(p_a)  [8] ks0(p_a + 1)  [9] ks0(p_b)
//   [10] expand items of p_a  [11] of the problems between  [12] all its expand items
//   [13] unit0(p_a)  [14] unit0(p_a + 1)  [15] unit0(p_b)
// and clears the shrink counts of every (problem, tile).
__device__ void sgmm_fused_ranges(char* ws, const SgLayout& L, const SgDesc* __restrict__ descs,
                                  const SgDesc& single, int32_t n_prob, int64_t total_ks, int64_t total_cb,
                                  int64_t nt) {
    int32_t* dep = (int32_t*)(ws + L.dep);
    int32_t* tab = (int32_t*)(ws + L.xcd);
    const int tid = threadIdx.x;
    for (int64_t i = tid; i < total_ks * L.tiles_max; i += kSegThreads) dep[i] = 0;
    __shared__ int64_t s_qb[9];
    const int64_t Wt = (total_ks + total_cb) * nt;
    if (tid < 9) s_qb[tid] = (int64_t)n_prob * nt;
    if (tid == 0) s_qb[0] = 0;
    __syncthreads();
    for (int p = tid; p < n_prob; p += kSegThreads) {
        const SgDesc& Dp = descs ? descs[p] : single;
        const int64_t w = Dp.n_ks + Dp.n_cb, lo = (Dp.ks0 + Dp.unit0) * nt, hi = lo + w * nt;
        for (int x = 1; x < 8; ++x) {
            const int64_t sx = x * Wt / 8;
            if (sx >= lo && sx < hi) s_qb[x] = (int64_t)p * nt + (sx - lo + w - 1) / w;
        }
    }
    __syncthreads();
    if (tid < 8) {
        int32_t e[kSgmmXcdWords] = {};
        const int64_t qa = s_qb[tid], qb = s_qb[tid + 1];
        if (qb > qa) {
            const int pa = (int)(qa / nt), ta = (int)(qa % nt);
            const int pb = (int)((qb - 1) / nt), tb = (int)((qb - 1) % nt) + 1;
            const SgDesc& Da = descs ? descs[pa] : single;
            const SgDesc& Db = descs ? descs[pb] : single;
            const int cnt_a = (pa == pb ? tb : (int)nt) - ta;
            e[0] = pa;
            e[1] = ta;
            e[2] = pb;
            e[3] = tb;
            e[4] = Da.n_ks * cnt_a;
            e[7] = (int32_t)Da.ks0;
            e[10] = Da.n_cb * cnt_a;
            e[13] = (int32_t)Da.unit0;
            e[6] = e[4];
            e[12] = e[10];
            if (pb > pa) {
                const SgDesc& Da1 = descs ? descs[pa + 1] : single;
                e[5] = (int32_t)((Db.ks0 - Da1.ks0) * nt);
                e[8] = (int32_t)Da1.ks0;
                e[9] = (int32_t)Db.ks0;
                e[6] = e[4] + e[5] + Db.n_ks * tb;
                e[11] = (int32_t)((Db.unit0 - Da1.unit0) * nt);
                e[14] = (int32_t)Da1.unit0;
                e[15] = (int32_t)Db.unit0;
                e[12] = e[10] + e[11] + Db.n_cb * tb;
            }
        }
        for (int k = 0; k < kSgmmXcdWords; ++k) tab[tid * kSgmmXcdWords + k] = e[k];
    }
}

// The segmentation is a stable counting sort of the rows by key, in chunks of
// kSegThreads rows (one workgroup each):
//   count  (only above kSegFewChunks chunks) each chunk's key counts (LDS
//          atomics) and whether it holds a bad set;
//   place  each workgroup adds up, per key, every chunk's count (the key's
//          total) and the earlier chunks' counts; an exclusive scan of the
//          totals over the keys gives each key's first position.  A row's
//          position = its key's first position + rows of that key in earlier
//          chunks + in earlier waves of its chunk + earlier lanes of its wave
//          with the same key (a lane's same-key mask is one ballot per key bit).
//          Up to kSegFewChunks chunks every workgroup counts all rows here
//          instead, so the batch needs one launch.
// Each position gets its row, pair and gates, so the later kernels read a
// tile's metadata in one round of independent loads; positions past the live
// rows get row -1.  The first workgroup writes the header.
__global__ __launch_bounds__(kSegThreads) void sgmm_seg_count(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ g, int64_t T, int E,
                                                              char* ws, SgLayout L) {
    int32_t* hist = (int32_t*)(ws + L.hist);
    int32_t* cerr = (int32_t*)(ws + L.cerr);
    __shared__ int s_cnt[kMaxKeys];
    __shared__ int s_err;
    const int tid = threadIdx.x;
    const int nk = (E + 1) * (E + 1);
    const int64_t chunk = blockIdx.x;
    const int64_t t = chunk * kSegThreads + tid;
    const SegRaw raw = seg_load(idx, g, t, T);
    if (tid == 0) s_err = 0;
    for (int k = tid; k < nk; k += kSegThreads) s_cnt[k] = 0;
    __syncthreads();
    const SegRow q = seg_row(raw, t < T, E);
    if (q.bad) s_err = 1;
    if (q.key >= 0) atomicAdd(&s_cnt[q.key], 1);
    __syncthreads();
    for (int k = tid; k < nk; k += kSegThreads) hist[chunk * nk + k] = s_cnt[k];
    if (tid == 0) cerr[chunk] = s_err;
}

__global__ __launch_bounds__(kSegThreads) void sgmm_seg_place(const int32_t* __restrict__ idx,
                                                              const float* __restrict__ g, int64_t T, int E,
                                                              char* ws, SgLayout L, int32_t* status_out,
                                                              const SgDesc* __restrict__ descs, SgDesc single,
                                                              int32_t n_prob, int64_t total_ks, int64_t total_cb,
                                                              int32_t fused) {
    int32_t* hdr = (int32_t*)(ws + L.hdr);
    int32_t* perm = (int32_t*)(ws + L.perm);
    uint32_t* epk = (uint32_t*)(ws + L.epk);
    float* gpk = (float*)(ws + L.gpk);
    const int32_t* hist = (const int32_t*)(ws + L.hist);
    const int32_t* cerr = (const int32_t*)(ws + L.cerr);
    __shared__ int s_err;
    __shared__ int s_tot[kMaxKeys];    // rows of each key over all chunks
    __shared__ int s_base[kMaxKeys];   // the key's first position, then this chunk's first
    __shared__ uint16_t s_wc[kSegWaves][kMaxKeys];  // per-wave counts, then their prefix over waves
    __shared__ int s_sum[kSegWaves];
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int nk = (E + 1) * (E + 1);
    const int nbits = 32 - __builtin_clz((unsigned)(nk - 1));
    const int64_t chunk = blockIdx.x, n_chunks = gridDim.x;
    const int64_t t = chunk * kSegThreads + tid;
    const SegRaw raw = seg_load(idx, g, t, T);  // first needed when the row is placed
    if (tid == 0) s_err = 0;
    for (int q = tid; q < kSegWaves * nk; q += kSegThreads) s_wc[q / nk][q % nk] = 0;
    if (n_chunks == 1) {
        for (int k = tid; k < nk; k += kSegThreads) s_tot[k] = 0;
        __syncthreads();
        const SegRow q = seg_row(raw, t < T, E);
        if (q.bad) s_err = 1;
        if (q.key >= 0) atomicAdd(&s_tot[q.key], 1);
        for (int k = tid; k < nk; k += kSegThreads) s_base[k] = 0;
    } else if (n_chunks <= kSegFewChunks) {
        // every chunk's rows counted here: the keys' totals and the earlier
        // chunks' share, one LDS atomic per distinct key of a wave; all the
        // chunks' sets are loaded before the first is counted
        SegRaw rr[kSegFewChunks];
#pragma unroll
        for (int c = 0; c < kSegFewChunks; ++c)
            if (c < n_chunks && c != chunk) rr[c] = seg_load(idx, g, (int64_t)c * kSegThreads + tid, T);
        for (int k = tid; k < nk; k += kSegThreads) {
            s_tot[k] = 0;
            s_base[k] = 0;
        }
        __syncthreads();
#pragma unroll
        for (int c = 0; c < kSegFewChunks; ++c) {
            if (c < n_chunks) {
                const int64_t tc = (int64_t)c * kSegThreads + tid;
                const SegRow q = seg_row(c == chunk ? raw : rr[c], tc < T, E);
                if (q.bad) s_err = 1;
                const uint64_t same = wave_match(q.key, nbits);
                if (same && (same & ((1ull << lane) - 1ull)) == 0) {
                    const int n = (int)__popcll(same);
                    atomicAdd(&s_tot[q.key], n);
                    if (c < chunk) atomicAdd(&s_base[q.key], n);
                }
            }
        }
    } else {
        // every chunk's counts: the key's total and the earlier chunks' share
        for (int k = tid; k < nk; k += kSegThreads) {
            int tot = 0, bef = 0;
            for (int64_t c = 0; c < n_chunks; ++c) {
                const int v = gld(hist + c * nk + k);
                tot += v;
                bef += c < chunk ? v : 0;
            }
            s_tot[k] = tot;
            s_base[k] = bef;
        }
        int e = 0;
        for (int64_t c = tid; c < n_chunks; c += kSegThreads) e |= gld(cerr + c);
        if (e) s_err = 1;
    }
    __syncthreads();
    const int err = s_err;

    // exclusive scan of the totals in key order (each thread owns a run of keys)
    constexpr int kPer = (kMaxKeys + kSegThreads - 1) / kSegThreads;
    int cnt[kPer], run = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int k = tid * kPer + j;
        cnt[j] = k < nk ? s_tot[k] : 0;
        run += cnt[j];
    }
    int n_pos;
    int start = block_exscan(run, s_sum, n_pos);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int k = tid * kPer + j;
        if (k < nk) s_base[k] += start;
        start += cnt[j];
    }
    if (err) n_pos = 0;

    if (!err) {
        const SegRow cur = seg_row(raw, t < T, E);
        const int k = cur.key;
        // stable rank within the wave and the wave's count of each key
        const uint64_t same = wave_match(k, nbits);
        const int rk = (int)__popcll(same & ((1ull << lane) - 1ull));
        if (same && rk == 0) s_wc[w][k] = (uint16_t)__popcll(same);
        __syncthreads();
        // rows of each key in earlier waves of the chunk, in wave order
        for (int kk = tid; kk < nk; kk += kSegThreads) {
            int acc = 0;
            for (int i = 0; i < kSegWaves; ++i) {
                const int c = s_wc[i][kk];
                s_wc[i][kk] = (uint16_t)acc;
                acc += c;
            }
        }
        __syncthreads();
        if (k >= 0) {
            const int64_t p = (int64_t)s_base[k] + s_wc[w][k] + rk;
            perm[p] = (int32_t)t;
            epk[p] = ((uint32_t)cur.e0 & 0xffffu) | ((uint32_t)cur.e1 << 16);
            gpk[2 * p] = cur.e0 >= 0 ? cur.g0 : 0.f;
            gpk[2 * p + 1] = cur.e1 >= 0 ? cur.g1 : 0.f;
        }
    }
    // positions past the live rows, split over the workgroups
    for (int64_t p = n_pos + chunk * kSegThreads + tid; p < L.T_pad; p += n_chunks * kSegThreads) {
        perm[p] = -1;
        epk[p] = 0xffffffffu;
        gpk[2 * p] = 0.f;
        gpk[2 * p + 1] = 0.f;
    }
    if (chunk == 0 && tid == 0) {
        hdr[SG_ERR] = err;
        hdr[SG_NPOS] = n_pos;
        hdr[SG_NTILES] = (n_pos + 31) / 32;
        if (status_out) *status_out = err;
    }
    if (fused && chunk == 0) sgmm_fused_ranges(ws, L, descs, single, n_prob, total_ks, total_cb,
                                               err ? 0 : (n_pos + 31) / 32);
}

// With at most kWave rows the shrink and expand workgroups order the rows
// themselves, in the segmentation's order: lane i of the calling wave holds
// row i, and a live row's position is the number of live rows with a smaller
// key (one ballot per key bit, from the top: at a bit where this key has a 1,
// the live rows that agree with it above that bit and have a 0 there are
// smaller), plus the live rows with the same key and a smaller index.  Each
// live lane writes its position of s_perm / s_ep (and s_g if given): row, pair
// and gates as the segmentation writes them; positions past the live rows get
// row -1.  Returns the live-row count, or -1 if any row's set is bad (nothing
// may then be written).  One wave, every lane; the caller synchronises before
// the arrays are read.
__device__ __forceinline__ int inline_order(const SgmmArgs& a, int32_t* s_perm, uint32_t* s_ep, f32x2* s_g) {
    const int lane = lane_id();
    const SegRow q = seg_row(seg_load(a.idx, a.g, lane, a.T), lane < a.T, a.E);
    const bool bad = __ballot(q.bad) != 0ull;
    const int key = q.key;
    const int nk = (a.E + 1) * (a.E + 1);
    const int nbits = 32 - __builtin_clz((unsigned)(nk - 1));
    const uint64_t live = __ballot(key >= 0);
    uint64_t eq = live;  // live lanes whose key agrees with this one on the bits seen so far
    int less = 0;
    for (int bit = nbits - 1; bit >= 0; --bit) {
        const uint64_t ones = __ballot(key >= 0 && ((key >> bit) & 1));
        const bool one = key >= 0 && ((key >> bit) & 1);
        if (one) less += (int)__popcll(eq & ~ones);
        eq &= one ? ones : (live & ~ones);
    }
    const int n_pos = (int)__popcll(live);
    if (key >= 0) {
        const int pos = less + (int)__popcll(eq & ((1ull << lane) - 1ull));
        s_perm[pos] = lane;
        s_ep[pos] = ((uint32_t)q.e0 & 0xffffu) | ((uint32_t)q.e1 << 16);
        if (s_g) s_g[pos] = f32x2{q.e0 >= 0 ? q.g0 : 0.f, q.e1 >= 0 ? q.g1 : 0.f};
    }
    if (lane >= n_pos) {
        s_perm[lane] = -1;
        s_ep[lane] = 0xffffffffu;
        if (s_g) s_g[lane] = f32x2{0.f, 0.f};
    }
    return bad ? -1 : n_pos;
}

// ---- helpers ---------------------------------------------------------------

// Experts set in a tile mask, ascending.
__device__ __forceinline__ int mask_list(uint32_t m, int* out) {
    int n = 0;
    while (m) {
        const int e = __ffs(m) - 1;
        out[n++] = e;
        m &= m - 1;
    }
    return n;
}

// ---- shrink (bf16, MFMA) -----------------------------------------------------

// Rows of one shrink work item (one tile).
constexpr int kXRows = 32;
// K is staged through LDS in kShrinkStep-wide steps: 64-wide K chunks of one
// step, and 16-byte chunks of one x row of a step.  A work item covers one
// kSgmmKSlice-wide slice, i.e. kShrinkSteps steps, with its accumulators held
// in registers across them.
constexpr int kShrinkStep = 512;
constexpr int kShrinkSteps = kSgmmKSlice / kShrinkStep;
static_assert(kSgmmKSlice % kShrinkStep == 0, "a slice is a whole number of steps");
constexpr int kKC = kShrinkStep / 64;
constexpr int kXC = kShrinkStep / 8;
// A chunks in flight per wave in the shrink's K loop.  The shrink runs at 4
// waves per SIMD (3 for ranks 17..32, which would spill at 4): several
// workgroups per CU, each with a 32 KB x step.
constexpr int kShrinkRing = 2;
static_assert(kKC >= kShrinkRing && kKC % kShrinkRing == 0, "a step is a whole number of ring steps");
static_assert(256 % kXC == 0 && kXRows % (256 / kXC) == 0, "x step load shape");
// x step in LDS: kXRows rows of kShrinkStep bf16; the 16-byte chunk c of row m
// is stored at chunk c ^ (m & 15), so the MFMA-layout reads (16 rows, one chunk)
// and the row-contiguous writes both touch 16 distinct bank groups.
__device__ __forceinline__ int x_off(int row, int c) { return row * kShrinkStep + ((c ^ (row & 15)) << 3); }
// per-wave 32x64 bf16 scratch of the expand: rows of eight 16-byte chunks, chunk XOR (row & 7)
__device__ __forceinline__ int y_off(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// One work item = (problem, K slice, tile), the tiles fastest so the work
// items that share a slice of A run next to each other on one XCD.  The N
// blocks (32 columns of (expert, rank) each, over the union of the tile's
// experts) are spread over the four waves: with four or more blocks each wave
// takes whole blocks (in rounds of four), with fewer the waves of one block
// split each step's chunks and their sums are added in a fixed order at the
// end.  Per step the four waves read the tile's x rows of the step,
// row-contiguous (each x byte once per round), into LDS, and the next step's
// x is in flight while the MFMAs run; the A rows of a block stream from L2
// kShrinkRing chunks ahead of the MFMAs.  Each row's two slots get the slice's
// partial v; a later pass adds the slices up when there are several.  Loads
// are never guarded: a padding row or (expert, rank) column reads an in-bounds
// dummy row whose products reach only accumulator entries that are never
// stored, and k past d_in reads a clamped address whose value is replaced by 0.
// i_perm / i_ep: the rows' order computed in the workgroup (inline_order), or
// nullptr to read the segmentation's from the workspace.
// This wave's XCD (HW_REG_XCC_ID, bits 3:0).
__device__ __forceinline__ int xcc_id() { return (int)(__builtin_amdgcn_s_getreg((3 << 11) | 20) & 15u); }

// LDS of one shrink work item.
struct ShrinkLds {
    __attribute__((aligned(16))) uint16_t x[kXRows * kShrinkStep];
    int U[32];
    int nU;
    int row[kXRows];
    // per row: slot 0's expert + 1 (bits 0-5), slot 1's + 1 (bits 6-11), bit 12
    // set for a padding position (no row)
    __attribute__((aligned(16))) uint16_t slots[kXRows];
};

// dep: the one-launch form's counts of finished shrink items per (problem,
// tile), or nullptr.  With it the item, once its v stores are in L2, adds one
// (and its XCD id + 1 in the upper half-word) to its (problem, tile) count; the
// expand items of that pair wait for the problem's K-slice count.  Both run on
// the same XCD, so the count and v meet in that XCD's L2 (the vector L1 writes
// through).
template <int R16, bool PK>
__device__ __forceinline__ void shrink_item(const SgmmArgs& a, int64_t gks, int tile0, int n_tiles,
                                            const int32_t* i_perm, const uint32_t* i_ep, ShrinkLds& sm,
                                            int32_t* dep = nullptr) {
    constexpr int RPAD = R16 * 16;
    const SgDesc D = a.descs ? a.ks_desc[gks] : a.single;
    const int k0 = (int)(gks - D.ks0) * kSgmmKSlice;
    const int32_t* perm = (const int32_t*)(a.ws + a.L.perm);
    const uint32_t* epk = (const uint32_t*)(a.ws + a.L.epk);
    float* v = (float*)(a.ws + a.L.v) + gks * a.L.T_pad * 2 * RPAD;

    uint16_t* s_x = sm.x;
    int* s_U = sm.U;
    int& s_nU = sm.nU;
    int* s_row = sm.row;
    uint16_t* s_slots = sm.slots;
    const int tid = threadIdx.x;
    static_assert(kXRows <= kWave, "one wave reads the tile's rows");
    if (tid < kWave) {
        // the tile's rows and slots; their expert union from a wave OR
        uint32_t m = 0;
        if (tid < kXRows) {
            const bool in = tile0 < n_tiles;
            const int p = tile0 * 32 + tid;
            const int row = in ? (i_perm ? i_perm[p] : gld(perm + p)) : -1;
            const uint32_t ep = in ? (i_ep ? i_ep[p] : gld(epk + p)) : 0xffffffffu;
            const int e0 = (int16_t)(ep & 0xffffu), e1 = (int16_t)(ep >> 16);
            s_row[tid] = row;
            s_slots[tid] = (uint16_t)((e0 + 1) | ((e1 + 1) << 6) | (row < 0 ? 1 << 12 : 0));
            m = (e0 >= 0 ? 1u << e0 : 0u) | (e1 >= 0 ? 1u << e1 : 0u);
        }
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) m |= __shfl_xor(m, o, kWave);
        if (tid == 0) s_nU = mask_list(m, s_U);
    }
    __syncthreads();

    const int d_in = uniform(D.d_in), r = a.r;
    const uint16_t* __restrict__ x = (const uint16_t*)D.x;
    const uint16_t* __restrict__ A = (const uint16_t*)(PK ? D.Ap : D.A);
    // steps of this slice inside d_in (the same for every wave)
    const int n_steps = (d_in - k0 + kShrinkStep - 1) / kShrinkStep < kShrinkSteps
                            ? (d_in - k0 + kShrinkStep - 1) / kShrinkStep : kShrinkSteps;

    // x step: thread tid reads chunk tid % kXC of rows tid / kXC + kXR j
    constexpr int kXR = 256 / kXC;           // rows per load instruction
    constexpr int kXL = kXRows / kXR;        // load instructions per thread
    const int xc = tid % kXC, xr0 = tid / kXC;
    auto load_x = [&](u32x4 (&xv)[kXL], int kb) {
        const bool ok = kb + 8 * xc < d_in;
#pragma unroll
        for (int j = 0; j < kXL; ++j) {
            const int rr = s_row[xr0 + kXR * j];
            xv[j] = ld128_nt(x + (int64_t)(rr >= 0 ? rr : 0) * d_in + (ok ? kb + 8 * xc : 0));
        }
    };
    auto store_x = [&](const u32x4 (&xv)[kXL], int kb) {
        const bool ok = kb + 8 * xc < d_in;
#pragma unroll
        for (int j = 0; j < kXL; ++j)
            *(u32x4*)(s_x + x_off(xr0 + kXR * j, xc)) = ok ? xv[j] : u32x4{0u, 0u, 0u, 0u};
    };
    u32x4 xv[kXL];
    load_x(xv, k0);

    const int nU = uniform(s_nU);
    const int NB = (nU * RPAD + 31) / 32;
    const int G = NB < 4 ? NB : 4;  // blocks in flight
    const int P = 4 / G;            // waves per block (1 when G == 3)
    const int n_rounds = (NB + G - 1) / G;
    const int w = wave_id(), lane = lane_id();
    const int gw = w % G, kp = w / G;
    const int nmy = kKC / P;        // chunks per wave: chunk kp + P i

    // MFMA step s2 of chunk kc takes, in half-wave h, the 8-wide k group
    // kq = (kb + 64 kc) / 8 + 2 s2 + h: the two halves read adjacent groups, so
    // in the packed A layout one load covers contiguous runs of 32 bytes x rank.
    const int nq = d_in / 8;
    const int64_t qstride = PK ? 8 * r : 8;  // elements from group kq to kq + 1
    // A group past d_in loads a clamped address and is replaced by zeros where
    // the MFMA takes it: a select right after the load would wait for it.
    auto load_a = [&](u32x4 (&dst)[4], const uint16_t* abase, int kc, int kb, int h) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int kq = kb / 8 + 8 * kc + 2 * s2 + h;
            dst[s2] = ld128(abase + (kq < nq ? kq : nq - 1) * qstride);
        }
    };
    // first element of this lane's (expert, rank) row in A (row start) or in
    // the packed A (its 8 values of group 0)
    auto a_row = [&](int blk, int n, int& u, int& rho) {
        const int nn = blk * 32 + n;
        u = nn / RPAD;
        rho = nn % RPAD;
        const bool ok = u < nU && rho < r;
        const int64_t e = ok ? s_U[u] : 0, rr = ok ? rho : 0;
        return PK ? A + e * r * d_in + rr * 8 : A + (e * r + rr) * d_in;
    };
    auto mma = [&](const u32x4 (&ab)[4], int kc, int kb, int h, int n, f32x16& acc) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const bool in = kb / 8 + 8 * kc + 2 * s2 + h < nq;
            const u32x4 av = in ? ab[s2] : u32x4{0u, 0u, 0u, 0u};
            const u32x4 xo = *(const u32x4*)(s_x + x_off(n, 8 * kc + 2 * s2 + h));
            acc = mfma32(xo, av, acc);
        }
    };
    auto store_v = [&](const f32x16& acc, int u, int rho, int h) {
        if (u >= nU || rho >= r) return;
        const int e = s_U[u];
        // the slots of this lane's 16 rows (8j + 4h + [0,4)): four 8-byte LDS
        // reads issued together, not a dependent read before every store
        typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
        u32x2_t sl[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) sl[j] = *(const u32x2_t*)(s_slots + 8 * j + 4 * h);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 8 * (i >> 2) + 4 * h + (i & 3);
            const uint32_t s = (sl[i >> 2][(i & 3) >> 1] >> (16 * (i & 1))) & 0xffffu;
            if (s >> 12) continue;
            float* vp = v + ((int64_t)(tile0 * 32 + m) * 2) * RPAD + rho;
            if ((int)(s & 63u) - 1 == e) gst(vp, acc[i]);
            if ((int)((s >> 6) & 63u) - 1 == e) gst(vp + RPAD, acc[i]);
        }
    };
    u32x4 ab[kShrinkRing][4];
    // K loop of one block over this wave's chunks of one step, A kShrinkRing
    // chunks ahead (the first kShrinkRing are loaded before the step starts)
    auto run_block = [&](f32x16& acc, const uint16_t* arow, int kb, int h, int n) {
#pragma unroll 1
        for (int i = 0; i < nmy; i += kShrinkRing) {
#pragma unroll
            for (int j = 0; j < kShrinkRing; ++j) {
                if (i + j < nmy) {
                    mma(ab[j], kp + P * (i + j), kb, h, n, acc);
                    if (i + j + kShrinkRing < nmy) load_a(ab[j], arow, kp + P * (i + j + kShrinkRing), kb, h);
                }
            }
        }
    };

#pragma unroll 1
    for (int rd = 0; rd < n_rounds; ++rd) {
        // this wave's block of the round (waves past the blocks only stage x)
        const int blk = gw + rd * G;
        const bool mine = kp < P && blk < NB;
        f32x16 acc = f32x16{};
#pragma unroll 1
        for (int ss = 0; ss < n_steps; ++ss) {
            const int kb = k0 + ss * kShrinkStep;
            // the lane index is opaque to this loop: the addresses derived from
            // it are rebuilt per step instead of being held across steps
            int ln = lane;
            asm volatile("" : "+v"(ln));
            const int h = ln >> 5, n = ln & 31;
            int u, rho;
            const uint16_t* arow = a_row(mine ? blk : gw, n, u, rho);
            // this step's first A chunks are in flight while x lands in LDS
#pragma unroll
            for (int j = 0; j < kShrinkRing; ++j)
                if (mine && j < nmy) load_a(ab[j], arow, kp + P * j, kb, h);
            __syncthreads();  // the previous step's MFMAs are done with the LDS
            store_x(xv, kb);
            __syncthreads();
            // next x step (or the next round's first): one call site, so the
            // loads land in the same registers on every path
            const int kn = ss + 1 < n_steps ? kb + kShrinkStep : k0;
            if (ss + 1 < n_steps || rd + 1 < n_rounds) load_x(xv, kn);
            if (mine) run_block(acc, arow, kb, h, n);
        }
        // (opaque again: the 16 v addresses of store_v are built here, not
        // held across the rounds)
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int h = ln >> 5, n = ln & 31;
        int u, rho;
        (void)a_row(mine ? blk : gw, n, u, rho);
        if (P == 1) {
            if (mine) store_v(acc, u, rho, h);
            continue;
        }
        // one block per group of P waves (a single round): parts 1..P-1 go
        // through LDS (the x step is no longer read) and the part-0 wave adds
        // them in order
        __syncthreads();
        f32x4* red = (f32x4*)s_x;  // [wave][4][lane]
        static_assert(4 * 4 * kWave * 16 <= kXRows * kShrinkStep * 2, "reduction fits the x step");
        if (kp > 0) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[(w * 4 + q) * kWave + lane] = f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        }
        __syncthreads();
        if (kp == 0) {
            for (int p = 1; p < P; ++p) {
                const int wp = gw + p * G;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 o = red[(wp * 4 + q) * kWave + lane];
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[4 * q + c] += o[c];
                }
            }
            store_v(acc, u, rho, h);
        }
    }
    if (dep) {
        // every thread's v stores have reached L2 before the count moves
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (tid == 0)
            __hip_atomic_fetch_add(dep + D.ks0 * a.L.tiles_max + tile0, 1 + ((xcc_id() + 1) << 16), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
    }
}

// Work items are the live ones only: (problem, K slice, tile) over the tiles
// the segmentation filled (released rows are left out), numbered with the
// tile fastest and spread over the 8 XCDs.  The grid is sized for the largest
// batch the workspace holds (the live count is known on the device only);
// workgroups past the live items exit after one header load, and as the
// dispatcher starts workgroups in index order they come last.
template <int R16, bool PK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R16 == 2 ? 3 : 4)))
void sgmm_shrink_bf16(SgmmArgs a) {
    int32_t* hdr = (int32_t*)(a.ws + a.L.hdr);
    __shared__ int32_t s_iperm[kWave];
    __shared__ uint32_t s_iep[kWave];
    __shared__ int s_inpos;
    int n_tiles;
    if (a.inline_seg) {
        // this workgroup orders the rows itself; workgroup 0 publishes the
        // header and the status word as the segmentation launch would
        if (threadIdx.x < kWave) {
            const int np = inline_order(a, s_iperm, s_iep, nullptr);
            if (threadIdx.x == 0) {
                s_inpos = np;
                if (blockIdx.x == 0) {
                    gst(hdr + SG_ERR, np < 0 ? 1 : 0);
                    gst(hdr + SG_NPOS, np < 0 ? 0 : np);
                    gst(hdr + SG_NTILES, np < 0 ? 0 : (np + 31) / 32);
                    if (a.status_out) gst(a.status_out, np < 0 ? 1 : 0);
                }
            }
        }
        __syncthreads();
        const int np = s_inpos;
        if (np < 0) return;
        n_tiles = (np + 31) / 32;
    } else {
        n_tiles = uniform(gld(hdr + SG_NTILES));
        if (gld(hdr + SG_ERR)) return;
    }
    const int64_t n_live = a.total_ks * n_tiles, per = (n_live + 7) / 8;
    const int64_t bid = blockIdx.x, j = bid >> 3;
    if (j >= per) return;
    const int64_t t = (bid & 7) * per + j;
    if (t >= n_live) return;
    const int64_t gks = t / n_tiles;  // slice index over all problems
    __shared__ ShrinkLds sm;
    shrink_item<R16, PK>(a, gks, (int)(t - gks * n_tiles), n_tiles, a.inline_seg ? s_iperm : nullptr,
                         a.inline_seg ? s_iep : nullptr, sm);
}

// ---- expand (bf16, MFMA) -----------------------------------------------------

__device__ __forceinline__ int perm_col(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Columns of one expand work item: 4 waves x kEB blocks x 64 columns.
constexpr int kEB = 4;
constexpr int kECols = 4 * kEB * 64;
// Items per XCD run as half items at the end of an expand launch: about the
// expand workgroups resident on one XCD (32 CUs x 3).
constexpr int kExpandSplit = 96;
static_assert(kECols == kSgmmExpandCols, "expand column group");
// The row-side MFMA operands (u = s*g*v as hi + lo bf16, per (expert, 16-rank
// chunk) pair q and lane) are the same for the four waves of a work item: they
// are built once into LDS when the tile's union has at most kQLds pairs; larger
// unions rebuild them per column block in registers.
constexpr int kQLds = 16;
// Up to this many 16-rank chunks the expand adds the K slices of its tile's v
// itself (the tile's v block fits the y scratch); larger ranks get a K-slice
// sum launch between the shrink and the expand.
constexpr int kExpandFoldR16 = kSgmmFoldRank / 16;
static_assert(32 * 2 * 16 * kExpandFoldR16 * 4 <= 4 * 32 * 64 * 2, "v block fits the y scratch");
static_assert(32 * 2 * 16 * kExpandFoldR16 * 4 <= kQLds * 2 * kWave * 16, "v block fits the operand table");

// work item = (problem, kECols-column group cgg over all problems, tile) with
// the tile fastest: neighbouring work items (same XCD) reuse the same B column
// slices.
// i_perm / i_ep / i_g: the rows' order computed in the workgroup
// (inline_order), or nullptr to read the segmentation's from the workspace.
// LDS of one expand work item.
struct ExpandLds {
    int U[32];
    int nU;
    __attribute__((aligned(16))) uint16_t y[4][32 * 64];
    __attribute__((aligned(16))) u32x4 u[kQLds][2][kWave];
};

// Bounded wait of the one-launch form (about a second): past it the item sets
// the error word to 2 and goes on.
constexpr int kDepSpinMax = 1 << 20;

// dep: the one-launch form's shrink counts (see shrink_item), or nullptr.
template <int R16, bool RVEC>
__device__ __forceinline__ void expand_item(const SgmmArgs& a, int64_t cgg, int tile, int half,
                                            const int32_t* i_perm, const uint32_t* i_ep, const f32x2* i_g,
                                            ExpandLds& sm, const int32_t* dep = nullptr) {
    constexpr int RPAD = R16 * 16;
    constexpr bool FOLD = R16 <= kExpandFoldR16;
    const int32_t* perm = (const int32_t*)(a.ws + a.L.perm);
    const uint32_t* epk = (const uint32_t*)(a.ws + a.L.epk);
    const float* gpk = (const float*)(a.ws + a.L.gpk);
    const int w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const int lr = lane >> 3, lc = lane & 7;
    // every load whose address does not depend on another load goes out
    // first: the header words, the column group's problem descriptor, the tile's rows
    // (row-major lane map: instruction i holds row 8i + lr, chunk lc), slots,
    // gates and expert mask
    int yrow[4];
    uint32_t ep;
    float g0, g1;
    if (i_perm) {
#pragma unroll
        for (int i = 0; i < 4; ++i) yrow[i] = i_perm[tile * 32 + 8 * i + lr];
        ep = i_ep[tile * 32 + n];
        g0 = i_g[tile * 32 + n].x;
        g1 = i_g[tile * 32 + n].y;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) yrow[i] = gld(perm + tile * 32 + 8 * i + lr);
        ep = gld(epk + tile * 32 + n);
        g0 = gld(gpk + 2 * (tile * 32 + n));
        g1 = gld(gpk + 2 * (tile * 32 + n) + 1);
    }
    const SgDesc D = a.descs ? a.cb_desc[cgg] : a.single;
    const int cg = (int)(cgg - D.unit0);
    const float* v = (const float*)(a.ws + a.L.v) + D.ks0 * a.L.T_pad * 2 * RPAD;

    int* s_U = sm.U;
    int& s_nU = sm.nU;
    uint16_t (*s_y)[32 * 64] = sm.y;
    u32x4 (*s_u)[2][kWave] = sm.u;

    const int d_out = uniform(D.d_out), r = a.r;
    // this wave's first column and blocks: kEB blocks of the whole item, or
    // kEB / 2 of one of its halves (the same columns split in two items)
    const int eb = half < 0 ? kEB : kEB / 2;
    const int cw = cg * kECols + (half < 0 ? 0 : half * (kECols / 2)) + w * (eb * 64);
    const int nblk = cw >= d_out ? 0 : ((d_out - cw + 63) / 64 < eb ? (d_out - cw + 63) / 64 : eb);
    const uint16_t* __restrict__ B = (const uint16_t*)D.B;
    uint16_t* __restrict__ y = (uint16_t*)D.y;
    uint16_t* ys = s_y[w];
    auto load_y = [&](u32x4 (&yv)[4], int blk) {
        const int col = cw + blk * 64 + 8 * lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = yrow[i] >= 0 && col < d_out;
            yv[i] = ld128_nt(y + (ok ? (int64_t)yrow[i] * d_out + col : 0));
        }
    };
    u32x4 ycur[4], ynxt[4];
    if (nblk > 0) load_y(ycur, 0);
    if (w == 0) {
        // the tile's expert union: OR of its positions' pairs (lane n holds position n)
        const int f0 = (int16_t)(ep & 0xffffu), f1 = (int16_t)(ep >> 16);
        uint32_t m = (f0 >= 0 ? 1u << f0 : 0u) | (f1 >= 0 ? 1u << f1 : 0u);
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) m |= __shfl_xor(m, o, kWave);
        if (lane == 0) s_nU = mask_list(m, s_U);
    }
    if (dep && threadIdx.x == 0) {
        // the tile's v is complete once every K slice's shrink item has counted
        const int32_t* c = dep + D.ks0 * a.L.tiles_max + tile;
        const int need = D.n_ks;
        int cv = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        for (int spins = 0; (cv & 0xffff) < need;) {
            if (++spins > kDepSpinMax) {
                gst((int32_t*)(a.ws + a.L.hdr) + SG_ERR, 2);
                if (a.status_out) gst(a.status_out, 2);
                break;
            }
            __builtin_amdgcn_s_sleep(2);
            cv = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        if ((cv & 0xffff) >= need && (cv >> 16) != need * (xcc_id() + 1)) {
            gst((int32_t*)(a.ws + a.L.hdr) + SG_ERR, 3);
            if (a.status_out) gst(a.status_out, 3);
        }
    }
    __syncthreads();
    const int nU = uniform(s_nU);

    // this lane's tile row (MFMA N index n): its two slots and gates (a padding
    // position has two empty slots)
    const int e0 = (int16_t)(ep & 0xffffu), e1 = (int16_t)(ep >> 16);
    const float c0 = a.scale * g0;
    const float c1 = a.scale * g1;
    // v of this lane's row: the tile's summed copy in LDS (FOLD), else slice 0
    // of the workspace (already summed by the K-slice sum launch)
    const int nq = nU * R16;
    const bool shared_u = nq <= kQLds;
    float* s_v = shared_u ? (float*)&s_y[0][0] : (float*)&s_u[0][0][0];
    if constexpr (FOLD) {
        // the tile's v block (32 rows x 2 slots x RPAD floats, contiguous in
        // each slice) with the problem's K slices added in slice order; it
        // takes the y scratch while the shared operands are built, else the
        // operand table, which a union too large for the table leaves unused
        const int nks = uniform(D.n_ks);
        const int64_t stride = a.L.T_pad * 2 * RPAD;
        const float* vt = v + (int64_t)tile * 32 * 2 * RPAD + 4 * threadIdx.x;
        constexpr int KB = 8 / R16;  // slices in flight per round
        u32x4 acc[R16];
#pragma unroll
        for (int k = 0; k < R16; ++k) acc[k] = ld128(vt + 1024 * k);
        for (int ks = 1; ks < nks; ks += KB) {
            u32x4 p[KB][R16];
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int k = 0; k < R16; ++k)
                    if (ks + j < nks) p[j][k] = ld128(vt + (ks + j) * stride + 1024 * k);
#pragma unroll
            for (int j = 0; j < KB; ++j)
#pragma unroll
                for (int k = 0; k < R16; ++k)
                    if (ks + j < nks)
#pragma unroll
                        for (int c = 0; c < 4; ++c)
                            acc[k][c] = __float_as_uint(__uint_as_float(acc[k][c]) + __uint_as_float(p[j][k][c]));
        }
#pragma unroll
        for (int k = 0; k < R16; ++k) *(u32x4*)(s_v + 4 * threadIdx.x + 1024 * k) = acc[k];
        __syncthreads();
    }
    const float* v0 = FOLD ? s_v + n * 2 * RPAD : v + ((int64_t)(tile * 32 + n) * 2) * RPAD;
    const float* v1 = v0 + RPAD;
    // row-side operand of (expert U[q / R16], ranks 16(q % R16) + 8h + [0,8)):
    // u = s*g*v as hi + lo bf16 (v = the K slices' sum).  v of a slot that is not this expert, or of a
    // padding rank, is never written: it is selected away, not multiplied by 0.
    auto make_u = [&](int q, u32x4& bhi, u32x4& blo) {
        const int e = s_U[q / R16];
        const int rho0 = (q % R16) * 16 + 8 * h;
        const bool m0 = (e0 == e), m1 = (e1 == e);
        u32x4 p0, p1, q0, q1;
        if constexpr (FOLD) {
            p0 = *(const u32x4*)(v0 + rho0);
            p1 = *(const u32x4*)(v0 + rho0 + 4);
            q0 = *(const u32x4*)(v1 + rho0);
            q1 = *(const u32x4*)(v1 + rho0 + 4);
        } else {
            p0 = ld128(v0 + rho0);
            p1 = ld128(v0 + rho0 + 4);
            q0 = ld128(v1 + rho0);
            q1 = ld128(v1 + rho0 + 4);
        }
        float va[8], vb[8];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            va[c] = __uint_as_float(p0[c]);
            va[c + 4] = __uint_as_float(p1[c]);
            vb[c] = __uint_as_float(q0[c]);
            vb[c + 4] = __uint_as_float(q1[c]);
        }
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            float uv[2];
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int jj = 2 * j + k;
                const bool okr = rho0 + jj < r;
                const float a0 = (m0 && okr) ? va[jj] : 0.f;
                const float a1 = (m1 && okr) ? vb[jj] : 0.f;
                uv[k] = fmaf(c1, a1, c0 * a0);
            }
            hw[j] = pack2_bf16(uv[0], uv[1]);
            lw[j] = pack2_bf16(uv[0] - bf_lo(hw[j]), uv[1] - bf_hi(hw[j]));
        }
        bhi = u32x4{hw[0], hw[1], hw[2], hw[3]};
        blo = u32x4{lw[0], lw[1], lw[2], lw[3]};
    };
    // column-side operand: B[e][col][16(q % R16) + 8h .. +8]; padding columns
    // read column 0 and are never stored.  With r % 8 == 0 (RVEC) the load is
    // one unguarded 16-byte access (a rank chunk past r reads rank 0 and is
    // replaced by zero), so the loads of consecutive q stay in flight together.
    auto load_bop = [&](int q, int col) {
        const int e = s_U[q / R16];
        const int rho0 = (q % R16) * 16 + 8 * h;
        const uint16_t* bp = B + ((int64_t)e * d_out + (col < d_out ? col : 0)) * r + rho0;
        u32x4 ao = {0u, 0u, 0u, 0u};
        if constexpr (RVEC) {
            const u32x4 t = ld128(bp - (rho0 < r ? 0 : rho0));
            ao = rho0 < r ? t : ao;
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = (rho0 + 2 * j < r) ? gld(bp + 2 * j) : 0u;
                const uint32_t hi = (rho0 + 2 * j + 1 < r) ? gld(bp + 2 * j + 1) : 0u;
                ao[j] = lo | (hi << 16);
            }
        }
        return ao;
    };

    if (shared_u) {
        for (int q = w; q < nq; q += 4) make_u(q, s_u[q][0][lane], s_u[q][1][lane]);
    }
    __syncthreads();
    if (nblk == 0) return;

#pragma unroll 1
    for (int blk = 0; blk < nblk; ++blk) {
        if (blk + 1 < nblk) load_y(ynxt, blk + 1);
        const int c0b = cw + blk * 64;
        int ocol[2];
#pragma unroll
        for (int b = 0; b < 2; ++b) ocol[b] = c0b + 32 * b + perm_col(n);
        f32x16 acc[2] = {f32x16{}, f32x16{}};
        if (shared_u) {
            // q in groups of four: the group's B operands are all loaded before
            // its MFMAs (q past nq re-reads q = nq - 1 and is skipped); each acc
            // still sums q in order
            for (int q0 = 0; q0 < nq; q0 += 4) {
                u32x4 bo[4][2];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int qj = q0 + j < nq ? q0 + j : nq - 1;
#pragma unroll
                    for (int b = 0; b < 2; ++b) bo[j][b] = load_bop(qj, ocol[b]);
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (q0 + j >= nq) break;
                    const u32x4 uh = s_u[q0 + j][0][lane], ul = s_u[q0 + j][1][lane];
#pragma unroll
                    for (int b = 0; b < 2; ++b) {
                        acc[b] = mfma32(bo[j][b], uh, acc[b]);
                        acc[b] = mfma32(bo[j][b], ul, acc[b]);
                    }
                }
            }
        } else {
            for (int q = 0; q < nq; ++q) {
                u32x4 bh, bl;
                make_u(q, bh, bl);
#pragma unroll
                for (int b = 0; b < 2; ++b) {
                    const u32x4 ao = load_bop(q, ocol[b]);
                    acc[b] = mfma32(ao, bh, acc[b]);
                    acc[b] = mfma32(ao, bl, acc[b]);
                }
            }
        }
        // y: row-major registers -> scratch -> MFMA layout (row n, columns
        // 32b + 16h + [0,16)); add, round once; back through the scratch -> global
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)(ys + y_off(8 * i + lr, lc)) = ycur[i];
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const u32x4 ym = *(const u32x4*)(ys + y_off(n, 4 * b + 2 * h + q));
                uint32_t ow[4];
#pragma unroll
                for (int p = 0; p < 4; ++p) {
                    const int i = 8 * q + 2 * p;
                    ow[p] = pack2_bf16(bf_lo(ym[p]) + acc[b][i], bf_hi(ym[p]) + acc[b][i + 1]);
                }
                *(u32x4*)(ys + y_off(n, 4 * b + 2 * h + q)) = u32x4{ow[0], ow[1], ow[2], ow[3]};
            }
        const int col = c0b + 8 * lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const u32x4 o = *(const u32x4*)(ys + y_off(8 * i + lr, lc));
            if (yrow[i] >= 0 && col < d_out) st128_nt(y + (int64_t)yrow[i] * d_out + col, o);
        }
        if (blk + 1 < nblk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ycur[i] = ynxt[i];
        }
    }
}

// Live work items only, as for the shrink: (column group, live tile).  The
// last kExpandSplit items of each XCD's share run as two half items each
// (kECols / 2 columns), dispatched last: a launch drains for about one item's
// duration while its last items finish, and half items halve that.  Every
// column is computed the same way in either form.
template <int R16, bool RVEC>
__global__ __launch_bounds__(256) void sgmm_expand_bf16(SgmmArgs a) {
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    __shared__ int32_t s_iperm[kWave];
    __shared__ uint32_t s_iep[kWave];
    __shared__ f32x2 s_ig[kWave];
    __shared__ int s_inpos;
    int n_tiles;
    if (a.inline_seg) {
        if (threadIdx.x < kWave) {
            const int np = inline_order(a, s_iperm, s_iep, s_ig);
            if (threadIdx.x == 0) s_inpos = np;
        }
        __syncthreads();
        const int np = s_inpos;
        if (np < 0) return;
        n_tiles = (np + 31) / 32;
    } else {
        n_tiles = uniform(gld(hdr + SG_NTILES));
        if (gld(hdr + SG_ERR)) return;
    }
    const int64_t n_live = a.total_cb * n_tiles, per = (n_live + 7) / 8;
    const int64_t m = per < kExpandSplit ? per : kExpandSplit;
    const int64_t bid = blockIdx.x, j = bid >> 3;
    if (j >= per + m) return;
    int64_t jj = j;
    int half = -1;
    if (j >= per - m) {
        const int64_t k = j - (per - m);
        jj = per - m + (k >> 1);
        half = (int)(k & 1);
    }
    const int64_t t = (bid & 7) * per + jj;
    if (t >= n_live) return;
    const int64_t cgg = t / n_tiles;
    __shared__ ExpandLds sm;
    expand_item<R16, RVEC>(a, cgg, (int)(t - cgg * n_tiles), half, a.inline_seg ? s_iperm : nullptr,
                           a.inline_seg ? s_iep : nullptr, a.inline_seg ? s_ig : nullptr, sm);
}

// ---- one launch: shrink then expand ---------------------------------------------
// After the segmentation (which wrote each XCD's work range and cleared the
// counts): workgroup b runs item b / 8 of XCD b % 8's range -- first the range's
// shrink items (problem by problem, K slice by K slice, tiles fastest), then
// its expand items (column group by column group, tiles fastest).  An expand
// item waits for its (problem, tile)'s K-slice count, which only shrink items
// of the same range -- lower item numbers on the same XCD, dispatched earlier --
// raise, so every wait ends; the last of a launch's shrink items overlap the
// first expand items instead of draining alone.  Each item's arithmetic is that
// of the two-launch form, so y gets the same bits.  The workgroups go to the
// XCDs round-robin (from an XCD that depends on what ran before, as HIP-graph
// replays show), so equal b % 8 means one XCD; the counts also carry their
// producers' XCD ids, and an expand item whose producers ran on another XCD
// sets the error word to 3.
union FusedLds {
    ShrinkLds s;
    ExpandLds e;
};

template <int R16, bool PK, bool RVEC>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3)))
void sgmm_fused_bf16(SgmmArgs a) {
    int32_t* hdr = (int32_t*)(a.ws + a.L.hdr);
    __shared__ FusedLds lds;
    const int x = (int)(blockIdx.x & 7), j = (int)(blockIdx.x >> 3);
    const u32x4* tab = (const u32x4*)(a.ws + a.L.xcd) + x * (kSgmmXcdWords / 4);
    const int n_tiles = gld(hdr + SG_NTILES), err = gld(hdr + SG_ERR);
    u32x4 tw[kSgmmXcdWords / 4];
#pragma unroll
    for (int k = 0; k < kSgmmXcdWords / 4; ++k) tw[k] = ld128(tab + k);
    if (uniform(err) == 1) return;  // a bad set: the call is a no-op
    int e[kSgmmXcdWords];
#pragma unroll
    for (int k = 0; k < kSgmmXcdWords; ++k) e[k] = uniform((int)tw[k / 4][k % 4]);
    const int nt = uniform(n_tiles);
    int32_t* dep = (int32_t*)(a.ws + a.L.dep);
    const int n_s = e[6], n_e = e[12];
    const int cnt_a = (e[0] == e[2] ? e[3] : nt) - e[1];
    if (j < n_s) {
        int64_t g;
        int t;
        if (j < e[4]) {
            g = e[7] + j / cnt_a;
            t = e[1] + j % cnt_a;
        } else if (j < e[4] + e[5]) {
            const int u = j - e[4];
            g = e[8] + u / nt;
            t = u % nt;
        } else {
            const int u = j - e[4] - e[5];
            g = e[9] + u / e[3];
            t = u % e[3];
        }
        shrink_item<R16, PK>(a, g, t, nt, nullptr, nullptr, lds.s, dep);
    } else if (j < n_s + n_e) {
        const int jj = j - n_s;
        int64_t c;
        int t;
        if (jj < e[10]) {
            c = e[13] + jj / cnt_a;
            t = e[1] + jj % cnt_a;
        } else if (jj < e[10] + e[11]) {
            const int u = jj - e[10];
            c = e[14] + u / nt;
            t = u % nt;
        } else {
            const int u = jj - e[10] - e[11];
            c = e[15] + u / e[3];
            t = u % e[3];
        }
        expand_item<R16, RVEC>(a, c, t, -1, nullptr, nullptr, nullptr, lds.e, dep);
    }
}

// Items one XCD's range can hold: its weight is at most an eighth of the
// total plus one pair's (see sgmm_fused_ranges).
inline int64_t fused_per_xcd(const SgmmArgs& a) {
    return ((a.total_ks + a.total_cb) * a.L.tiles_max + 7) / 8 + 1 + a.w_max;
}

// ---- few rows (bf16, T <= kSgmmSmallT) -----------------------------------------

// With at most kSgmmSmallT rows there is nothing to segment: every workgroup
// reads all rows' sets itself (a rejected set makes the whole call a no-op, as
// in the segmented path) and works on all rows at once.
//   * one problem: one launch.  Each kSgmmExpandCols-column group computes the
//     rank vectors v[t][k][rho] = sum_j x[t][j] A[e_tk][rho][j] over all of K,
//     then its columns.
//   * a group: two launches.  One workgroup per (problem, kSgmmKSlice-wide K
//     slice) writes the slice's partial v to the workspace; then each column
//     group adds its problem's slices in slice order and updates its columns.
//     The K slices spread a problem's A over several workgroups, which a
//     column group computing all of v by itself cannot.
// The dot products run with all threads over the 16-byte chunks of K, 16 or
// 32 of them at a time and every load of a chunk issued before its FMAs, then a
// fixed-order reduction (wave butterfly, then the waves in order): every
// column group of a problem gets the same bits.  The columns:
//     y[t][o] = round(y[t][o] + (c_t0 p_t0 + c_t1 p_t1)),
//     p_tk = sum_rho v[t][k][rho] B[e_tk][o][rho],  c = s g,
// four consecutive columns per thread; rows with two empty slots are not
// written.  For one decode token this is one or two launches instead of four.
__device__ __forceinline__ float wave_sum_f(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

constexpr int kSmallThreads = 512;
constexpr int kSmallMaxR = 128;

// Every thread checks every row's set; workgroup 0 publishes the result.
__device__ __forceinline__ bool small_sets_bad(const SgmmArgs& a) {
    bool bad = false;
    for (int q = 0; q < 2 * (int)a.T; ++q) {
        const int e = gld(a.idx + q);
        const float g = gld(a.g + q);
        if (e < -1 || e >= a.E || (e >= 0 && !__builtin_isfinite(g))) bad = true;
    }
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        int32_t* hdr = (int32_t*)(a.ws + a.L.hdr);
        gst(hdr + SG_ERR, bad ? 1 : 0);
        if (a.status_out) gst(a.status_out, bad ? 1 : 0);
    }
    return bad;
}

// v[t][k][rho] over the 16-byte K chunks [c0, c1), handed to out(d, value) for
// dot product d = (t * 2 + k) * r + rho (0 for an empty slot), kSmallDots of
// them per sweep over the chunks.  Uses s_red[waves][kSmallDots]; every
// thread calls it.
template <int kSmallDots, typename Out>
__device__ __forceinline__ void small_dots(const SgmmArgs& a, const uint16_t* __restrict__ x,
                                           const uint16_t* __restrict__ A, int d_in, int c0, int c1,
                                           float (*s_red)[kSmallDots], Out out) {
    constexpr int kSW = kSmallThreads / kWave;
    const int T = (int)a.T, r = a.r, tid = threadIdx.x, w = wave_id(), lane = lane_id();
    const int nd = T * 2 * r;
    for (int d0 = 0; d0 < nd; d0 += kSmallDots) {
        float p[kSmallDots];
#pragma unroll
        for (int i = 0; i < kSmallDots; ++i) p[i] = 0.f;
        for (int c = c0 + tid; c < c1; c += kSmallThreads) {
            u32x4 xv[kSgmmSmallT], av[kSmallDots];
#pragma unroll
            for (int t = 0; t < kSgmmSmallT; ++t)
                if (t < T) xv[t] = ld128(x + (int64_t)t * d_in + 8 * c);
#pragma unroll
            for (int i = 0; i < kSmallDots; ++i) {
                const int d = d0 + i < nd ? d0 + i : nd - 1;
                const int t = d / (2 * r), k = (d / r) & 1, rho = d % r;
                const int e = gld(a.idx + 2 * t + k);
                av[i] = ld128(A + ((int64_t)(e >= 0 ? e : 0) * r + rho) * d_in + 8 * c);
            }
#pragma unroll
            for (int i = 0; i < kSmallDots; ++i) {
                const int d = d0 + i < nd ? d0 + i : nd - 1;
                const int t = d / (2 * r);
                u32x4 xt = xv[0];
#pragma unroll
                for (int tt = 1; tt < kSgmmSmallT; ++tt)
                    if (t == tt) xt = xv[tt];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p[i] = fmaf(bf_lo(xt[q]), bf_lo(av[i][q]), p[i]);
                    p[i] = fmaf(bf_hi(xt[q]), bf_hi(av[i][q]), p[i]);
                }
            }
        }
#pragma unroll
        for (int i = 0; i < kSmallDots; ++i) {
            const float sw = wave_sum_f(p[i]);
            if (lane == 0) s_red[w][i] = sw;
        }
        __syncthreads();
        if (tid < kSmallDots && d0 + tid < nd) {
            const int d = d0 + tid;
            const int t = d / (2 * r), k = (d / r) & 1;
            float sv = s_red[0][tid];
#pragma unroll
            for (int ww = 1; ww < kSW; ++ww) sv += s_red[ww][tid];
            out(d, gld(a.idx + 2 * t + k) >= 0 ? sv : 0.f);
        }
        __syncthreads();
    }
}

// The columns of column group cg from v (LDS, [t][k][kSmallMaxR]).
__device__ __forceinline__ void small_columns(const SgmmArgs& a, const SgDesc& D, int cg,
                                              float (*s_v)[2][kSmallMaxR]) {
    const int T = (int)a.T, r = a.r, tid = threadIdx.x, d_out = D.d_out;
    const uint16_t* __restrict__ B = (const uint16_t*)D.B;
    uint16_t* __restrict__ y = (uint16_t*)D.y;
    // four consecutive columns per thread of the first 256 (d_out is a
    // multiple of 8, so a thread's columns are all in range or all out)
    const int col = cg * kSgmmExpandCols + 4 * tid;
    if (tid >= kSgmmExpandCols / 4 || col >= d_out) return;
    const bool rvec = (r & 7) == 0;
    for (int t = 0; t < T; ++t) {
        const int e0 = gld(a.idx + 2 * t), e1 = gld(a.idx + 2 * t + 1);
        if (e0 < 0 && e1 < 0) continue;
        float part[2][4];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = k ? e1 : e0;
            const float c = e >= 0 ? a.scale * gld(a.g + 2 * t + k) : 0.f;
            float acc[4] = {0.f, 0.f, 0.f, 0.f};
            if (e >= 0) {
                const uint16_t* br = B + ((int64_t)e * d_out + col) * r;  // 4 rows of r, contiguous
                if (rvec) {
                    // 16-byte rank chunks of the four rows, 8 in flight
                    for (int r0 = 0; r0 < r; r0 += 16) {
                        u32x4 bv[4][2];
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                const int rr = r0 + 8 * h2 < r ? r0 + 8 * h2 : r0;
                                bv[j][h2] = ld128(br + j * r + rr);
                            }
#pragma unroll
                        for (int j = 0; j < 4; ++j)
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                if (r0 + 8 * h2 >= r) continue;
#pragma unroll
                                for (int q = 0; q < 4; ++q) {
                                    const int rho = r0 + 8 * h2 + 2 * q;
                                    acc[j] = fmaf(s_v[t][k][rho], bf_lo(bv[j][h2][q]), acc[j]);
                                    acc[j] = fmaf(s_v[t][k][rho + 1], bf_hi(bv[j][h2][q]), acc[j]);
                                }
                            }
                    }
                } else {
                    for (int rho = 0; rho < r; ++rho)
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[j] = fmaf(s_v[t][k][rho], bf_to_f(br[j * r + rho]), acc[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) part[k][j] = c * acc[j];
        }
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        uint16_t* yp = y + (int64_t)t * d_out + col;
        const u32x2 yv = *(gcptr<u32x2>)yp;
        const uint32_t o0 = pack2_bf16(bf_lo(yv[0]) + (part[0][0] + part[1][0]), bf_hi(yv[0]) + (part[0][1] + part[1][1]));
        const uint32_t o1 = pack2_bf16(bf_lo(yv[1]) + (part[0][2] + part[1][2]), bf_hi(yv[1]) + (part[0][3] + part[1][3]));
        *(gptr<u32x2>)yp = u32x2{o0, o1};
    }
}

// One problem (a.single also describes a one-problem group): one workgroup per
// column group, v over all of K.
__global__ __launch_bounds__(kSmallThreads) void sgmm_small_bf16(SgmmArgs a) {
    __shared__ float s_v[kSgmmSmallT][2][kSmallMaxR];
    __shared__ float s_red[kSmallThreads / kWave][16];
    if (small_sets_bad(a)) return;
    const SgDesc D = a.single;
    const int r = a.r;
    small_dots<16>(a, (const uint16_t*)D.x, (const uint16_t*)D.A, D.d_in, 0, D.d_in / 8, s_red,
               [&](int d, float v) { s_v[d / (2 * r)][(d / r) & 1][d % r] = v; });
    small_columns(a, D, (int)blockIdx.x, s_v);
}

// A group, first launch: one workgroup per (problem, K slice); the slice's
// partial v goes to the workspace as v[slice][t][k][rho] (rows padded to r_pad).
__global__ __launch_bounds__(kSmallThreads) void sgmm_small_shrink_bf16(SgmmArgs a) {
    // a 2048-wide slice is 256 chunks: half the threads would sweep nothing,
    // so the sweep covers 32 dot products (one for rank 16 and one row)
    __shared__ float s_red[kSmallThreads / kWave][32];
    if (small_sets_bad(a)) return;
    const int64_t gks = blockIdx.x;
    const SgDesc D = a.ks_desc[gks];
    const int k0 = (int)(gks - D.ks0) * kSgmmKSlice;
    const int k1 = k0 + kSgmmKSlice < D.d_in ? k0 + kSgmmKSlice : D.d_in;
    const int r = a.r, RPAD = a.L.r_pad;
    float* v = (float*)(a.ws + a.L.v) + gks * a.L.T_pad * 2 * RPAD;
    small_dots<32>(a, (const uint16_t*)D.x, (const uint16_t*)D.A, D.d_in, k0 / 8, k1 / 8, s_red,
               [&](int d, float val) { gst(v + (d / r) * RPAD + d % r, val); });
}

// A group, second launch: one workgroup per column group; v = the problem's
// slices added in slice order.
__global__ __launch_bounds__(kSmallThreads) void sgmm_small_expand_bf16(SgmmArgs a) {
    __shared__ float s_v[kSgmmSmallT][2][kSmallMaxR];
    bool bad = false;  // the first launch published the result
    for (int q = 0; q < 2 * (int)a.T; ++q) {
        const int e = gld(a.idx + q);
        const float g = gld(a.g + q);
        if (e < -1 || e >= a.E || (e >= 0 && !__builtin_isfinite(g))) bad = true;
    }
    if (bad) return;
    const int64_t cgg = blockIdx.x;
    const SgDesc D = a.cb_desc[cgg];
    const int r = a.r, RPAD = a.L.r_pad, nd = (int)a.T * 2 * r;
    const int64_t stride = a.L.T_pad * 2 * RPAD;  // floats per slice
    const float* v = (const float*)(a.ws + a.L.v) + D.ks0 * stride;
    for (int d = threadIdx.x; d < nd; d += kSmallThreads) {
        const int o = (d / r) * RPAD + d % r;
        // the slices' partials eight at a time, all loads first, added in order
        float sv = 0.f;
        for (int s0 = 0; s0 < D.n_ks; s0 += 8) {
            float pv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) pv[j] = s0 + j < D.n_ks ? gld(v + (s0 + j) * stride + o) : 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (s0 + j < D.n_ks) sv = (s0 + j == 0) ? pv[j] : sv + pv[j];
        }
        s_v[d / (2 * r)][(d / r) & 1][d % r] = sv;
    }
    __syncthreads();
    small_columns(a, D, (int)(cgg - D.unit0), s_v);
}

// ---- element-wise path (fp32) ------------------------------------------------

template <typename T> __device__ __forceinline__ float ldf(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, int64_t i) { return p[i]; }
template <typename T> __device__ __forceinline__ void stf(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, int64_t i, float v) { p[i] = v; }

// v[pos][slot][rho] = sum_j x[row][j] * A[e_slot][rho][j], one thread each.
template <typename T>
__global__ __launch_bounds__(256) void sgmm_shrink_generic(SgmmArgs a) {
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    if (hdr[SG_ERR]) return;
    const int prob = blockIdx.y;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int RPAD = a.L.r_pad;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_pos = hdr[SG_NPOS];
    if (q >= n_pos * 2 * a.r) return;
    const int64_t pos = q / (2 * a.r);
    const int slot = (int)((q / a.r) % 2), rho = (int)(q % a.r);
    const int row = ((const int32_t*)(a.ws + a.L.perm))[pos];
    const int e = a.idx[2 * (int64_t)row + slot];
    float acc = 0.f;
    if (e >= 0) {
        const T* x = (const T*)D.x + (int64_t)row * D.d_in;
        const T* A = (const T*)D.A + ((int64_t)e * a.r + rho) * D.d_in;
        for (int j = 0; j < D.d_in; ++j) acc = fmaf(ldf(x, j), ldf(A, j), acc);
    }
    float* v = (float*)(a.ws + a.L.v) + D.ks0 * a.L.T_pad * 2 * RPAD;
    v[(pos * 2 + slot) * RPAD + rho] = acc;
}

// y[row][o] += c0 * (v0 . B[e0][o]) + c1 * (v1 . B[e1][o]), one thread each.
template <typename T>
__global__ __launch_bounds__(256) void sgmm_expand_generic(SgmmArgs a) {
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    if (hdr[SG_ERR]) return;
    const int prob = blockIdx.y;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int RPAD = a.L.r_pad;
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t n_pos = hdr[SG_NPOS];
    if (q >= n_pos * D.d_out) return;
    const int64_t pos = q / D.d_out;
    const int o = (int)(q % D.d_out);
    const int row = ((const int32_t*)(a.ws + a.L.perm))[pos];
    const float* v = (const float*)(a.ws + a.L.v) + D.ks0 * a.L.T_pad * 2 * RPAD;
    const T* B = (const T*)D.B;
    float part[2];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int e = a.idx[2 * (int64_t)row + k];
        float acc = 0.f;
        if (e >= 0)
            for (int rho = 0; rho < a.r; ++rho)
                acc = fmaf(v[(pos * 2 + k) * RPAD + rho], ldf(B, ((int64_t)e * D.d_out + o) * a.r + rho), acc);
        part[k] = e >= 0 ? a.scale * a.g[2 * (int64_t)row + k] * acc : 0.f;
    }
    T* y = (T*)D.y;
    const int64_t i = (int64_t)row * D.d_out + o;
    stf(y, i, ldf(y, i) + (part[0] + part[1]));
}

// ---- K-slice sum ---------------------------------------------------------------

// v of every problem with several K slices: slice 0 <- slice 0 + slice 1 + ...,
// added in slice order (the sum is the same on every run).  One thread per
// four floats of the rows in use.
__global__ __launch_bounds__(256) void sgmm_vsum_kernel(SgmmArgs a) {
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    if (gld(hdr + SG_ERR)) return;
    const int prob = blockIdx.y;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int nks = D.n_ks;
    if (nks <= 1) return;
    const int64_t n4 = (int64_t)gld(hdr + SG_NPOS) * 2 * a.L.r_pad / 4;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n4) return;
    const int64_t stride = a.L.T_pad * 2 * a.L.r_pad;  // floats per slice
    float* v = (float*)(a.ws + a.L.v) + D.ks0 * stride + 4 * i;
    u32x4 acc = ld128(v);
    int ks = 1;
    for (; ks + 4 <= nks; ks += 4) {
        u32x4 p[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) p[j] = ld128(v + (ks + j) * stride);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[c] = __float_as_uint(__uint_as_float(acc[c]) + __uint_as_float(p[j][c]));
    }
    for (; ks < nks; ++ks) {
        const u32x4 p = ld128(v + ks * stride);
#pragma unroll
        for (int c = 0; c < 4; ++c) acc[c] = __float_as_uint(__uint_as_float(acc[c]) + __uint_as_float(p[c]));
    }
    st128(v, acc);
}

// ---- A packing -------------------------------------------------------------------

// One thread per 16-byte group: Ap[e][kq][rho] = A[e][rho][8kq .. 8kq+8).
__global__ __launch_bounds__(256) void sgmm_pack_a_kernel(const uint16_t* __restrict__ A,
                                                          uint16_t* __restrict__ Ap, int r,
                                                          int64_t nq, int64_t total) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int64_t rho = i % r, kq = (i / r) % nq, e = i / (r * nq);
    st128(Ap + 8 * i, ld128(A + ((e * r + rho) * nq + kq) * 8));
}

// Grid for at most max_items work items (a multiple of 8: one share per XCD).
inline int64_t item_grid(int64_t max_items) { return 8 * ((max_items + 7) / 8); }

template <int R16>
hipError_t launch_mfma(const SgmmArgs& a, hipStream_t s) {
    const dim3 gs((unsigned)item_grid(a.total_ks * a.L.tiles_max));
    if (a.packed)
        hipLaunchKernelGGL((sgmm_shrink_bf16<R16, true>), gs, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((sgmm_shrink_bf16<R16, false>), gs, dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (R16 > kExpandFoldR16 && a.total_ks > a.n_prob) {  // K slices the expand does not add itself
        const dim3 gs((unsigned)((a.L.T_pad * 2 * a.L.r_pad / 4 + 255) / 256), (unsigned)a.n_prob);
        hipLaunchKernelGGL(sgmm_vsum_kernel, gs, dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t per_max = (a.n_expand_units + 7) / 8;
    const dim3 ge((unsigned)(8 * (per_max + (per_max < kExpandSplit ? per_max : kExpandSplit))));
    if (a.r % 8 == 0)
        hipLaunchKernelGGL((sgmm_expand_bf16<R16, true>), ge, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((sgmm_expand_bf16<R16, false>), ge, dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int R16>
hipError_t launch_fused(const SgmmArgs& a, hipStream_t s) {
    const dim3 gf((unsigned)(8 * fused_per_xcd(a)));
    if (a.packed) {
        if (a.r % 8 == 0) hipLaunchKernelGGL((sgmm_fused_bf16<R16, true, true>), gf, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((sgmm_fused_bf16<R16, true, false>), gf, dim3(256), 0, s, a);
    } else {
        if (a.r % 8 == 0) hipLaunchKernelGGL((sgmm_fused_bf16<R16, false, true>), gf, dim3(256), 0, s, a);
        else hipLaunchKernelGGL((sgmm_fused_bf16<R16, false, false>), gf, dim3(256), 0, s, a);
    }
    return hipGetLastError();
}

hipError_t launch_fused_r(const SgmmArgs& a, hipStream_t s) {
    switch (a.L.r_pad / 16) {
        case 1: return launch_fused<1>(a, s);
        case 2: return launch_fused<2>(a, s);
        case 3: return launch_fused<3>(a, s);
        case 4: return launch_fused<4>(a, s);
        default: return hipErrorInvalidValue;
    }
}

// The MFMA launches for the workspace's padded rank.
hipError_t launch_mfma_r(const SgmmArgs& a, hipStream_t s) {
    switch (a.L.r_pad / 16) {
        case 1: return launch_mfma<1>(a, s);
        case 2: return launch_mfma<2>(a, s);
        case 3: return launch_mfma<3>(a, s);
        case 4: return launch_mfma<4>(a, s);
        case 5: return launch_mfma<5>(a, s);
        case 6: return launch_mfma<6>(a, s);
        case 7: return launch_mfma<7>(a, s);
        case 8: return launch_mfma<8>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

hipError_t launch_sgmm_pack_a(const void* A, void* Ap, int E, int r, int64_t d_in, hipStream_t s) {
    const int64_t nq = d_in / 8, total = (int64_t)E * r * nq;
    if (!grid_fits((total + 255) / 256, 256)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(sgmm_pack_a_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s,
                       (const uint16_t*)A, (uint16_t*)Ap, r, nq, total);
    return hipGetLastError();
}

// Every grid of the call fits (checked before the first launch, so a refused
// call leaves the workspace and y untouched).
static bool sgmm_grids_fit(const SgmmArgs& a, int dtype) {
    if (!grid_fits(a.L.n_chunks, kSegThreads)) return false;
    if (dtype == 1) {
        const int64_t per_max = (a.n_expand_units + 7) / 8;
        return grid_fits((a.L.T_pad * 2 * a.L.r_pad / 4 + 255) / 256, 256) &&
               grid_fits(item_grid(a.total_ks * a.L.tiles_max), 256) && grid_fits(8 * fused_per_xcd(a), 256) &&
               grid_fits(8 * (per_max + (per_max < kExpandSplit ? per_max : kExpandSplit)), 256);
    }
    return grid_fits((a.L.T_pad * 2 * a.r + 255) / 256, 256) &&
           grid_fits((a.L.T_pad * a.d_out_max + 255) / 256, 256);
}

hipError_t launch_sgmm(const SgmmArgs& a, int dtype, hipStream_t s) {
    if (dtype == 1 && a.T <= kSgmmSmallT) {
        if (!grid_fits(a.total_cb, kSmallThreads) || !grid_fits(a.total_ks, kSmallThreads))
            return hipErrorInvalidConfiguration;
        if (a.n_prob == 1) {
            hipLaunchKernelGGL(sgmm_small_bf16, dim3((unsigned)a.total_cb), dim3(kSmallThreads), 0, s, a);
            return hipGetLastError();
        }
        hipLaunchKernelGGL(sgmm_small_shrink_bf16, dim3((unsigned)a.total_ks), dim3(kSmallThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL(sgmm_small_expand_bf16, dim3((unsigned)a.total_cb), dim3(kSmallThreads), 0, s, a);
        return hipGetLastError();
    }
    if (!sgmm_grids_fit(a, dtype)) return hipErrorInvalidConfiguration;
    // at most one wave of rows and no K-slice sum launch: the shrink and
    // expand workgroups order the rows themselves, no segmentation launch
    static_assert(kSgmmInlineRows <= kWave, "inline ordering: one row per lane");
    const bool fold = a.L.r_pad / 16 <= kExpandFoldR16;
    const bool fused = dtype == 1 && fold && a.L.max_ks <= kSgmmFusedMaxKs && kSgmmFused > 0 &&
                       (int64_t)a.n_prob * a.L.tiles_max >= kSgmmFusedMinPairs &&
                       (kSgmmFused > 1 || a.T > kSgmmInlineRows);
    const bool inl = !fused && dtype == 1 && a.T <= kSgmmInlineRows &&
                     !(a.L.r_pad / 16 > kExpandFoldR16 && a.total_ks > a.n_prob);
    if (inl) {
        SgmmArgs b = a;
        b.inline_seg = 1;
        return launch_mfma_r(b, s);
    }
    static_assert(kSegThreads == kSgmmSegRows, "segmentation chunk");
    const int64_t n_chunks = a.L.n_chunks;
    if (n_chunks > kSegFewChunks) {
        hipLaunchKernelGGL(sgmm_seg_count, dim3((unsigned)n_chunks), dim3(kSegThreads), 0, s, a.idx, a.g, a.T, a.E,
                           a.ws, a.L);
        hipError_t e0 = hipGetLastError();
        if (e0 != hipSuccess) return e0;
    }
    hipLaunchKernelGGL(sgmm_seg_place, dim3((unsigned)n_chunks), dim3(kSegThreads), 0, s, a.idx, a.g, a.T, a.E,
                       a.ws, a.L, a.status_out, a.descs, a.single, a.n_prob, a.total_ks, a.total_cb,
                       fused ? 1 : 0);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fused) return launch_fused_r(a, s);
    if (dtype == 1) return launch_mfma_r(a, s);
    // fp32: element-wise kernels, grid sized for the most rows possible
    const dim3 g1((unsigned)((a.L.T_pad * 2 * a.r + 255) / 256), (unsigned)a.n_prob);
    hipLaunchKernelGGL(sgmm_shrink_generic<float>, g1, dim3(256), 0, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const dim3 g2((unsigned)((a.L.T_pad * a.d_out_max + 255) / 256), (unsigned)a.n_prob);
    hipLaunchKernelGGL(sgmm_expand_generic<float>, g2, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dlm
