// SGMM: batched unmerged adapters for rows carrying different expert sets,
//     y[t] <- round( y[t] + sum_k s*g[t][k] * B_{e_k} (A_{e_k} x[t]) ).
// The AdaFuse digest (section 2-na) names its core kernel SGMM, "segmented
// gather matrix multiplication"; this is the batched form of the same adapters.
//
// Launches:
//   segment  (one workgroup) every row gets the key of its unordered expert
//            pair; a stable counting sort lists the rows by key (perm, with
//            each position's pair and gates beside it), so rows sharing
//            experts sit next to each other.  The sorted list is cut into
//            32-row tiles and each tile records the union of the experts its
//            rows use (a bitmask).  Rows with two empty slots are left out.
//            The same segmentation serves every problem of a grouped call
//            (one routing decision per token for all layers).
//   shrink   per (problem, 512-wide K slice, tile): the slice's partial
//            v = x_rows A_U^T for the tile's experts U, bf16 MFMA 32x32x16 with
//            M = tile rows (gathered through perm, staged in LDS), N = (expert,
//            rank); each row keeps the fp32 partial v of its own two slots.
//   sum      (problems with d_in > 512) the slices' partials added in slice
//            order.
//   expand   per (problem, 1024 output columns, tile): y_rows += u B_U^T with
//            u = s*g*v per (row, expert, rank).  u stays fp32-accurate by
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
    (void)E;
    size_t o = 0;
    L.hdr = o;   o += 256;
    L.perm = o;  o += a256((size_t)L.T_pad * 4);
    L.epk = o;   o += a256((size_t)L.T_pad * 4);
    L.gpk = o;   o += a256((size_t)L.T_pad * 8);
    L.tmask = o; o += a256((size_t)L.tiles_max * 4);
    L.v = o;     o += a256((size_t)n_prob * L.max_ks * L.T_pad * 2 * L.r_pad * 4);
    L.total = o;
    return L;
}

namespace {

constexpr int kSegThreads = 1024;
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

// One workgroup: a stable counting sort of the rows by key, all bookkeeping in
// LDS.  Pass 1 counts the keys (and keeps the keys of the first kKeyCache rows
// in LDS); their exclusive scan gives each key's first position.  Pass 2 takes
// the rows in batches of kSegThreads, in order: a row's position = its key's
// first position + rows of that key in earlier batches + in earlier waves of
// this batch + earlier lanes of its wave with the same key (a lane's
// same-key mask comes from one ballot per key bit, so the cost does not grow
// with the number of distinct keys in the wave).  A batch's sets are loaded at
// its start and first needed when the rows are written out.
constexpr int kKeyCache = 8192;
constexpr int kTileCache = kKeyCache / 32;
__global__ __launch_bounds__(kSegThreads) void sgmm_segment_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ g, int64_t T, int E, char* ws,
    SgLayout L) {
    int32_t* hdr = (int32_t*)(ws + L.hdr);
    int32_t* perm = (int32_t*)(ws + L.perm);
    uint32_t* epk = (uint32_t*)(ws + L.epk);
    float* gpk = (float*)(ws + L.gpk);
    uint32_t* tmask = (uint32_t*)(ws + L.tmask);
    __shared__ int s_err;
    __shared__ int s_next[kMaxKeys];   // counts, then the next free position of each key
    __shared__ int s_base[kMaxKeys];   // first position of each key in the current batch
    __shared__ uint16_t s_wc[kSegWaves][kMaxKeys];  // per-wave counts of a batch, then
                                                    // their exclusive prefix over waves
    __shared__ int16_t s_key[kKeyCache];
    __shared__ uint32_t s_tm[kTileCache];
    __shared__ int s_tot[kSegWaves];
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int nk = (E + 1) * (E + 1);
    const int nbits = 32 - __builtin_clz((unsigned)(nk - 1));
    const uint64_t lt_mask = (1ull << lane) - 1ull;
    if (tid == 0) s_err = 0;
    for (int k = tid; k < nk; k += kSegThreads) s_next[k] = 0;
    for (int q = tid; q < kTileCache; q += kSegThreads) s_tm[q] = 0;
    __syncthreads();

    // pass 1: key counts (LDS atomics)
    for (int64_t b0 = 0; b0 < T; b0 += 4 * kSegThreads) {
        SegRaw raw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) raw[j] = seg_load(idx, g, b0 + j * kSegThreads + tid, T);
        __builtin_amdgcn_sched_barrier(0);  // all four rows' loads are issued first
        SegRow q[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = seg_row(raw[j], b0 + j * kSegThreads + tid < T, E);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int64_t t = b0 + j * kSegThreads + tid;
            if (q[j].bad) s_err = 1;
            if (t < kKeyCache) s_key[t] = (int16_t)q[j].key;
            if (q[j].key >= 0) atomicAdd(&s_next[q[j].key], 1);
        }
    }
    __syncthreads();
    const int err = s_err;

    // exclusive scan of the counts in key order (each thread owns a run of keys)
    constexpr int kPer = (kMaxKeys + kSegThreads - 1) / kSegThreads;
    int cnt[kPer], run = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int k = tid * kPer + j;
        cnt[j] = k < nk ? s_next[k] : 0;
        run += cnt[j];
    }
    int n_pos;
    int base = block_exscan(run, s_tot, n_pos);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
        const int k = tid * kPer + j;
        if (k < nk) s_next[k] = base;
        base += cnt[j];
    }
    if (err) n_pos = 0;
    const int n_tiles = (n_pos + 31) / 32;
    const bool lds_masks = n_tiles <= kTileCache;
    __syncthreads();

    // pass 2: place the rows batch by batch
    for (int64_t b0 = 0; !err && b0 < T; b0 += kSegThreads) {
        const int64_t t = b0 + tid;
        const SegRaw raw = seg_load(idx, g, t, T);  // first needed when the row is written
        static_assert(kKeyCache % kSegThreads == 0, "key cache holds whole batches");
        for (int q = tid; q < kSegWaves * nk; q += kSegThreads) s_wc[q / nk][q % nk] = 0;
        __syncthreads();
        int k;
        if (b0 + kSegThreads <= kKeyCache)  // batch-uniform: keys from LDS, the loads stay in flight
            k = t < T ? (int)s_key[t] : -1;
        else
            k = seg_row(raw, t < T, E).key;
        // stable rank within the wave and the wave's count of each key
        const uint64_t same = wave_match(k, nbits);
        const int rk = (int)__popcll(same & lt_mask);
        if (same && rk == 0) s_wc[w][k] = (uint16_t)__popcll(same);
        __syncthreads();
        // rows of each key in earlier waves of the batch, in wave order
        for (int kk = tid; kk < nk; kk += kSegThreads) {
            int acc = 0;
            for (int i = 0; i < kSegWaves; ++i) {
                const int c = s_wc[i][kk];
                s_wc[i][kk] = (uint16_t)acc;
                acc += c;
            }
            s_base[kk] = s_next[kk];
            s_next[kk] += acc;
        }
        __syncthreads();
        if (k >= 0) {
            const SegRow cur = seg_row(raw, true, E);
            const int64_t p = (int64_t)s_base[k] + s_wc[w][k] + rk;
            perm[p] = (int32_t)t;
            epk[p] = ((uint32_t)cur.e0 & 0xffffu) | ((uint32_t)cur.e1 << 16);
            gpk[2 * p] = cur.e0 >= 0 ? cur.g0 : 0.f;
            gpk[2 * p + 1] = cur.e1 >= 0 ? cur.g1 : 0.f;
            if (lds_masks) {
                const uint32_t m = (cur.e0 >= 0 ? 1u << cur.e0 : 0u) | (cur.e1 >= 0 ? 1u << cur.e1 : 0u);
                atomicOr(&s_tm[p >> 5], m);
            }
        }
    }
    for (int64_t p = n_pos + tid; p < L.T_pad; p += kSegThreads) {
        perm[p] = -1;
        epk[p] = 0xffffffffu;
        gpk[2 * p] = 0.f;
        gpk[2 * p + 1] = 0.f;
    }
    __syncthreads();

    // tile masks: from LDS, or (more tiles than LDS keeps) each half-wave ORs
    // the expert bits of one tile's 32 positions read back from epk
    if (lds_masks) {
        for (int q = tid; q < n_tiles; q += kSegThreads) tmask[q] = s_tm[q];
    } else {
        for (int64_t q0 = 2 * w; q0 < n_tiles; q0 += 8 * kSegWaves) {
            uint32_t m[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t q = q0 + 2 * kSegWaves * j + (lane >> 5);
                const uint32_t ep = q < n_tiles ? epk[q * 32 + (lane & 31)] : 0xffffffffu;
                const int e0 = (int16_t)(ep & 0xffffu), e1 = (int16_t)(ep >> 16);
                m[j] = (e0 >= 0 ? 1u << e0 : 0u) | (e1 >= 0 ? 1u << e1 : 0u);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int o = 1; o < 32; o <<= 1) m[j] |= __shfl_xor(m[j], o, kWave);
                const int64_t q = q0 + 2 * kSegWaves * j + (lane >> 5);
                if ((lane & 31) == 0 && q < n_tiles) tmask[q] = m[j];
            }
        }
    }
    if (tid == 0) {
        hdr[SG_ERR] = err;
        hdr[SG_NPOS] = n_pos;
        hdr[SG_NTILES] = n_tiles;
    }
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

// Tiles per shrink work item: every A operand feeds one MFMA per tile.  Only
// one tile per item is built and tested (two measured slower on both
// workloads); the loops over kTM keep the shape of the multi-tile form.
constexpr int kTM = 1;
static_assert(kTM == 1, "only single-tile shrink work items are tested");
constexpr int kXRows = 32 * kTM;
// 64-wide K chunks of one slice, and 16-byte chunks of one x row of a slice
constexpr int kKC = kSgmmKSlice / 64;
constexpr int kXC = kSgmmKSlice / 8;
// A chunks in flight per wave in the shrink's K loop.  The shrink runs at 4
// waves per SIMD (3 for ranks 17..32, which would spill at 4): several
// workgroups per CU, each with a 32 KB x slice.  Measured on the 4096-token
// prefill: 114 us with 1024-wide slices, a 4-chunk ring and 2 waves per SIMD;
// 102 us like this at 3 waves per SIMD, 98 us at 4.
constexpr int kShrinkRing = 2;
static_assert(kKC >= kShrinkRing && kKC % kShrinkRing == 0, "slice is a whole number of ring steps");
static_assert(256 % kXC == 0 && kXRows % (256 / kXC) == 0, "x slice load shape");
// x slice in LDS: kXRows rows of kSgmmKSlice bf16; the 16-byte chunk c of row m
// is stored at chunk c ^ (m & 15), so the MFMA-layout reads (16 rows, one chunk)
// and the row-contiguous writes both touch 16 distinct bank groups.
__device__ __forceinline__ int x_off(int row, int c) { return row * kSgmmKSlice + ((c ^ (row & 15)) << 3); }
// per-wave 32x64 bf16 scratch of the expand: rows of eight 16-byte chunks, chunk XOR (row & 7)
__device__ __forceinline__ int y_off(int row, int chunk) { return row * 64 + ((chunk ^ (row & 7)) << 3); }

// One work item = (problem, K slice, kTM consecutive tiles), the tiles fastest
// so the work items that share a slice of A run next to each other on one XCD.
// The four waves first read the tiles' x rows of the slice, row-contiguous
// (each x byte is read once), into LDS.  The N blocks (32 columns of (expert,
// rank) each, over the union of the tiles' experts) are then spread over the
// waves: with four or more blocks each wave takes whole blocks; with fewer, the
// waves of one block split the slice's chunks and their sums are added in a
// fixed order.  The A rows of a block stream from L2 kShrinkRing chunks ahead
// of the MFMAs, and each A operand serves the kTM tiles.  Each row's two
// slots get the slice's partial v; a later pass adds the slices up.  Loads are
// never guarded: a padding row or (expert, rank) column reads an in-bounds
// dummy row whose products reach only accumulator entries that are never
// stored, and k past d_in reads a clamped address whose value is replaced by 0.
template <int R16, bool PK>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(R16 == 2 ? 3 : 4)))
void sgmm_shrink_bf16(SgmmArgs a, int64_t n_units, int64_t per_xcd) {
    constexpr int RPAD = R16 * 16;
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    if (gld(hdr + SG_ERR)) return;
    const int64_t bid = blockIdx.x;
    const int64_t t = (bid & 7) * per_xcd + (bid >> 3);
    if (t >= n_units) return;
    const int64_t ntp = (a.L.tiles_max + kTM - 1) / kTM;
    const int64_t gks = t / ntp;  // slice index over all problems
    const int tile0 = (int)(t - gks * ntp) * kTM;
    const int n_tiles = gld(hdr + SG_NTILES);
    if (tile0 >= n_tiles) return;
    const int prob = a.descs ? gld(a.ks_owner + gks) : 0;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int k0 = (int)(gks - D.ks0) * kSgmmKSlice;
    const int32_t* perm = (const int32_t*)(a.ws + a.L.perm);
    const uint32_t* epk = (const uint32_t*)(a.ws + a.L.epk);
    const uint32_t* tmask = (const uint32_t*)(a.ws + a.L.tmask);
    float* v = (float*)(a.ws + a.L.v) + gks * a.L.T_pad * 2 * RPAD;

    __shared__ __attribute__((aligned(16))) uint16_t s_x[kXRows * kSgmmKSlice];
    __shared__ int s_U[32];
    __shared__ int s_nU;
    __shared__ int s_row[kXRows], s_e0[kXRows], s_e1[kXRows];
    const int tid = threadIdx.x;
    if (tid < kXRows) {
        const bool in = tile0 + tid / 32 < n_tiles;
        const int p = tile0 * 32 + tid;
        const int row = in ? gld(perm + p) : -1;
        const uint32_t ep = in ? gld(epk + p) : 0xffffffffu;
        s_row[tid] = row;
        s_e0[tid] = (int16_t)(ep & 0xffffu);
        s_e1[tid] = (int16_t)(ep >> 16);
    }
    if (tid == 0) {
        uint32_t m = 0;
        for (int j = 0; j < kTM; ++j)
            if (tile0 + j < n_tiles) m |= gld(tmask + tile0 + j);
        s_nU = mask_list(m, s_U);
    }
    __syncthreads();

    const int d_in = uniform(D.d_in), r = a.r;
    const uint16_t* __restrict__ x = (const uint16_t*)D.x;
    const uint16_t* __restrict__ A = (const uint16_t*)(PK ? D.Ap : D.A);

    // 1) x slice: thread tid reads chunk tid % kXC of rows tid / kXC + kXR j
    constexpr int kXR = 256 / kXC;           // rows per load instruction
    constexpr int kXL = kXRows / kXR;        // load instructions per thread
    const int xc = tid % kXC, xr0 = tid / kXC;
    const int xk = k0 + 8 * xc;
    const bool xok = xk < d_in;
    u32x4 xv[kXL];
#pragma unroll
    for (int j = 0; j < kXL; ++j) {
        const int rr = s_row[xr0 + kXR * j];
        xv[j] = ld128(x + (int64_t)(rr >= 0 ? rr : 0) * d_in + (xok ? xk : 0));
    }

    const int nU = uniform(s_nU);
    const int NB = (nU * RPAD + 31) / 32;
    const int G = NB < 4 ? NB : 4;  // blocks in flight
    const int P = 4 / G;            // waves per block (1 when G == 3)
    const int w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const int gw = w % G, kp = w / G;
    const int nmy = kKC / P;        // chunks per wave: chunk kp + P i

    // MFMA step s2 of chunk kc takes, in half-wave h, the 8-wide k group
    // kq = (k0 + 64 kc) / 8 + 2 s2 + h: the two halves read adjacent groups, so
    // in the packed A layout one load covers contiguous runs of 32 bytes x rank.
    const int nq = d_in / 8;
    const int64_t qstride = PK ? 8 * r : 8;  // elements from group kq to kq + 1
    // A group past d_in loads a clamped address and is replaced by zeros where
    // the MFMA takes it: a select right after the load would wait for it.
    auto load_a = [&](u32x4 (&dst)[4], const uint16_t* abase, int kc) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const int kq = k0 / 8 + 8 * kc + 2 * s2 + h;
            dst[s2] = ld128(abase + (kq < nq ? kq : nq - 1) * qstride);
        }
    };
    // first element of this lane's (expert, rank) row in A (row start) or in
    // the packed A (its 8 values of group 0)
    auto a_row = [&](int blk, int& u, int& rho) {
        const int nn = blk * 32 + n;
        u = nn / RPAD;
        rho = nn % RPAD;
        const bool ok = u < nU && rho < r;
        const int64_t e = ok ? s_U[u] : 0, rr = ok ? rho : 0;
        return PK ? A + e * r * d_in + rr * 8 : A + (e * r + rr) * d_in;
    };
    auto mma = [&](const u32x4 (&ab)[4], int kc, f32x16 (&acc)[kTM]) {
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) {
            const bool in = k0 / 8 + 8 * kc + 2 * s2 + h < nq;
            const u32x4 av = in ? ab[s2] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
            for (int j = 0; j < kTM; ++j) {
                const u32x4 xo = *(const u32x4*)(s_x + x_off(32 * j + n, 8 * kc + 2 * s2 + h));
                acc[j] = mfma32(xo, av, acc[j]);
            }
        }
    };
    auto store_v = [&](const f32x16 (&acc)[kTM], int u, int rho) {
        if (u >= nU || rho >= r) return;
        const int e = s_U[u];
#pragma unroll
        for (int j = 0; j < kTM; ++j)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int m = 32 * j + 8 * (i >> 2) + 4 * h + (i & 3);
                if (s_row[m] < 0) continue;
                float* vp = v + ((int64_t)(tile0 * 32 + m) * 2) * RPAD + rho;
                if (s_e0[m] == e) gst(vp, acc[j][i]);
                if (s_e1[m] == e) gst(vp + RPAD, acc[j][i]);
            }
    };

    // first block's A: its first chunks are in flight while x lands in LDS
    u32x4 ab[kShrinkRing][4];
    int u, rho;
    const uint16_t* arow = a_row(gw, u, rho);
    const bool act = kp < P;
#pragma unroll
    for (int j = 0; j < kShrinkRing; ++j)
        if (act && j < nmy) load_a(ab[j], arow, kp + P * j);

#pragma unroll
    for (int j = 0; j < kXL; ++j) {
        const u32x4 val = xok ? xv[j] : u32x4{0u, 0u, 0u, 0u};
        *(u32x4*)(s_x + x_off(xr0 + kXR * j, xc)) = val;
    }
    __syncthreads();

    // K loop of one block over this wave's chunks, A kShrinkRing chunks ahead
    auto run_block = [&](f32x16 (&acc)[kTM]) {
#pragma unroll 1
        for (int i = 0; i < nmy; i += kShrinkRing) {
#pragma unroll
            for (int j = 0; j < kShrinkRing; ++j) {
                if (i + j < nmy) {
                    mma(ab[j], kp + P * (i + j), acc);
                    if (i + j + kShrinkRing < nmy) load_a(ab[j], arow, kp + P * (i + j + kShrinkRing));
                }
            }
        }
    };

    if (P == 1) {
        if (!act) return;
        for (int blk = gw; blk < NB; blk += G) {
            if (blk != gw) {
                arow = a_row(blk, u, rho);
#pragma unroll
                for (int j = 0; j < kShrinkRing; ++j)
                    if (j < nmy) load_a(ab[j], arow, j);
            }
            f32x16 acc[kTM];
#pragma unroll
            for (int j = 0; j < kTM; ++j) acc[j] = f32x16{};
            run_block(acc);
            store_v(acc, u, rho);
        }
        return;
    }
    // one block per group of P waves: parts 1..P-1 go through LDS (the x
    // slice is no longer read) and the part-0 wave adds them in order
    f32x16 acc[kTM];
#pragma unroll
    for (int j = 0; j < kTM; ++j) acc[j] = f32x16{};
    run_block(acc);
    __syncthreads();
    f32x4* red = (f32x4*)s_x;  // [wave][tile][4][lane]
    static_assert(4 * kTM * 4 * kWave * 16 <= kXRows * kSgmmKSlice * 2, "reduction fits the x slice");
    if (kp > 0) {
#pragma unroll
        for (int j = 0; j < kTM; ++j)
#pragma unroll
            for (int q = 0; q < 4; ++q)
                red[((w * kTM + j) * 4 + q) * kWave + lane] =
                    f32x4{acc[j][4 * q], acc[j][4 * q + 1], acc[j][4 * q + 2], acc[j][4 * q + 3]};
    }
    __syncthreads();
    if (kp == 0) {
        for (int p = 1; p < P; ++p) {
            const int wp = gw + p * G;
#pragma unroll
            for (int j = 0; j < kTM; ++j)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const f32x4 o = red[((wp * kTM + j) * 4 + q) * kWave + lane];
#pragma unroll
                    for (int c = 0; c < 4; ++c) acc[j][4 * q + c] += o[c];
                }
        }
        store_v(acc, u, rho);
    }
}

// ---- expand (bf16, MFMA) -----------------------------------------------------

__device__ __forceinline__ int perm_col(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

// Columns of one expand work item: 4 waves x kEB blocks x 64 columns.
constexpr int kEB = 4;
constexpr int kECols = 4 * kEB * 64;
static_assert(kECols == kSgmmExpandCols, "expand column group");
// The row-side MFMA operands (u = s*g*v as hi + lo bf16, per (expert, 16-rank
// chunk) pair q and lane) are the same for the four waves of a work item: they
// are built once into LDS when the tile's union has at most kQLds pairs; larger
// unions rebuild them per column block in registers.
constexpr int kQLds = 16;

template <int R16, bool RVEC>
__global__ __launch_bounds__(256) void sgmm_expand_bf16(SgmmArgs a, int64_t per_xcd) {
    constexpr int RPAD = R16 * 16;
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    const int64_t bid = blockIdx.x;
    const int64_t t = (bid & 7) * per_xcd + (bid >> 3);
    if (t >= a.n_expand_units) return;
    // work item = (problem, kECols-column group, tile) with the tile fastest:
    // neighbouring work items (same XCD) reuse the same B column slices.  A
    // problem's first item is a multiple of the tile count, so the tile is
    // known before the problem's descriptor.
    const int64_t nt = a.L.tiles_max;
    const int tile = (int)(t % nt);
    const int32_t* perm = (const int32_t*)(a.ws + a.L.perm);
    const uint32_t* epk = (const uint32_t*)(a.ws + a.L.epk);
    const float* gpk = (const float*)(a.ws + a.L.gpk);
    const uint32_t* tmask = (const uint32_t*)(a.ws + a.L.tmask);
    const int tid = threadIdx.x;
    const int w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const int lr = lane >> 3, lc = lane & 7;
    // every load whose address does not depend on another load goes out
    // first: the header words, the owner of the column group, the tile's rows
    // (row-major lane map: instruction i holds row 8i + lr, chunk lc), slots,
    // gates and expert mask
    int yrow[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) yrow[i] = gld(perm + tile * 32 + 8 * i + lr);
    const uint32_t ep = gld(epk + tile * 32 + n);
    const float g0 = gld(gpk + 2 * (tile * 32 + n)), g1 = gld(gpk + 2 * (tile * 32 + n) + 1);
    const uint32_t tm = tid == 0 ? gld(tmask + tile) : 0u;
    const int err = gld(hdr + SG_ERR), n_tiles = gld(hdr + SG_NTILES);
    const int prob = a.descs ? gld(a.cb_owner + t / nt) : 0;
    if (err || tile >= n_tiles) return;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int cg = (int)(t / nt - D.unit0);
    const float* v = (const float*)(a.ws + a.L.v) + D.ks0 * a.L.T_pad * 2 * RPAD;

    __shared__ int s_U[32];
    __shared__ int s_nU;
    __shared__ __attribute__((aligned(16))) uint16_t s_y[4][32 * 64];
    __shared__ __attribute__((aligned(16))) u32x4 s_u[kQLds][2][kWave];

    const int d_out = uniform(D.d_out), r = a.r;
    const int cw = cg * kECols + w * (kEB * 64);  // this wave's first column
    const int nblk = cw >= d_out ? 0 : ((d_out - cw + 63) / 64 < kEB ? (d_out - cw + 63) / 64 : kEB);
    const uint16_t* __restrict__ B = (const uint16_t*)D.B;
    uint16_t* __restrict__ y = (uint16_t*)D.y;
    uint16_t* ys = s_y[w];
    auto load_y = [&](u32x4 (&yv)[4], int blk) {
        const int col = cw + blk * 64 + 8 * lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const bool ok = yrow[i] >= 0 && col < d_out;
            yv[i] = ld128(y + (ok ? (int64_t)yrow[i] * d_out + col : 0));
        }
    };
    u32x4 ycur[4], ynxt[4];
    if (nblk > 0) load_y(ycur, 0);
    if (tid == 0) s_nU = mask_list(tm, s_U);
    __syncthreads();
    const int nU = uniform(s_nU);

    // this lane's tile row (MFMA N index n): its two slots and gates (a padding
    // position has two empty slots)
    const int e0 = (int16_t)(ep & 0xffffu), e1 = (int16_t)(ep >> 16);
    const float c0 = a.scale * g0;
    const float c1 = a.scale * g1;
    const float* v0 = v + ((int64_t)(tile * 32 + n) * 2) * RPAD;
    const float* v1 = v0 + RPAD;
    // row-side operand of (expert U[q / R16], ranks 16(q % R16) + 8h + [0,8)):
    // u = s*g*v as hi + lo bf16 (v = the K slices' sum, kept in slice 0).  v of a slot that is not this expert, or of a
    // padding rank, is never written: it is selected away, not multiplied by 0.
    auto make_u = [&](int q, u32x4& bhi, u32x4& blo) {
        const int e = s_U[q / R16];
        const int rho0 = (q % R16) * 16 + 8 * h;
        const bool m0 = (e0 == e), m1 = (e1 == e);
        const u32x4 p0 = ld128(v0 + rho0), p1 = ld128(v0 + rho0 + 4);
        const u32x4 q0 = ld128(v1 + rho0), q1 = ld128(v1 + rho0 + 4);
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

    const int nq = nU * R16;
    const bool shared_u = nq <= kQLds;
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
            if (yrow[i] >= 0 && col < d_out) st128(y + (int64_t)yrow[i] * d_out + col, o);
        }
        if (blk + 1 < nblk) {
#pragma unroll
            for (int i = 0; i < 4; ++i) ycur[i] = ynxt[i];
        }
    }
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

template <int R16>
hipError_t launch_mfma(const SgmmArgs& a, hipStream_t s) {
    const int64_t n_units = a.total_ks * ((a.L.tiles_max + kTM - 1) / kTM);
    const int64_t sh_per_xcd = (n_units + 7) / 8;
    if (a.packed)
        hipLaunchKernelGGL((sgmm_shrink_bf16<R16, true>), dim3((unsigned)(8 * sh_per_xcd)), dim3(256), 0, s,
                           a, n_units, sh_per_xcd);
    else
        hipLaunchKernelGGL((sgmm_shrink_bf16<R16, false>), dim3((unsigned)(8 * sh_per_xcd)), dim3(256), 0, s,
                           a, n_units, sh_per_xcd);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (a.total_ks > a.n_prob) {  // some problem has more than one K slice
        const dim3 gs((unsigned)((a.L.T_pad * 2 * a.L.r_pad / 4 + 255) / 256), (unsigned)a.n_prob);
        hipLaunchKernelGGL(sgmm_vsum_kernel, gs, dim3(256), 0, s, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const int64_t per_xcd = (a.n_expand_units + 7) / 8;
    if (a.r % 8 == 0)
        hipLaunchKernelGGL((sgmm_expand_bf16<R16, true>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, a,
                           per_xcd);
    else
        hipLaunchKernelGGL((sgmm_expand_bf16<R16, false>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, a,
                           per_xcd);
    return hipGetLastError();
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
    if (dtype == 1) {
        const int64_t n_units = a.total_ks * ((a.L.tiles_max + kTM - 1) / kTM);
        return grid_fits(8 * ((n_units + 7) / 8), 256) &&
               grid_fits((a.L.T_pad * 2 * a.L.r_pad / 4 + 255) / 256, 256) &&
               grid_fits(8 * ((a.n_expand_units + 7) / 8), 256);
    }
    return grid_fits((a.L.T_pad * 2 * a.r + 255) / 256, 256) &&
           grid_fits((a.L.T_pad * a.d_out_max + 255) / 256, 256);
}

hipError_t launch_sgmm(const SgmmArgs& a, int dtype, hipStream_t s) {
    if (!sgmm_grids_fit(a, dtype)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(sgmm_segment_kernel, dim3(1), dim3(kSegThreads), 0, s, a.idx, a.g, a.T, a.E,
                       a.ws, a.L);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dtype == 1) {
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
