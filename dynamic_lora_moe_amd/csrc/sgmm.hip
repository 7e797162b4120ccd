// SGMM: batched unmerged adapters for rows carrying different expert sets,
//     y[t] <- round( y[t] + sum_k s*g[t][k] * B_{e_k} (A_{e_k} x[t]) ).
// The AdaFuse digest (section 2-na) names its core kernel SGMM, "segmented
// gather matrix multiplication"; this is the batched form of the same adapters.
//
// Three launches:
//   segment  (one workgroup) every row gets the key of its unordered expert
//            pair; a stable counting sort lists the rows by key (perm), so
//            rows sharing experts sit next to each other.  The sorted list is
//            cut into 32-row tiles and each tile records the union of the
//            experts its rows use (a bitmask).  Rows with two empty slots are
//            left out.  The same segmentation serves every problem of a
//            grouped call (one routing decision per token for all layers).
//   shrink   per (tile, problem): v = x_rows A_U^T for the tile's experts U,
//            bf16 MFMA 32x32x16 with M = tile rows (gathered through perm),
//            N = (expert, rank), K = d_in split over the four waves and summed
//            in a fixed order; each row keeps the fp32 v of its own two slots.
//   expand   per (tile, 256 output columns, problem): y_rows += u B_U^T with
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

namespace dlm {

static size_t a256(size_t v) { return (v + 255) & ~(size_t)255; }

SgLayout sgmm_layout(int64_t T, int E, int r, int n_prob) {
    SgLayout L;
    L.T = T;
    L.T_pad = ((T > 0 ? T : 1) + 31) / 32 * 32;
    L.n_chunks = (T + 63) / 64;
    if (L.n_chunks < 1) L.n_chunks = 1;
    L.n_keys = (int64_t)(E + 1) * (E + 1);
    L.tiles_max = L.T_pad / 32;
    L.r_pad = (r + 15) / 16 * 16;
    size_t o = 0;
    L.hdr = o;   o += 256;
    L.perm = o;  o += a256((size_t)L.T_pad * 4);
    L.rank = o;  o += a256((size_t)(T > 0 ? T : 1) * 4);
    L.key = o;   o += a256((size_t)(T > 0 ? T : 1) * 4);
    L.hist = o;  o += a256((size_t)L.n_chunks * L.n_keys * 4);
    L.tmask = o; o += a256((size_t)L.tiles_max * 4);
    L.v = o;     o += a256((size_t)n_prob * L.T_pad * 2 * L.r_pad * 4);
    L.total = o;
    return L;
}

namespace {

constexpr int kSegThreads = 1024;

// ---- segment ---------------------------------------------------------------

__global__ __launch_bounds__(kSegThreads) void sgmm_segment_kernel(
    const int32_t* __restrict__ idx, const float* __restrict__ g, int64_t T, int E, char* ws,
    SgLayout L) {
    int32_t* hdr = (int32_t*)(ws + L.hdr);
    int32_t* perm = (int32_t*)(ws + L.perm);
    int32_t* rank = (int32_t*)(ws + L.rank);
    int32_t* key = (int32_t*)(ws + L.key);
    int32_t* hist = (int32_t*)(ws + L.hist);
    uint32_t* tmask = (uint32_t*)(ws + L.tmask);
    __shared__ int s_err;
    __shared__ int s_sum[kSegThreads];
    const int tid = threadIdx.x, lane = lane_id(), w = wave_id();
    const int nw = kSegThreads / kWave;
    const int64_t nk = L.n_keys, nc = L.n_chunks;
    if (tid == 0) s_err = 0;
    for (int64_t q = tid; q < nc * nk; q += kSegThreads) hist[q] = 0;
    __threadfence_block();
    __syncthreads();

    // 1) keys, per-chunk counts and the rank of each row among the earlier rows
    //    of its 64-row chunk with the same key (wave ballots: stable).
    for (int64_t c = w; c < nc; c += nw) {
        const int64_t t = c * kWave + lane;
        int k = -1;
        if (t < T) {
            const int e0 = idx[2 * t], e1 = idx[2 * t + 1];
            bool bad = e0 < -1 || e0 >= E || e1 < -1 || e1 >= E;
            if (e0 >= 0 && !__builtin_isfinite(g[2 * t])) bad = true;
            if (e1 >= 0 && !__builtin_isfinite(g[2 * t + 1])) bad = true;
            if (bad) s_err = 1;
            const int a = e0 < e1 ? e0 : e1, b = e0 < e1 ? e1 : e0;
            if (!bad && b >= 0) k = (a + 1) * (E + 1) + (b + 1);
            key[t] = k;
        }
        uint64_t todo = __ballot(k >= 0);
        int rk = 0;
        while (todo) {
            const int leader = __ffsll((unsigned long long)todo) - 1;
            const int lk = __shfl(k, leader, kWave);
            const uint64_t same = __ballot(k == lk) & todo;
            if (k == lk) rk = __popcll(same & ((1ull << lane) - 1ull));
            if (lane == leader) hist[c * nk + lk] = __popcll(same);
            todo &= ~same;
        }
        if (t < T) rank[t] = rk;
    }
    __threadfence_block();
    __syncthreads();

    // 2) exclusive scan of the counts in (key, chunk) order: the start of each
    //    key's segment, and within it of each chunk's rows.
    const int64_t N = nk * nc;
    const int64_t per = (N + kSegThreads - 1) / kSegThreads;
    const int64_t q0 = tid * per, q1 = (q0 + per < N) ? q0 + per : N;
    int run = 0;
    for (int64_t q = q0; q < q1; ++q) run += hist[(q % nc) * nk + q / nc];
    s_sum[tid] = run;
    __syncthreads();
    for (int off = 1; off < kSegThreads; off <<= 1) {
        const int v = tid >= off ? s_sum[tid - off] : 0;
        __syncthreads();
        s_sum[tid] += v;
        __syncthreads();
    }
    int base = s_sum[tid] - run;
    for (int64_t q = q0; q < q1; ++q) {
        int32_t* p = &hist[(q % nc) * nk + q / nc];
        const int cnt = *p;
        *p = base;
        base += cnt;
    }
    const int n_pos = s_sum[kSegThreads - 1];
    __threadfence_block();
    __syncthreads();

    // 3) scatter rows to their sorted positions.
    for (int64_t t = tid; t < T; t += kSegThreads) {
        const int k = key[t];
        if (k >= 0) perm[hist[(t / kWave) * nk + k] + rank[t]] = (int32_t)t;
    }
    for (int64_t p = n_pos + tid; p < L.T_pad; p += kSegThreads) perm[p] = -1;
    __threadfence_block();
    __syncthreads();

    // 4) 32-row tiles and the experts each one uses.
    const int n_tiles = s_err ? 0 : (n_pos + 31) / 32;
    for (int64_t tl = tid; tl < n_tiles; tl += kSegThreads) {
        uint32_t m = 0;
        for (int j = 0; j < 32; ++j) {
            const int t = perm[tl * 32 + j];
            if (t < 0) continue;
            const int e0 = idx[2 * (int64_t)t], e1 = idx[2 * (int64_t)t + 1];
            if (e0 >= 0) m |= 1u << e0;
            if (e1 >= 0) m |= 1u << e1;
        }
        tmask[tl] = m;
    }
    if (tid == 0) {
        hdr[SG_ERR] = s_err;
        hdr[SG_NPOS] = s_err ? 0 : n_pos;
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

__device__ __forceinline__ int find_prob(const SgDesc* __restrict__ d, int n, int64_t u) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (d[mid].unit0 <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// ---- shrink (bf16, MFMA) -----------------------------------------------------

// N blocks (32 columns of (expert, rank)) accumulated per pass over K.
constexpr int kNBG = 2;

template <int R16>
__global__ __launch_bounds__(256) void sgmm_shrink_bf16(SgmmArgs a) {
    constexpr int RPAD = R16 * 16;
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    if (gld(hdr + SG_ERR)) return;
    const int tile = blockIdx.x;
    if (tile >= gld(hdr + SG_NTILES)) return;
    const int prob = blockIdx.y;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int32_t* perm = (const int32_t*)(a.ws + a.L.perm);
    const uint32_t* tmask = (const uint32_t*)(a.ws + a.L.tmask);
    float* v = (float*)(a.ws + a.L.v) + (int64_t)prob * a.L.T_pad * 2 * RPAD;

    __shared__ int s_U[32];
    __shared__ int s_nU;
    __shared__ int s_row[32], s_e0[32], s_e1[32];
    __shared__ float s_red[3][kWave][16];
    const int tid = threadIdx.x;
    if (tid < 32) {
        const int row = gld(perm + tile * 32 + tid);
        s_row[tid] = row;
        s_e0[tid] = row >= 0 ? gld(a.idx + 2 * (int64_t)row) : -1;
        s_e1[tid] = row >= 0 ? gld(a.idx + 2 * (int64_t)row + 1) : -1;
    }
    if (tid == 0) s_nU = mask_list(gld(tmask + tile), s_U);
    __syncthreads();

    const int nU = s_nU;
    const int NB = (nU * RPAD + 31) / 32;
    const int w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const int d_in = D.d_in, r = a.r;
    const uint16_t* __restrict__ x = (const uint16_t*)D.x;
    const uint16_t* __restrict__ A = (const uint16_t*)D.A;
    const int xrow = s_row[n];
    const uint16_t* xr = xrow >= 0 ? x + (int64_t)xrow * d_in : nullptr;
    const int n_kc = (d_in + 63) / 64;

    for (int g0 = 0; g0 < NB; g0 += kNBG) {
        const int nbg = NB - g0 < kNBG ? NB - g0 : kNBG;
        // lane's column of each N block: (expert U[u], rank rho)
        const uint16_t* arow[kNBG];
#pragma unroll
        for (int j = 0; j < kNBG; ++j) {
            const int nn = (g0 + j) * 32 + n;
            const int u = nn / RPAD, rho = nn % RPAD;
            arow[j] = (j < nbg && u < nU && rho < r) ? A + ((int64_t)s_U[u] * r + rho) * d_in : nullptr;
        }
        f32x16 acc[kNBG];
#pragma unroll
        for (int j = 0; j < kNBG; ++j) acc[j] = f32x16{};
        // K: 64-wide chunks, wave w takes chunks w, w+4, ...; inside a chunk the
        // half-wave h covers k in [32h, 32h+32) as four 8-wide MFMA k-steps, so
        // each lane reads 64 contiguous bytes of x and of each A row.
        for (int kc = w; kc < n_kc; kc += 4) {
            const int k0 = kc * 64 + 32 * h;
            u32x4 xo[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int col = k0 + 8 * s;
                xo[s] = (xr && col < d_in) ? ld128(xr + col) : u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int j = 0; j < kNBG; ++j) {
                if (j >= nbg) break;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int col = k0 + 8 * s;
                    const u32x4 ao = (arow[j] && col < d_in) ? ld128(arow[j] + col) : u32x4{0u, 0u, 0u, 0u};
                    acc[j] = mfma32(xo[s], ao, acc[j]);
                }
            }
        }
        // fixed-order sum of the four waves' partial products, one block at a time
#pragma unroll
        for (int j = 0; j < kNBG; ++j) {
            if (j >= nbg) break;
            if (w > 0) {
#pragma unroll
                for (int i = 0; i < 16; ++i) s_red[w - 1][lane][i] = acc[j][i];
            }
            __syncthreads();
            if (w == 0) {
                const int nn = (g0 + j) * 32 + n;
                const int u = nn / RPAD, rho = nn % RPAD;
                if (u < nU && rho < r) {
                    const int e = s_U[u];
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const float val = ((acc[j][i] + s_red[0][lane][i]) + s_red[1][lane][i]) + s_red[2][lane][i];
                        const int m = 8 * (i >> 2) + 4 * h + (i & 3);
                        if (s_row[m] < 0) continue;
                        float* vp = v + ((int64_t)(tile * 32 + m) * 2) * RPAD + rho;
                        if (s_e0[m] == e) gst(vp, val);
                        if (s_e1[m] == e) gst(vp + RPAD, val);
                    }
                }
            }
            __syncthreads();
        }
    }
}

// ---- expand (bf16, MFMA) -----------------------------------------------------

__device__ __forceinline__ int perm_col(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

template <int R16>
__global__ __launch_bounds__(256) void sgmm_expand_bf16(SgmmArgs a, int64_t per_xcd) {
    constexpr int RPAD = R16 * 16;
    const int32_t* hdr = (const int32_t*)(a.ws + a.L.hdr);
    if (gld(hdr + SG_ERR)) return;
    const int64_t bid = blockIdx.x;
    const int64_t t = (bid & 7) * per_xcd + (bid >> 3);
    if (t >= a.n_expand_units) return;
    // work item = (tile, problem, 256-column block), tile-major
    const int tile = (int)(t / a.total_cb);
    if (tile >= gld(hdr + SG_NTILES)) return;
    const int64_t rem = t - (int64_t)tile * a.total_cb;
    const int prob = a.descs ? find_prob(a.descs, a.n_prob, rem) : 0;
    const SgDesc D = a.descs ? a.descs[prob] : a.single;
    const int cb = (int)(rem - D.unit0);
    const int32_t* perm = (const int32_t*)(a.ws + a.L.perm);
    const uint32_t* tmask = (const uint32_t*)(a.ws + a.L.tmask);
    const float* v = (const float*)(a.ws + a.L.v) + (int64_t)prob * a.L.T_pad * 2 * RPAD;

    __shared__ int s_U[32];
    __shared__ int s_nU;
    const int tid = threadIdx.x;
    if (tid == 0) s_nU = mask_list(gld(tmask + tile), s_U);
    __syncthreads();

    const int w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const int d_out = D.d_out, r = a.r;
    const int cw = cb * 256 + w * 64;  // this wave's 64 output columns
    if (cw >= d_out) return;
    const int nU = s_nU;
    const uint16_t* __restrict__ B = (const uint16_t*)D.B;
    uint16_t* __restrict__ y = (uint16_t*)D.y;

    // this lane's row (MFMA N index = tile row n) and its two slots
    const int row = gld(perm + tile * 32 + n);
    int e0 = -1, e1 = -1;
    float c0 = 0.f, c1 = 0.f;
    if (row >= 0) {
        e0 = gld(a.idx + 2 * (int64_t)row);
        e1 = gld(a.idx + 2 * (int64_t)row + 1);
        c0 = e0 >= 0 ? a.scale * gld(a.g + 2 * (int64_t)row) : 0.f;
        c1 = e1 >= 0 ? a.scale * gld(a.g + 2 * (int64_t)row + 1) : 0.f;
    }
    const float* v0 = v + ((int64_t)(tile * 32 + n) * 2) * RPAD;
    const float* v1 = v0 + RPAD;

    // the lane's two output-column rows of B for each 32-column block
    int ocol[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) ocol[b] = cw + 32 * b + perm_col(n);

    f32x16 acc[2] = {f32x16{}, f32x16{}};
    for (int u = 0; u < nU; ++u) {
        const int e = s_U[u];
        const bool m0 = (e0 == e), m1 = (e1 == e);
#pragma unroll
        for (int rc = 0; rc < R16; ++rc) {
            const int rho0 = rc * 16 + 8 * h;
            // u = s*g*v for this row, expert e, ranks rho0..rho0+7, as hi + lo bf16
            // ranks beyond r are padding: v there was never written, keep u at 0
            float uv[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) uv[j] = 0.f;
            if (m0) {
                const u32x4 p0 = ld128(v0 + rho0), p1 = ld128(v0 + rho0 + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (rho0 + j < r) uv[j] = c0 * __uint_as_float(j < 4 ? p0[j] : p1[j - 4]);
            }
            if (m1) {
                const u32x4 p0 = ld128(v1 + rho0), p1 = ld128(v1 + rho0 + 4);
#pragma unroll
                for (int j = 0; j < 8; ++j)
                    if (rho0 + j < r) uv[j] = fmaf(c1, __uint_as_float(j < 4 ? p0[j] : p1[j - 4]), uv[j]);
            }
            uint32_t hw[4], lw[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a0 = uv[2 * j], a1 = uv[2 * j + 1];
                hw[j] = pack2_bf16(a0, a1);
                lw[j] = pack2_bf16(a0 - bf_lo(hw[j]), a1 - bf_hi(hw[j]));
            }
            const u32x4 bhi = {hw[0], hw[1], hw[2], hw[3]};
            const u32x4 blo = {lw[0], lw[1], lw[2], lw[3]};
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                u32x4 ao = {0u, 0u, 0u, 0u};
                if (ocol[b] < d_out && rho0 < r) {
                    const uint16_t* bp = B + ((int64_t)e * d_out + ocol[b]) * r + rho0;
                    if ((r & 7) == 0) {
                        ao = ld128(bp);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t lo = (rho0 + 2 * j < r) ? gld(bp + 2 * j) : 0u;
                            const uint32_t hi = (rho0 + 2 * j + 1 < r) ? gld(bp + 2 * j + 1) : 0u;
                            ao[j] = lo | (hi << 16);
                        }
                    }
                }
                acc[b] = mfma32(ao, bhi, acc[b]);
                acc[b] = mfma32(ao, blo, acc[b]);
            }
        }
    }
    if (row < 0) return;
    uint16_t* yr = y + (int64_t)row * d_out;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const int col = cw + 32 * b + 16 * h + 8 * q;
            if (col >= d_out) continue;
            const u32x4 yv = ld128(yr + col);
            uint32_t ow[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                const int i = 8 * q + 2 * p;
                ow[p] = pack2_bf16(bf_lo(yv[p]) + acc[b][i], bf_hi(yv[p]) + acc[b][i + 1]);
            }
            st128(yr + col, u32x4{ow[0], ow[1], ow[2], ow[3]});
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
    float* v = (float*)(a.ws + a.L.v) + (int64_t)prob * a.L.T_pad * 2 * RPAD;
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
    const float* v = (const float*)(a.ws + a.L.v) + (int64_t)prob * a.L.T_pad * 2 * RPAD;
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

template <int R16>
hipError_t launch_mfma(const SgmmArgs& a, hipStream_t s) {
    hipLaunchKernelGGL((sgmm_shrink_bf16<R16>), dim3((unsigned)a.L.tiles_max, (unsigned)a.n_prob),
                       dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t per_xcd = (a.n_expand_units + 7) / 8;
    hipLaunchKernelGGL((sgmm_expand_bf16<R16>), dim3((unsigned)(8 * per_xcd)), dim3(256), 0, s, a,
                       per_xcd);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_sgmm(const SgmmArgs& a, int dtype, hipStream_t s) {
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
