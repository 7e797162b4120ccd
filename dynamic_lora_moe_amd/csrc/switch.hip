// Fused adapter switch (AdaFuse digest, section 2-na "fused adapter
// switching"): one launch removes the previous token's gated adapters from
// every adapted weight of every layer and merges the current token's, in
// place:
//     W <- round( W - s*sum_old g_k B_k A_k + s*sum_new g_k B_k A_k ).
// The pages do this with concatenated adapter matrices and a parallel GEMM
// inside one kernel, updating the backbone in place and hiding load latency
// with a prefetch buffer.
//
// gfx950 design (bf16 path):
//   * The switch is a stream over W (read once, written once, 4 bytes per
//     element) with 4r MACs per element: HBM-bound, with the delta on MFMA.
//   * Work unit = a 256-row x CT-column tile of one weight (ranks 17..64 use
//     the wide tiles below instead).  Tiles of all L*P
//     weights form one launch; a workgroup finds its weight by binary search in
//     the device descriptor table.  Consecutive tiles go to the same XCD so each
//     XCD streams a contiguous band of W and its L2 keeps the band's slices.
//   * The four slots [new0, new1, old0, old1] are the concatenated K = 4r
//     contraction.  Their A column slices for the tile are staged once in LDS,
//     transposed to [column][rank] so a lane reads its 8 MFMA k-values with one
//     16-byte LDS read.  B row slices are already k-contiguous and go straight
//     from global memory into MFMA operand registers.
//   * The MFMA runs "transposed": M = W columns, N = W rows.  With the columns
//     of each 32-column block permuted (perm_row below) the accumulator of
//     lane l holds 16 consecutive columns of row l%32.  W itself is read and
//     written row-major (8 rows x 128 bytes per wave instruction, coalesced)
//     and passes through a per-wave swizzled LDS block into and out of that
//     MFMA layout.
//   * Each slot has its own fp32 accumulator chain (K = r).  The epilogue
//     forms S_new = c1*P1 + c0*P0 and S_old the same way (one fma each), then
//     W - (S_old - S_new) in fp32 and one RNE to bf16.  Identical expressions
//     for both halves make a switch to the same set an exact no-op; each set's
//     slots are put in a canonical order first so slot order cannot matter.
//   * W is read and written with the nontemporal cache policy (touched once),
//     so the A/B slices the tiles share stay in L2: measured 1-2% faster on
//     the switches and 10% on the merged-weight product.
#include <type_traits>

#include "gfx950.hpp"
#include "internal.hpp"

namespace dlm {

// Wide tiles (ranks 17..64): 64-column sub-bands per tile (4096 columns:
// measured 74.6 / 72.2 / 70.5 ms per 70B-shaped switch for 16 / 32 / 64),
// waves = 32-row groups per workgroup, row bands per tile group.
constexpr int kWideSB = 64;
constexpr int kWW = 8;
constexpr int kWRT = kWW * 32;
constexpr int kWGroup = 8;

SwTile switch_tile_for_rank(int r) {
    SwTile t;
    t.r16 = (r + 15) / 16;
    t.ct = t.r16 <= 1 ? 256 : (t.r16 <= 4 ? 64 * kWideSB : 64);
    t.rt = (t.r16 >= 2 && t.r16 <= 4) ? kWRT : 256;
    return t;
}

namespace {

constexpr int kWaves = 4;
constexpr int kRowGroups = 2;  // 32-row groups per wave
constexpr int kRT = kWaves * kRowGroups * 32;

struct Sets {
    int e[4];    // experts of [new0, new1, old0, old1]; -1 = empty
    float c[4];  // s * g of each slot (0 for an empty slot)
    bool ok;
};

// The two sets' raw words (an absent set reads as both slots empty).
struct SetWords {
    int e[4];
    float g[4];
};

__device__ __forceinline__ SetWords load_sets(const SwitchArgs& a) {
    SetWords w;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int32_t* ip = h == 0 ? a.new_idx : a.old_idx;
        const float* gp = h == 0 ? a.new_g : a.old_g;
        w.e[2 * h] = w.e[2 * h + 1] = -1;
        w.g[2 * h] = w.g[2 * h + 1] = 0.f;
        if (ip != nullptr) {
            w.e[2 * h] = ip[0];
            w.e[2 * h + 1] = ip[1];
            w.g[2 * h] = gp[0];
            w.g[2 * h + 1] = gp[1];
        }
    }
    return w;
}

// Validates both sets (every thread reads the same words, so every decision
// below is uniform) and orders each set's two slots canonically by (expert,
// coefficient).
__device__ __forceinline__ Sets check_sets(const SwitchArgs& a, const SetWords& w) {
    Sets s;
    s.ok = true;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        int e0 = w.e[2 * h], e1 = w.e[2 * h + 1];
        float c0 = 0.f, c1 = 0.f;
        {
            const float g0 = w.g[2 * h], g1 = w.g[2 * h + 1];
            if (e0 < -1 || e0 >= a.E || e1 < -1 || e1 >= a.E) s.ok = false;
            if (e0 >= 0 && !__builtin_isfinite(g0)) s.ok = false;
            if (e1 >= 0 && !__builtin_isfinite(g1)) s.ok = false;
            c0 = e0 >= 0 ? a.scale * g0 : 0.f;
            c1 = e1 >= 0 ? a.scale * g1 : 0.f;
            if (e1 < e0 || (e1 == e0 && c1 < c0)) {
                const int te = e0; e0 = e1; e1 = te;
                const float tc = c0; c0 = c1; c1 = tc;
            }
        }
        s.e[2 * h] = e0;
        s.e[2 * h + 1] = e1;
        s.c[2 * h] = c0;
        s.c[2 * h + 1] = c1;
    }
    return s;
}

// Reads both sets from device memory and validates them.
__device__ __forceinline__ Sets read_sets(const SwitchArgs& a) { return check_sets(a, load_sets(a)); }

// Which prefix a launch's work units are numbered by.
enum { kKeyElem = 0, kKeyTile = 1, kKeyRowBlock = 2, kKeyBand = 3, kKeyKSlice = 4 };

template <int K>
__device__ __forceinline__ int64_t desc_key(const SwDesc& d) {
    return K == kKeyElem ? d.elem0
                         : (K == kKeyTile ? d.tile0 : (K == kKeyRowBlock ? d.rb0 : (K == kKeyBand ? d.rt0 : d.ks0)));
}

template <int K>
__device__ __forceinline__ int find_desc(const SwDesc* __restrict__ d, int n, int64_t u) {
    int lo = 0, hi = n - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (desc_key<K>(d[mid]) <= u) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Column cc (0..31) of a 32-column block -> the MFMA row index m that carries it.
// With this order, accumulator register a of lane l holds column 16*(l/32) + a.
__device__ __forceinline__ int perm_row(int cc) { return 8 * ((cc >> 2) & 3) + 4 * (cc >> 4) + (cc & 3); }

// LDS layouts.
//  A slices: As[slot][cb][m][RPAD] bf16, one row per MFMA row index m (one W
//    column), RPAD ranks.  The 16-byte chunks of a row are XOR-swizzled so the
//    8 lanes of each ds_read_b128 phase hit 8 different bank groups.
//  W scratch: one 32-row x 64-column bf16 block per wave (4 KB), rows of eight
//    16-byte chunks, chunk index XOR (row & 7): both the row-major (global)
//    and the MFMA-layout accesses are conflict-free.
template <int R16>
__device__ __forceinline__ int a_chunk_swz(int m, int c) {
    constexpr int P = 2 * R16;                            // chunks per row
    constexpr int G = (P % 8 == 0) ? 8 : (P % 4 == 0 ? 4 : 2);  // gcd(P, 8)
    constexpr int PER = 8 / G;
    return c ^ ((m / PER) % G);
}
__device__ __forceinline__ int w_off(int row, int chunk) {  // bf16 element offset
    return row * 64 + ((chunk ^ (row & 7)) << 3);
}

// One 256-row x CT-column tile.  FULL = every row, column and rank of the tile
// is in range (all tiles of model-sized weights): then no load or store carries
// a guard, so the compiler issues them back to back instead of branching
// around each one.  Edge tiles run the guarded instance.
//
// GEMV = also form the tile's share of y = W' x (the fused switch + product):
// every lane multiplies its 16 new (rounded) weights of a 32-column block with
// the matching x values, in column order, and adds them to a running sum over
// the tile's columns; the two half-waves' sums of a row are then added (lower
// half first) and stored as the tile's partial product of that row.  Xs holds
// the tile's CT x values (zero past d_in).
template <int R16, int CT, bool FULL, bool GEMV = false>
__device__ __forceinline__ void switch_tile(const SwitchArgs& a, const Sets& sc, const SwDesc& D,
                                            int row_base, int col_base, uint16_t* As, uint16_t* Ws,
                                            const uint16_t* Xs = nullptr) {
    constexpr int RPAD = R16 * 16;
    constexpr int NCB = CT / 32;   // 32-column MFMA blocks per tile
    constexpr int NSUB = CT / 64;  // 64-column steps per row group
    constexpr int U = kRowGroups * NSUB;  // (row group, step) units per wave
    constexpr int SLOT_ELEMS = NCB * 32 * RPAD;
    constexpr int CHUNKS = CT / 8;  // 16-byte chunks per rank row of the A slice
    constexpr int NQ = RPAD * CHUNKS;
    constexpr int NSTAGE = (NQ + kWaves * kWave - 1) / (kWaves * kWave);
    const int d_out = D.d_out, d_in = D.d_in, r = a.r;
    const uint16_t* __restrict__ Ab = (const uint16_t*)D.A;
    const uint16_t* __restrict__ Bb = (const uint16_t*)D.B;
    uint16_t* __restrict__ W = (uint16_t*)D.W;
    const int tid = threadIdx.x, w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const bool act[4] = {sc.e[0] >= 0, sc.e[1] >= 0, sc.e[2] >= 0, sc.e[3] >= 0};
    const bool r_vec = (r & 7) == 0;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    uint16_t* ws = Ws + w * (32 * 64);  // this wave's W scratch
    // row-major lane map of a 32x64 block: instruction i covers rows 8i + lane/8,
    // lane%8 is the 16-byte chunk within the 128-byte row segment
    const int lr = lane >> 3, lc = lane & 7;

    // 1) A column slices of the active slots: issue every load first.
    u32x4 av[4][NSTAGE];
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
#pragma unroll
        for (int i = 0; i < NSTAGE; ++i) {
            const int q = tid + i * kWaves * kWave;
            const int rho = q / CHUNKS, col = col_base + (q % CHUNKS) * 8;
            bool ok = act[slot] && (NQ % (kWaves * kWave) == 0 || q < NQ);
            if (!FULL) ok = ok && rho < r && col < d_in;
            av[slot][i] = ok ? ld128(Ab + ((int64_t)sc.e[slot] * r + rho) * d_in + col) : zero;
        }
    }

    // row group g of this wave covers rows row_base + (w*kRowGroups + g)*32 + [0,32)
    auto load_b = [&](u32x4 (&bo)[4][R16], int g) {
        const int row = row_base + (w * kRowGroups + g) * 32 + n;
#pragma unroll
        for (int slot = 0; slot < 4; ++slot)
#pragma unroll
            for (int ks = 0; ks < R16; ++ks) {
                const int rho0 = ks * 16 + 8 * h;
                const uint16_t* bp = Bb + ((int64_t)sc.e[slot] * d_out + row) * r + rho0;
                u32x4 v = zero;
                if (FULL) {
                    if (act[slot]) v = ld128(bp);
                } else if (act[slot] && row < d_out && rho0 < r) {
                    if (r_vec) {
                        v = ld128(bp);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const uint32_t lo = (rho0 + 2 * j < r) ? gld(bp + 2 * j) : 0u;
                            const uint32_t hi = (rho0 + 2 * j + 1 < r) ? gld(bp + 2 * j + 1) : 0u;
                            v[j] = lo | (hi << 16);
                        }
                    }
                }
                bo[slot][ks] = v;
            }
    };
    // unit u = (row group u / NSUB, 64-column step u % NSUB), read row-major:
    // instruction i reads row 8i + lr, columns c0 + 8lc .. +8
    auto load_w = [&](u32x4 (&wv)[4], int u) {
        const int row0 = row_base + (w * kRowGroups + u / NSUB) * 32;
        const int col = col_base + (u % NSUB) * 64 + 8 * lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + 8 * i + lr;
            const uint16_t* p = W + (int64_t)row * d_in + col;
            if (FULL) wv[i] = ld128_nt(p);
            else wv[i] = (row < d_out && col < d_in) ? ld128(p) : zero;
        }
    };

    u32x4 bcur[4][R16];
    u32x4 wcur[4], wnxt[4];
    load_b(bcur, 0);
    load_w(wcur, 0);
    float ysum = 0.f;  // GEMV: this lane's running share of its row's product

    // 2) transpose the A slices into LDS: As[slot][cb][m][rho] = A[e][rho][col(cb, m)]
    //    (an inactive slot's slice too: its loads gave zeros, so the MFMAs below
    //    need no per-slot branch)
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
        uint16_t* dst_slot = As + slot * SLOT_ELEMS;
#pragma unroll
        for (int i = 0; i < NSTAGE; ++i) {
            const int q = tid + i * kWaves * kWave;
            if (NQ % (kWaves * kWave) != 0 && q >= NQ) continue;
            const int rho = q / CHUNKS, ch = q % CHUNKS;
            uint16_t* dst = dst_slot + (ch >> 2) * 32 * RPAD + (rho & 7);
            const int cc0 = (ch & 3) * 8;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int m = perm_row(cc0 + j);
                const uint32_t word = av[slot][i][j >> 1];
                dst[m * RPAD + (a_chunk_swz<R16>(m, rho >> 3) << 3)] =
                    (j & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
            }
        }
    }
    __syncthreads();

    // 3) stream the wave's units: the next unit's W is in flight while the
    //    current unit runs its MFMAs and epilogue; the next row group's B slices
    //    are fetched right after the last MFMA that reads the current ones.
#pragma unroll 1
    for (int u = 0; u < U; ++u) {
        const int g = u / NSUB, sub = u % NSUB;
        if (u + 1 < U) load_w(wnxt, u + 1);
        // row-major registers -> scratch; each block then reads its MFMA layout
        // (row n, chunks 4b + 2h + q) and writes its result back in place
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4*)(ws + w_off(8 * i + lr, lc)) = wcur[i];
#pragma unroll 1
        for (int b = 0; b < 2; ++b) {
            u32x4 wm[2];
#pragma unroll
            for (int q = 0; q < 2; ++q) wm[q] = *(const u32x4*)(ws + w_off(n, 4 * b + 2 * h + q));
            // rank chunk outermost: the four slots' MFMAs of a chunk are
            // independent and issue back to back; each slot sums its chunks in
            // order (an inactive slot multiplies zeros)
            f32x16 P[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
            const uint16_t* ap = As + (sub * 2 + b) * 32 * RPAD + n * RPAD;
#pragma unroll
            for (int ks = 0; ks < R16; ++ks) {
                u32x4 ao[4];
#pragma unroll
                for (int slot = 0; slot < 4; ++slot)
                    ao[slot] = *(const u32x4*)(ap + slot * SLOT_ELEMS + (a_chunk_swz<R16>(n, 2 * ks + h) << 3));
#pragma unroll
                for (int slot = 0; slot < 4; ++slot) P[slot] = mfma32(ao[slot], bcur[slot][ks], P[slot]);
            }
            if (b == 1 && u + 1 < U && (u + 1) % NSUB == 0) load_b(bcur, (u + 1) / NSUB);
            uint32_t ow[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t word = wm[p >> 2][p & 3];
                float o2[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int i = 2 * p + j;
                    const float sn = fmaf(sc.c[1], P[1][i], sc.c[0] * P[0][i]);
                    const float so = fmaf(sc.c[3], P[3][i], sc.c[2] * P[2][i]);
                    const float wf = j ? bf_hi(word) : bf_lo(word);
                    o2[j] = wf - (so - sn);
                }
                ow[p] = pack2_bf16(o2[0], o2[1]);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *(u32x4*)(ws + w_off(n, 4 * b + 2 * h + q)) =
                    u32x4{ow[4 * q], ow[4 * q + 1], ow[4 * q + 2], ow[4 * q + 3]};
            if constexpr (GEMV) {
                // columns 32b + 16h + 2p (+1) of this 64-column step hold ow[p]
                const uint16_t* xp = Xs + sub * 64 + 32 * b + 16 * h;
                const u32x4 x0 = *(const u32x4*)xp, x1 = *(const u32x4*)(xp + 8);
#pragma unroll
                for (int p = 0; p < 8; ++p) {
                    const uint32_t xw = p < 4 ? x0[p] : x1[p - 4];
                    ysum = fmaf(bf_lo(ow[p]), bf_lo(xw), ysum);
                    ysum = fmaf(bf_hi(ow[p]), bf_hi(xw), ysum);
                }
            }
        }
        if constexpr (GEMV) {
            if (sub == NSUB - 1) {
                const float other = __shfl_xor(ysum, 32, kWave);
                const int row = row_base + (w * kRowGroups + g) * 32 + n;
                if (h == 0 && (FULL || row < d_out)) gst(D.part + (int64_t)(col_base / CT) * d_out + row, ysum + other);
                ysum = 0.f;
            }
        }
        // scratch -> row-major registers -> global
        const int row0 = row_base + (w * kRowGroups + g) * 32;
        const int col = col_base + sub * 64 + 8 * lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + 8 * i + lr;
            const u32x4 v = *(const u32x4*)(ws + w_off(8 * i + lr, lc));
            if (FULL || (row < d_out && col < d_in)) st128_nt(W + (int64_t)row * d_in + col, v);
        }
        if (u + 1 < U) {
#pragma unroll
            for (int i = 0; i < 4; ++i) wcur[i] = wnxt[i];
        }
    }
}

// Rank 16 fits three waves per SIMD without spilling, ranks up to 96 two, larger
// ranks one.
template <int R16, int CT>
__global__ __launch_bounds__(kWaves* kWave) __attribute__((amdgpu_waves_per_eu(R16 <= 1 ? 3 : (R16 <= 6 ? 2 : 1))))
void switch_bf16_kernel(SwitchArgs a) {
    // [4 slots][CT/32][32][R16*16] A slices, then 4 x [32][64] W scratch
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* As = smem;
    uint16_t* Ws = smem + 4 * (CT / 32) * 32 * (R16 * 16);
    const int64_t bid = blockIdx.x;
    const int64_t t = (bid & 7) * a.per_xcd + (bid >> 3);
    if (t >= a.n_units) return;
    const Sets sc = read_sets(a);
    if (!sc.ok) {
        if (t == 0 && threadIdx.x == 0) *a.err = 1;
        return;
    }
    const SwDesc D = a.descs[find_desc<kKeyTile>(a.descs, a.n_desc, t)];
    const int64_t local = t - D.tile0;
    const int row_base = (int)(local / D.n_ct) * kRT;
    const int col_base = (int)(local % D.n_ct) * CT;
    const bool full = row_base + kRT <= D.d_out && col_base + CT <= D.d_in && a.r == R16 * 16;
    if (full)
        switch_tile<R16, CT, true>(a, sc, D, row_base, col_base, As, Ws);
    else
        switch_tile<R16, CT, false>(a, sc, D, row_base, col_base, As, Ws);
}

// ---- wide tiles for ranks 17..64 -------------------------------------------
//
// At these ranks the A/B slices of a tile are as large as its W, so the
// 256 x CT tiles above spend most of their time waiting for operands.  Here a
// workgroup of 8 waves takes a 256-row x (64 * NSB)-column tile; each wave owns
// one 32-row group and keeps its B rows in registers for the whole tile.  Tiles
// of a weight run in groups of kWGroup row bands, column band by column band,
// so the A slices of a column band and the B rows of the group's row bands are
// reused from L2 instead of re-read from HBM.  The per-slot fp32 products and
// the epilogue are those of switch_tile.
//
// Both operands are staged with direct global -> LDS copies instead of
// through registers, so the copies run well ahead of the MFMAs:
//   * A: the handle keeps every (expert, 64-column block) slice as a packed
//     image already in the LDS layout of switch_tile (zero past r and d_in),
//     so a 64-column sub-band's four slot slices are four contiguous copies (an
//     inactive slot copies the zero image).  Two buffers; the next sub-band's
//     copy is issued right after the barrier that frees its buffer.
//   * W: each wave copies its own 32 x 64 block, row-major and chunk-swizzled
//     (lane L fetches the chunk that belongs at LDS position L), into one of
//     three per-wave buffers, two sub-bands ahead; the result goes back out
//     through the same buffer.  Edge tiles copy from clamped addresses (rows
//     past d_out and columns past d_in are never stored).
// Each wait names the exact number of vector-memory instructions (copies and W
// stores, the only ones issued in the loop) that follow the copy it waits for;
// scheduling barriers keep the compiler from moving any of them across.
constexpr int kWideWBufs = 3;

template <typename T>
__device__ __forceinline__ T pick4(int i, T v0, T v1, T v2, T v3) {
    return i == 0 ? v0 : (i == 1 ? v1 : (i == 2 ? v2 : v3));
}

template <int R16, int NSB, bool FULL>
__device__ __forceinline__ void switch_wide_tile(const SwitchArgs& a, const Sets& sc, const SwDesc& D,
                                                 int row_base, int col_base, uint16_t* smem) {
    constexpr int RPAD = R16 * 16;
    constexpr int SLOT_ELEMS = 2 * 32 * RPAD;        // one slot's image of one sub-band
    constexpr int BUF_ELEMS = 4 * SLOT_ELEMS;
    constexpr int KB = 512;                          // bf16 elements per 1 KB copy instruction
    constexpr int NAI = 4 * SLOT_ELEMS / KB / kWW;   // A copies per wave per sub-band (= R16)
    constexpr int WBLK = 32 * 64;                    // one wave's W block
    constexpr int WBUF = kWW * WBLK;
    static_assert((4 * SLOT_ELEMS / KB) % kWW == 0, "A copies split evenly over the waves");
    uint16_t* As = smem;                              // [2][BUF_ELEMS]
    uint16_t* Wb = smem + 2 * BUF_ELEMS;              // [kWideWBufs][kWW][WBLK]
    const int d_in = D.d_in, d_out = D.d_out, r = a.r;
    const uint16_t* __restrict__ Bb = (const uint16_t*)D.B;
    uint16_t* __restrict__ W = (uint16_t*)D.W;
    const int w = wave_id(), lane = lane_id(), h = lane >> 5, n = lane & 31;
    const int lr = lane >> 3, lc = lane & 7;
    const int row0 = row_base + w * 32;
    const int nsb = FULL ? NSB : uniform((d_in - col_base + 63) / 64 < NSB ? (d_in - col_base + 63) / 64 : NSB);

    // first-sub-band image of each slot; the zero image does not advance
    const int64_t n_cb = (d_in + 63) / 64;
    const uint16_t* img[4];
    int step[4];
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
        const bool on = sc.e[slot] >= 0;
        img[slot] = on ? (const uint16_t*)D.Ap + ((int64_t)sc.e[slot] * n_cb + col_base / 64) * SLOT_ELEMS
                       : (const uint16_t*)a.zimg;
        step[slot] = on ? SLOT_ELEMS : 0;
    }
    auto copy_a = [&](int sb) {
        uint16_t* dst = As + (sb & 1) * BUF_ELEMS;
#pragma unroll
        for (int j = 0; j < NAI; ++j) {
            const int q = j * kWW + w;  // 1 KB piece q of the sub-band's four images
            const int slot = q / (SLOT_ELEMS / KB), piece = q % (SLOT_ELEMS / KB);
            const uint16_t* src = pick4(slot, img[0], img[1], img[2], img[3]) +
                                  (int64_t)sb * pick4(slot, step[0], step[1], step[2], step[3]) + piece * KB;
            copy16_to_lds(src + lane * 8, dst + q * KB);
        }
    };
    auto copy_w = [&](int sb) {
        uint16_t* dst = Wb + (sb % kWideWBufs) * WBUF + w * WBLK;
        int col = col_base + sb * 64 + 8 * (lc ^ lr);
        if (!FULL) col = col < d_in ? col : d_in - 8;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            int row = row0 + 8 * i + lr;
            if (!FULL) row = row < d_out ? row : d_out - 1;
            copy16_to_lds_nt(W + (int64_t)row * d_in + col, dst + i * KB);
        }
    };

    // B rows of the wave's 32 rows.  An inactive slot, and a full-rank tile's
    // every slot, load unconditionally (an inactive slot from the zero image,
    // rows of RPAD there).  The compiler drains the prologue's copies before
    // entering the loop, which uses registers loaded outside it: one latency
    // per tile.
    u32x4 bcur[4][R16];
    {
        const int row = FULL ? row0 + n : (row0 + n < d_out ? row0 + n : d_out - 1);
        const bool r_full = FULL || r == RPAD;
        const bool r_vec = (r & 7) == 0;
#pragma unroll
        for (int slot = 0; slot < 4; ++slot) {
            const bool on = sc.e[slot] >= 0;
            const uint16_t* bp = on ? Bb + ((int64_t)sc.e[slot] * d_out + row) * r + 8 * h
                                    : (const uint16_t*)a.zimg + n * RPAD + 8 * h;
#pragma unroll
            for (int ks = 0; ks < R16; ++ks) {
                const int rho0 = ks * 16 + 8 * h;
                if (r_full || !on) {
                    bcur[slot][ks] = ld128(bp + ks * 16);
                } else if (r_vec) {
                    bcur[slot][ks] = rho0 < r ? ld128(bp + ks * 16) : u32x4{0u, 0u, 0u, 0u};
                } else {
                    u32x4 v;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const uint32_t lo = (rho0 + 2 * j < r) ? gld(bp + ks * 16 + 2 * j) : 0u;
                        const uint32_t hi = (rho0 + 2 * j + 1 < r) ? gld(bp + ks * 16 + 2 * j + 1) : 0u;
                        v[j] = lo | (hi << 16);
                    }
                    bcur[slot][ks] = v;
                }
            }
        }
    }

    // One sub-band: per 32-column half, the MFMAs of slots 0 and 1, then those
    // of slots 2 and 3 while the VALU forms S_new from slots 0 and 1, then the
    // next half's slot-0/1 MFMAs while the VALU finishes this half (S_old, the
    // new weights, their rounding and the write back to the W buffer): the
    // matrix cores and the VALU work side by side instead of in turns, with no
    // more accumulators alive than the four slots of one half plus two.
    auto unit = [&](int sb) {
        const uint16_t* Acur = As + (sb & 1) * BUF_ELEMS;
        uint16_t* ws = Wb + (sb % kWideWBufs) * WBUF + w * WBLK;
        auto a_op = [&](int b, int slot, int ks) {
            const uint16_t* ap = Acur + b * 32 * RPAD + n * RPAD;
            return *(const u32x4*)(ap + slot * SLOT_ELEMS + (a_chunk_swz<R16>(n, 2 * ks + h) << 3));
        };
        // slots s0 and s0 + 1 of half b over every rank chunk (each slot sums
        // its chunks in order; the next chunk's operands are read meanwhile)
        auto mfma_pair = [&](int b, int s0, f32x16& Pa, f32x16& Pb) {
            u32x4 ao[2][2];
            ao[0][0] = a_op(b, s0, 0);
            ao[0][1] = a_op(b, s0 + 1, 0);
#pragma unroll
            for (int ks = 0; ks < R16; ++ks) {
                if (ks + 1 < R16) {
                    ao[(ks + 1) & 1][0] = a_op(b, s0, ks + 1);
                    ao[(ks + 1) & 1][1] = a_op(b, s0 + 1, ks + 1);
                }
                Pa = mfma32(ao[ks & 1][0], bcur[s0][ks], Pa);
                Pb = mfma32(ao[ks & 1][1], bcur[s0 + 1][ks], Pb);
            }
        };
        auto load_wm = [&](int b, u32x4 (&wm)[2]) {
#pragma unroll
            for (int q = 0; q < 2; ++q) wm[q] = *(const u32x4*)(ws + w_off(n, 4 * b + 2 * h + q));
        };
        // S_new of the 16 outputs from slots 0 and 1
        auto s_new = [&](const f32x16& P0, const f32x16& P1, float (&sn)[16]) {
#pragma unroll
            for (int i = 0; i < 16; ++i) sn[i] = fmaf(sc.c[1], P1[i], sc.c[0] * P0[i]);
        };
        // S_old, W' = RNE(W - (S_old - S_new)) and the write back of half b
        auto finish = [&](int b, const u32x4 (&wm)[2], const float (&sn)[16], const f32x16& P2,
                          const f32x16& P3) {
            uint32_t ow[8];
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const uint32_t word = wm[p >> 2][p & 3];
                float o2[2];
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int i = 2 * p + j;
                    const float so = fmaf(sc.c[3], P3[i], sc.c[2] * P2[i]);
                    const float wf = j ? bf_hi(word) : bf_lo(word);
                    o2[j] = wf - (so - sn[i]);
                }
                ow[p] = pack2_bf16(o2[0], o2[1]);
            }
#pragma unroll
            for (int q = 0; q < 2; ++q)
                *(u32x4*)(ws + w_off(n, 4 * b + 2 * h + q)) =
                    u32x4{ow[4 * q], ow[4 * q + 1], ow[4 * q + 2], ow[4 * q + 3]};
        };
        u32x4 wm0[2], wm1[2];
        load_wm(0, wm0);
        load_wm(1, wm1);
        float sn0[16], sn1[16];
        f32x16 H0[2] = {f32x16{}, f32x16{}}, H1[2] = {f32x16{}, f32x16{}};
        // interleave the MFMAs of a region with its VALU work: one MFMA, then
        // NV VALU instructions, for each of the region's 2 R16 MFMAs
        auto interleave = [&](auto nv) {
#pragma unroll
            for (int i = 0; i < 2 * R16; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, decltype(nv)::value, 0);  // VALU
            }
        };
        mfma_pair(0, 0, H0[0], H0[1]);
        __builtin_amdgcn_sched_barrier(0);
        {
            f32x16 Q0[2] = {f32x16{}, f32x16{}};
            mfma_pair(0, 2, Q0[0], Q0[1]);
            s_new(H0[0], H0[1], sn0);
            interleave(std::integral_constant<int, 32 / (2 * R16)>{});
            __builtin_amdgcn_sched_barrier(0);
            mfma_pair(1, 0, H1[0], H1[1]);
            finish(0, wm0, sn0, Q0[0], Q0[1]);
            interleave(std::integral_constant<int, 96 / (2 * R16)>{});
            __builtin_amdgcn_sched_barrier(0);
        }
        {
            f32x16 Q1[2] = {f32x16{}, f32x16{}};
            mfma_pair(1, 2, Q1[0], Q1[1]);
            s_new(H1[0], H1[1], sn1);
            interleave(std::integral_constant<int, 32 / (2 * R16)>{});
            __builtin_amdgcn_sched_barrier(0);
            finish(1, wm1, sn1, Q1[0], Q1[1]);
        }
        const int col = col_base + sb * 64 + 8 * lc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = row0 + 8 * i + lr;
            const u32x4 v = *(const u32x4*)(ws + w_off(8 * i + lr, lc));
            if (FULL || (row < d_out && col < d_in)) st128_nt(W + (int64_t)row * d_in + col, v);
        }
    };

    // issue order: B loads, A(0), W(0), W(1); then per sub-band sb: A(sb+1),
    // W(sb+2), the stores of sb (4 per wave in full tiles; an edge tile's
    // guarded stores are drained before the next sub-band so the counts hold)
    copy_a(0);
    __builtin_amdgcn_sched_barrier(0);
    copy_w(0);
    __builtin_amdgcn_sched_barrier(0);
    if (nsb > 1) copy_w(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll 1
    for (int sb = 0; sb < nsb; ++sb) {
        const bool more1 = sb + 1 < nsb, more2 = sb + 2 < nsb;
        // A(sb) is followed by W(sb+1) (if any) and the stores of sb-1 (W(0)
        // for sb = 0: the same count)
        wait_vmcnt_le<8>(4 + (more1 ? 4 : 0));
        __builtin_amdgcn_s_barrier();  // A(sb) is in LDS for every wave; A buffer (sb+1)&1 is free
        __builtin_amdgcn_sched_barrier(0);
        if (more1) copy_a(sb + 1);
        __builtin_amdgcn_sched_barrier(0);
        if (more2) copy_w(sb + 2);
        __builtin_amdgcn_sched_barrier(0);
        // W(sb) is followed, in issue order, by: the stores of sb-2 (sb >= 2);
        // A(sb) (sb >= 1); W(sb+1) (if any); the stores of sb-1 (sb >= 1);
        // A(sb+1) and W(sb+2) (if any)
        if (FULL && sb >= 2 && more2) {
            wait_vmcnt<16 + 2 * NAI>();
        } else {
            const int after = (sb >= 1 ? 4 + NAI : 0) + (sb >= 2 ? 4 : 0) + (more1 ? 4 + NAI : 0) + (more2 ? 4 : 0);
            wait_vmcnt_le<16 + 2 * NAI>(after);
        }
        __builtin_amdgcn_sched_barrier(0);
        unit(sb);
        if (!FULL) wait_vmcnt<0>();
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int R16, int NSB>
__global__ __launch_bounds__(kWW* kWave) __attribute__((amdgpu_waves_per_eu(2)))
void switch_wide_kernel(SwitchArgs a) {
    // 2 x [4 slots][2][32][R16*16] A images, then kWideWBufs x 8 x [32][64] W buffers
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    const int64_t bid = blockIdx.x;
    const int64_t t = (bid & 7) * a.per_xcd + (bid >> 3);
    if (t >= a.n_units) return;
    const Sets sc = read_sets(a);
    if (!sc.ok) {
        if (t == 0 && threadIdx.x == 0) *a.err = 1;
        return;
    }
    const SwDesc D = a.descs[find_desc<kKeyTile>(a.descs, a.n_desc, t)];
    // groups of kWGroup row bands; inside a group, column band by column band
    const int64_t local = t - D.tile0;
    const int64_t per_group = (int64_t)kWGroup * D.n_ct;
    const int grp = (int)(local / per_group);
    const int in_grp = D.n_rt - grp * kWGroup < kWGroup ? D.n_rt - grp * kWGroup : kWGroup;
    const int64_t lg = local - grp * per_group;
    const int rt = grp * kWGroup + (int)(lg % in_grp), ct = (int)(lg / in_grp);
    const int row_base = rt * kWRT, col_base = ct * (64 * NSB);
    const bool full = row_base + kWRT <= D.d_out && col_base + 64 * NSB <= D.d_in && a.r == R16 * 16;
    if (full)
        switch_wide_tile<R16, NSB, true>(a, sc, D, row_base, col_base, smem);
    else
        switch_wide_tile<R16, NSB, false>(a, sc, D, row_base, col_base, smem);
}

// ---- merged-weight products -------------------------------------------------
//
// After a switch the adapted projection of a decode step is the plain product
// of the merged weight with the layer input (the pages' fused kernel merges
// the selected adapters into the backbone and carries out the computation in a
// single kernel).  Two forms:
//   * switch_gemv_kernel: the rank-16 switch tile above with GEMV = true, so
//     every weight is read once, written once and multiplied by x in the same
//     pass; each 256 x 256 tile stores its partial products, and
//     gemv_reduce_kernel adds a row's n_ct partials in column-tile order (a
//     kernel boundary in between, so no cross-workgroup synchronisation).
//   * gemv_kernel: the product alone (the unfused baseline, or after a switch
//     the fused kernel does not serve): one row per wave, lanes striding over
//     16-byte chunks of the row (four in flight) with fp32 sums, then a
//     fixed-order butterfly across the wave.  Every result is bitwise
//     reproducible.

__global__ __launch_bounds__(kWaves* kWave) __attribute__((amdgpu_waves_per_eu(3)))
void switch_gemv_kernel(SwitchArgs a) {
    constexpr int R16 = 1, CT = 256;
    extern __shared__ __attribute__((aligned(16))) uint16_t smem[];
    uint16_t* As = smem;
    uint16_t* Ws = smem + 4 * (CT / 32) * 32 * (R16 * 16);
    uint16_t* Xs = Ws + kWaves * 32 * 64;
    const int64_t bid = blockIdx.x;
    const int64_t t = (bid & 7) * a.per_xcd + (bid >> 3);
    if (t >= a.n_units) return;
    const Sets sc = read_sets(a);
    if (!sc.ok) {
        if (t == 0 && threadIdx.x == 0) *a.err = 1;
        return;
    }
    const SwDesc D = a.descs[find_desc<kKeyTile>(a.descs, a.n_desc, t)];
    const int64_t local = t - D.tile0;
    const int row_base = (int)(local / D.n_ct) * kRT;
    const int col_base = (int)(local % D.n_ct) * CT;
    const int tid = threadIdx.x;
    if (tid < CT / 8) {
        const int col = col_base + 8 * tid;
        *(u32x4*)(Xs + 8 * tid) = col < D.d_in ? ld128((const uint16_t*)D.xv + col) : u32x4{0u, 0u, 0u, 0u};
    }
    __syncthreads();
    const bool full = row_base + kRT <= D.d_out && col_base + CT <= D.d_in && a.r == R16 * 16;
    if (full)
        switch_tile<R16, CT, true, true>(a, sc, D, row_base, col_base, As, Ws, Xs);
    else
        switch_tile<R16, CT, false, true>(a, sc, D, row_base, col_base, As, Ws, Xs);
}

// y[row] = sum over column tiles c = 0, 1, ... of part[c][row]; one thread per
// row of a 256-row band.  Sets the switch rejects (same check) leave y alone.
__global__ __launch_bounds__(256) void gemv_reduce_kernel(SwitchArgs a, int64_t n_bands) {
    const int64_t t = blockIdx.x;
    if (t >= n_bands || !read_sets(a).ok) return;
    const SwDesc D = a.descs[find_desc<kKeyBand>(a.descs, a.n_desc, t)];
    const int row = (int)(t - D.rt0) * kRT + threadIdx.x;
    if (row >= D.d_out) return;
    // eight independent loads in flight per step; the additions stay in c order
    const float* pp = D.part + row;
    const int64_t st = D.d_out;
    float sum = 0.f;
    int c = 0;
    for (; c + 8 <= D.n_ct; c += 8) {
        float v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = gld(pp + (c + j) * st);
#pragma unroll
        for (int j = 0; j < 8; ++j) sum += v[j];
    }
    for (; c < D.n_ct; ++c) sum += gld(pp + c * st);
    gst(D.yv + row, sum);
}

static_assert(kGemvRows == kWaves, "one row per wave");
constexpr int kGemvUnroll = 4;  // 16-byte chunks of the row in flight per lane

// Blocks run last-first: in a layer the longest rows (the MLP's down
// projection) come last, so they start early instead of forming the tail.

// W row . x for one wave: lanes over 16-byte chunks of the row (kGemvUnroll in
// flight), fp32 FMA chains, then a fixed-order butterfly (every lane ends with
// the row's sum).
template <typename T>
__device__ __forceinline__ float row_dot(const T* __restrict__ Wr, const T* __restrict__ x, int d_in, int lane) {
    float acc = 0.f;
    if constexpr (sizeof(T) == 2) {
        const int nch = d_in / 8;
        int c = lane;
        for (; c + (kGemvUnroll - 1) * kWave < nch; c += kGemvUnroll * kWave) {
            u32x4 xv[kGemvUnroll], wv[kGemvUnroll];
#pragma unroll
            for (int u = 0; u < kGemvUnroll; ++u) {
                wv[u] = ld128_nt(Wr + 8 * (c + u * kWave));
                xv[u] = ld128(x + 8 * (c + u * kWave));
            }
#pragma unroll
            for (int u = 0; u < kGemvUnroll; ++u)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    acc = fmaf(bf_lo(wv[u][q]), bf_lo(xv[u][q]), acc);
                    acc = fmaf(bf_hi(wv[u][q]), bf_hi(xv[u][q]), acc);
                }
        }
        for (; c < nch; c += kWave) {
            const u32x4 xv = ld128(x + 8 * c), wv = ld128_nt(Wr + 8 * c);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                acc = fmaf(bf_lo(wv[q]), bf_lo(xv[q]), acc);
                acc = fmaf(bf_hi(wv[q]), bf_hi(xv[q]), acc);
            }
        }
    } else {
        int j = lane;
        for (; j + (kGemvUnroll - 1) * kWave < d_in; j += kGemvUnroll * kWave) {
            float w[kGemvUnroll], xv[kGemvUnroll];
#pragma unroll
            for (int u = 0; u < kGemvUnroll; ++u) {
                w[u] = gld(Wr + j + u * kWave);
                xv[u] = gld(x + j + u * kWave);
            }
#pragma unroll
            for (int u = 0; u < kGemvUnroll; ++u) acc = fmaf(w[u], xv[u], acc);
        }
        for (; j < d_in; j += kWave) acc = fmaf(gld(Wr + j), gld(x + j), acc);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc += __shfl_xor(acc, o, kWave);
    return acc;
}

template <typename T>
__global__ __launch_bounds__(kWaves* kWave) void gemv_kernel(SwitchArgs a, int64_t n_blocks) {
    const int64_t t = n_blocks - 1 - (int64_t)blockIdx.x;
    if (t < 0 || !read_sets(a).ok) return;
    const SwDesc D = a.descs[find_desc<kKeyRowBlock>(a.descs, a.n_desc, t)];
    const int d_in = D.d_in, d_out = D.d_out;
    const int lane = lane_id();
    const int row = (int)(t - D.rb0) * kGemvRows + wave_id();
    if (row >= d_out) return;
    const float acc = row_dot<T>((const T*)D.W + (int64_t)row * d_in, (const T*)D.xv, d_in, lane);
    if (lane == 0) gst(D.yv + row, acc);
}

// ---- the product with one set's adapters unmerged ---------------------------
//
// The pre-gated decision with the adapters left unmerged (the token's set,
// made once, applied by every layer; W is never rewritten):
//     y = W x + c_0 B_{e_0} (A_{e_0} x) + c_1 B_{e_1} (A_{e_1} x),  c = s g.
// First launch: one workgroup per (weight, kLoraKSlice-wide K slice, group of
// kLoraDots rank vectors) computes the slice's partials sum_j x[j] A[e_k][rho][j]
// of its group's dots d = k r + rho (each thread one 16-byte chunk of the slice,
// every load of a chunk issued before its FMAs, a wave butterfly, then the waves
// in order).  Second launch: the product kernel, each row then adding
// sum_{k, rho} (c_k v_k[rho]) B[e_k][row][rho], with v_k the slices' partials
// added in slice order; lane l takes the terms (k, rho) = (l / r, l % r) for
// l = lane, lane + 64, ..., they are added with the product's butterfly, and
// y = W x + terms (one more rounding).  The operands of the first term and its
// first slices are loaded before the row's stream, so their latency is hidden
// behind it.  The first launch is short and latency-bound, so its work is cut
// finely (a 7B-shaped layer: 72 workgroups) and its descriptor lookup is one
// vector load and a ballot instead of a dependent search.
constexpr int kLoraDots = 8;
constexpr int kLoraPre = 8;  // slices of the first term loaded ahead

// The fields the first launch reads of the weight holding K slice u (ks0
// ascends over the descriptors).  Up to 64 descriptors, lane i loads key and
// fields of descriptor i in one round and the holder's copy is read from its
// lane; past 64, a ballot per 64 keys finds the holder, then its fields load.
struct LoraDesc {
    int64_t ks0;
    const void* xv;
    const void* A;
    int d_in;
};

__device__ __forceinline__ int64_t lane64(int64_t v, int l) {
    const uint64_t b = (uint64_t)v;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)b, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(b >> 32), l);
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ LoraDesc lora_desc(const SwDesc* __restrict__ d, int n, int64_t u) {
    LoraDesc D;
    const int lane = lane_id();
    if (n <= kWave) {
        int64_t key = INT64_MAX, xv = 0, A = 0;
        int d_in = 0;
        if (lane < n) {
            key = d[lane].ks0;
            xv = (int64_t)d[lane].xv;
            A = (int64_t)d[lane].A;
            d_in = d[lane].d_in;
        }
        const int sel = __popcll(__ballot(key <= u)) - 1;  // descriptor 0 starts at slice 0
        D.ks0 = lane64(key, sel);
        D.xv = (const void*)lane64(xv, sel);
        D.A = (const void*)lane64(A, sel);
        D.d_in = __builtin_amdgcn_readlane(d_in, sel);
        return D;
    }
    int idx = -1;
    for (int b0 = 0; b0 < n; b0 += kWave) {
        const int i = b0 + lane;
        const uint64_t m = __ballot(i < n && d[i].ks0 <= u);
        idx += __popcll(m);
        if (m != ~0ull) break;
    }
    idx = uniform(idx);
    D.ks0 = d[idx].ks0;
    D.xv = d[idx].xv;
    D.A = d[idx].A;
    D.d_in = d[idx].d_in;
    return D;
}

template <typename T>
__global__ __launch_bounds__(kWaves* kWave) void lora_shrink_kernel(SwitchArgs a, int n_dg) {
    // the grid is exactly the work units (slices x dot groups, < 2^31); the
    // set is always given (the entry point refuses a null one) and there is
    // no old set, so the set words load unconditionally, in flight with the
    // descriptor round
    const int u = blockIdx.x;
    const int gks = u / n_dg;
    const int d0 = (u - gks * n_dg) * kLoraDots;
    SetWords sw;
    sw.e[0] = a.new_idx[0];
    sw.e[1] = a.new_idx[1];
    sw.g[0] = a.new_g[0];
    sw.g[1] = a.new_g[1];
    sw.e[2] = sw.e[3] = -1;
    sw.g[2] = sw.g[3] = 0.f;
    const LoraDesc D = lora_desc(a.descs, a.n_desc, gks);
    const Sets sc = check_sets(a, sw);
    if (!sc.ok) {
        if (u == 0 && threadIdx.x == 0) *a.err = 1;
        return;
    }
    const int d_in = D.d_in, r = a.r, nd = 2 * r;
    const int k0 = (int)(gks - D.ks0) * kLoraKSlice;
    const int k1 = k0 + kLoraKSlice < d_in ? k0 + kLoraKSlice : d_in;
    const T* __restrict__ x = (const T*)D.xv;
    const T* __restrict__ A = (const T*)D.A;
    __shared__ float s_red[kWaves][kLoraDots];
    const int tid = threadIdx.x, w = wave_id(), lane = lane_id();
    float p[kLoraDots];
#pragma unroll
    for (int i = 0; i < kLoraDots; ++i) p[i] = 0.f;
    // dot d = k r + rho; past nd the last dot again (not stored)
    auto a_row = [&](int i) {
        const int d = d0 + i < nd ? d0 + i : nd - 1;
        const int k = d >= r ? 1 : 0;
        const int e = k ? sc.e[1] : sc.e[0];
        return A + ((int64_t)(e >= 0 ? e : 0) * r + (d - k * r)) * d_in;
    };
    if constexpr (sizeof(T) == 2) {
        for (int c = k0 / 8 + tid; c < k1 / 8; c += kWaves * kWave) {
            const u32x4 xv = ld128(x + 8 * c);
            u32x4 av[kLoraDots];
#pragma unroll
            for (int i = 0; i < kLoraDots; ++i) av[i] = ld128(a_row(i) + 8 * c);
#pragma unroll
            for (int i = 0; i < kLoraDots; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    p[i] = fmaf(bf_lo(xv[q]), bf_lo(av[i][q]), p[i]);
                    p[i] = fmaf(bf_hi(xv[q]), bf_hi(av[i][q]), p[i]);
                }
        }
    } else {
        for (int j = k0 + tid; j < k1; j += kWaves * kWave) {
            const float xv = gld(x + j);
#pragma unroll
            for (int i = 0; i < kLoraDots; ++i) p[i] = fmaf(xv, gld(a_row(i) + j), p[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < kLoraDots; ++i) {
        float sw = p[i];
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) sw += __shfl_xor(sw, o, kWave);
        if (lane == 0) s_red[w][i] = sw;
    }
    __syncthreads();
    if (tid < kLoraDots && d0 + tid < nd) {
        const int d = d0 + tid;
        float sv = s_red[0][tid];
#pragma unroll
        for (int ww = 1; ww < kWaves; ++ww) sv += s_red[ww][tid];
        const int e = d >= r ? sc.e[1] : sc.e[0];
        gst(a.vpart + (int64_t)gks * nd + d, e >= 0 ? sv : 0.f);
    }
}

template <typename T>
__device__ __forceinline__ float elem_f(const T* p) {
    if constexpr (sizeof(T) == 2) return bf_to_f(gld((const uint16_t*)p));
    else return gld((const float*)p);
}

template <typename T>
__global__ __launch_bounds__(kWaves* kWave) void gemv_lora_kernel(SwitchArgs a, int64_t n_blocks) {
    const int64_t t = n_blocks - 1 - (int64_t)blockIdx.x;
    if (t < 0) return;
    const Sets sc = read_sets(a);
    if (!sc.ok) return;
    const SwDesc D = a.descs[find_desc<kKeyRowBlock>(a.descs, a.n_desc, t)];
    const int d_in = D.d_in, d_out = D.d_out, r = a.r, nd = 2 * r, n_ks = D.n_ks;
    const int lane = lane_id();
    const int row = (int)(t - D.rb0) * kGemvRows + wave_id();
    if (row >= d_out) return;
    const T* __restrict__ B = (const T*)D.B;
    const float* vp = a.vpart + D.ks0 * nd;  // slice s of this weight at vp + s * nd
    // term l = lane (the first of this lane's): B element and the first slices
    const int k_f = lane >= r ? 1 : 0, e_f = k_f ? sc.e[1] : sc.e[0];
    const bool on_f = lane < nd && e_f >= 0;
    float b_f = 0.f, pv[kLoraPre];
    if (on_f) b_f = elem_f(B + ((int64_t)e_f * d_out + row) * r + (lane - k_f * r));
#pragma unroll
    for (int s = 0; s < kLoraPre; ++s) pv[s] = (on_f && s < n_ks) ? gld(vp + s * nd + lane) : 0.f;

    const float acc = row_dot<T>((const T*)D.W + (int64_t)row * d_in, (const T*)D.xv, d_in, lane);

    float ad = 0.f;
    if (on_f) {
        float v = pv[0];
#pragma unroll
        for (int s = 1; s < kLoraPre; ++s)
            if (s < n_ks) v += pv[s];
        for (int s = kLoraPre; s < n_ks; ++s) v += gld(vp + s * nd + lane);
        ad = (sc.c[k_f] * v) * b_f;
    }
    for (int l = lane + kWave; l < nd; l += kWave) {  // ranks above 32: more terms per lane
        const int k = l >= r ? 1 : 0, e = k ? sc.e[1] : sc.e[0];
        if (e < 0) continue;
        float v = gld(vp + l);
        for (int s = 1; s < n_ks; ++s) v += gld(vp + s * nd + l);
        ad = fmaf(sc.c[k] * v, elem_f(B + ((int64_t)e * d_out + row) * r + (l - k * r)), ad);
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) ad += __shfl_xor(ad, o, kWave);
    if (lane == 0) gst(D.yv + row, acc + ad);
}

// ---- element-wise path: fp32 weights (and any shape) ----------------------

template <typename T> __device__ __forceinline__ float ldf(const T* p, int64_t i);
template <> __device__ __forceinline__ float ldf<float>(const float* p, int64_t i) { return p[i]; }
template <> __device__ __forceinline__ float ldf<uint16_t>(const uint16_t* p, int64_t i) {
    return bf_to_f(p[i]);
}
template <typename T> __device__ __forceinline__ void stf(T* p, int64_t i, float v);
template <> __device__ __forceinline__ void stf<float>(float* p, int64_t i, float v) { p[i] = v; }
template <> __device__ __forceinline__ void stf<uint16_t>(uint16_t* p, int64_t i, float v) {
    p[i] = f_to_bf(v);
}

template <typename T>
__global__ __launch_bounds__(256) void switch_generic_kernel(SwitchArgs a) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= a.n_units) return;
    const Sets sc = read_sets(a);
    if (!sc.ok) {
        if (u == 0) *a.err = 1;
        return;
    }
    const SwDesc D = a.descs[find_desc<kKeyElem>(a.descs, a.n_desc, u)];
    const int64_t local = u - D.elem0;
    const int64_t row = local / D.d_in, col = local % D.d_in;
    const T* A = (const T*)D.A;
    const T* B = (const T*)D.B;
    T* W = (T*)D.W;
    float P[4];
#pragma unroll
    for (int slot = 0; slot < 4; ++slot) {
        float acc = 0.f;
        const int e = sc.e[slot];
        if (e >= 0)
            for (int rho = 0; rho < a.r; ++rho)
                acc = fmaf(ldf(B, ((int64_t)e * D.d_out + row) * a.r + rho),
                           ldf(A, ((int64_t)e * a.r + rho) * D.d_in + col), acc);
        P[slot] = acc;
    }
    const float sn = fmaf(sc.c[1], P[1], sc.c[0] * P[0]);
    const float so = fmaf(sc.c[3], P[3], sc.c[2] * P[2]);
    const int64_t i = row * D.d_in + col;
    stf(W, i, ldf(W, i) - (so - sn));
}

// Packed A images of the copy-staged wide tiles: thread (e, cb, rank chunk
// ch, column c) writes the 16 bytes holding ranks 8ch..8ch+7 of column
// 64cb + c at the position the MFMA reads them from (zero past r and d_in).
// Consecutive threads take consecutive columns, so the A reads coalesce.
template <int R16>
__global__ __launch_bounds__(256) void switch_pack_a_kernel(const uint16_t* __restrict__ A, uint16_t* __restrict__ Ap,
                                                            int64_t d_in, int E, int r, int64_t n_cb) {
    constexpr int RPAD = R16 * 16, SLOT_ELEMS = 2 * 32 * RPAD, NCH = RPAD / 8;
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= (int64_t)E * n_cb * NCH * 64) return;
    const int c = (int)(t % 64), ch = (int)((t / 64) % NCH);
    const int64_t blk = t / (64 * NCH);  // e * n_cb + cb
    const int e = (int)(blk / n_cb);
    const int64_t col = (blk % n_cb) * 64 + c;
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r0 = ch * 8 + 2 * j;
        const uint32_t lo = (r0 < r && col < d_in) ? gld(A + ((int64_t)e * r + r0) * d_in + col) : 0u;
        const uint32_t hi = (r0 + 1 < r && col < d_in) ? gld(A + ((int64_t)e * r + r0 + 1) * d_in + col) : 0u;
        v[j] = lo | (hi << 16);
    }
    const int m = perm_row(c & 31);
    st128(Ap + blk * SLOT_ELEMS + (c >> 5) * 32 * RPAD + m * RPAD + (a_chunk_swz<R16>(m, ch) << 3),
          u32x4{v[0], v[1], v[2], v[3]});
}

template <int R16, int CT>
constexpr size_t lds_r() {
    return ((size_t)4 * (CT / 32) * 32 * (R16 * 16) + (size_t)kWaves * 32 * 64) * sizeof(uint16_t);
}

// Dynamic LDS past 64 KB needs the kernel's attribute raised once, at set-up,
// so that launches (which a caller may capture into a graph) only launch.
template <int R16, int CT>
hipError_t prepare_r() {
    if (lds_r<R16, CT>() <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void*)switch_bf16_kernel<R16, CT>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_r<R16, CT>());
}

template <int R16, int CT>
hipError_t launch_r(const SwitchArgs& a, hipStream_t s) {
    const int64_t grid = 8 * a.per_xcd;
    if (!grid_fits(grid, kWaves * kWave)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((switch_bf16_kernel<R16, CT>), dim3((unsigned)grid), dim3(kWaves * kWave),
                       (lds_r<R16, CT>()), s, a);
    return hipGetLastError();
}

}  // namespace

template <int R16>
constexpr size_t lds_wide() {
    return ((size_t)2 * 4 * 2 * 32 * (R16 * 16) + (size_t)kWideWBufs * kWW * 32 * 64) * sizeof(uint16_t);
}

template <int R16>
hipError_t prepare_wide() {
    if (lds_wide<R16>() <= 65536) return hipSuccess;
    return hipFuncSetAttribute((const void*)switch_wide_kernel<R16, kWideSB>,
                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds_wide<R16>());
}

template <int R16>
hipError_t launch_wide(const SwitchArgs& a, hipStream_t s) {
    const int64_t grid = 8 * a.per_xcd;
    if (!grid_fits(grid, kWW * kWave)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((switch_wide_kernel<R16, kWideSB>), dim3((unsigned)grid), dim3(kWW * kWave),
                       lds_wide<R16>(), s, a);
    return hipGetLastError();
}

hipError_t prepare_switch_bf16(const SwTile& t) {
    switch (t.r16) {
        case 1: return prepare_r<1, 256>();
        case 2: return prepare_wide<2>();
        case 3: return prepare_wide<3>();
        case 4: return prepare_wide<4>();
        case 5: return prepare_r<5, 64>();
        case 6: return prepare_r<6, 64>();
        case 7: return prepare_r<7, 64>();
        case 8: return prepare_r<8, 64>();
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_switch_bf16(const SwitchArgs& a, const SwTile& t, hipStream_t s) {
    switch (t.r16) {
        case 1: return launch_r<1, 256>(a, s);
        case 2: return launch_wide<2>(a, s);
        case 3: return launch_wide<3>(a, s);
        case 4: return launch_wide<4>(a, s);
        case 5: return launch_r<5, 64>(a, s);
        case 6: return launch_r<6, 64>(a, s);
        case 7: return launch_r<7, 64>(a, s);
        case 8: return launch_r<8, 64>(a, s);
        default: return hipErrorInvalidValue;
    }
}

bool switch_packs_a(const SwTile& t) { return t.r16 >= 2 && t.r16 <= 4; }

size_t switch_packed_a_elems(int64_t d_in, int E, const SwTile& t) {
    return (size_t)E * (size_t)((d_in + 63) / 64) * 2 * 32 * (t.r16 * 16);
}

size_t switch_zero_image_elems(const SwTile& t) { return (size_t)2 * 32 * (t.r16 * 16); }

hipError_t launch_switch_pack_a(const void* A, void* Ap, int64_t d_in, int E, int r, const SwTile& t,
                                hipStream_t s) {
    const int64_t n_cb = (d_in + 63) / 64;
    const int64_t threads = (int64_t)E * n_cb * (t.r16 * 2) * 64;
    if (!grid_fits((threads + 255) / 256, 256)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((threads + 255) / 256));
    const uint16_t* a = (const uint16_t*)A;
    uint16_t* ap = (uint16_t*)Ap;
    switch (t.r16) {
        case 2: hipLaunchKernelGGL(switch_pack_a_kernel<2>, grid, dim3(256), 0, s, a, ap, d_in, E, r, n_cb); break;
        case 3: hipLaunchKernelGGL(switch_pack_a_kernel<3>, grid, dim3(256), 0, s, a, ap, d_in, E, r, n_cb); break;
        case 4: hipLaunchKernelGGL(switch_pack_a_kernel<4>, grid, dim3(256), 0, s, a, ap, d_in, E, r, n_cb); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

bool switch_gemv_fused(const SwTile& t, int dtype) { return dtype == 1 && t.r16 == 1 && t.ct == 256; }

hipError_t launch_switch_gemv_bf16(const SwitchArgs& a, hipStream_t s) {
    const size_t lds = ((size_t)4 * 8 * 32 * 16 + (size_t)kWaves * 32 * 64 + 256) * sizeof(uint16_t);
    if (!grid_fits(8 * a.per_xcd, kWaves * kWave)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(switch_gemv_kernel, dim3((unsigned)(8 * a.per_xcd)), dim3(kWaves * kWave), lds, s, a);
    return hipGetLastError();
}

hipError_t launch_gemv_reduce(const SwitchArgs& a, int64_t n_bands, hipStream_t s) {
    if (n_bands == 0) return hipSuccess;
    if (!grid_fits(n_bands, 256)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(gemv_reduce_kernel, dim3((unsigned)n_bands), dim3(256), 0, s, a, n_bands);
    return hipGetLastError();
}

hipError_t launch_gemv_unmerged(const SwitchArgs& a, int64_t n_ks_total, int64_t n_blocks, int dtype,
                                hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    const int n_dg = (2 * a.r + kLoraDots - 1) / kLoraDots;
    const int64_t n_units = n_ks_total * n_dg;
    if (!grid_fits(n_units, kWaves * kWave) || !grid_fits(n_blocks, kWaves * kWave))
        return hipErrorInvalidConfiguration;
    if (dtype == 0)
        hipLaunchKernelGGL(lora_shrink_kernel<float>, dim3((unsigned)n_units), dim3(kWaves * kWave), 0, s, a, n_dg);
    else
        hipLaunchKernelGGL(lora_shrink_kernel<uint16_t>, dim3((unsigned)n_units), dim3(kWaves * kWave), 0, s, a, n_dg);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (dtype == 0)
        hipLaunchKernelGGL(gemv_lora_kernel<float>, dim3((unsigned)n_blocks), dim3(kWaves * kWave), 0, s, a, n_blocks);
    else
        hipLaunchKernelGGL(gemv_lora_kernel<uint16_t>, dim3((unsigned)n_blocks), dim3(kWaves * kWave), 0, s, a,
                           n_blocks);
    return hipGetLastError();
}

hipError_t launch_gemv(const SwitchArgs& a, int64_t n_blocks, int dtype, hipStream_t s) {
    if (n_blocks == 0) return hipSuccess;
    if (!grid_fits(n_blocks, kWaves * kWave)) return hipErrorInvalidConfiguration;
    if (dtype == 0)
        hipLaunchKernelGGL(gemv_kernel<float>, dim3((unsigned)n_blocks), dim3(kWaves * kWave), 0, s, a, n_blocks);
    else
        hipLaunchKernelGGL(gemv_kernel<uint16_t>, dim3((unsigned)n_blocks), dim3(kWaves * kWave), 0, s, a, n_blocks);
    return hipGetLastError();
}

hipError_t launch_switch_generic(const SwitchArgs& a, int dtype, hipStream_t s) {
    if (!grid_fits((a.n_units + 255) / 256, 256)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((a.n_units + 255) / 256));
    if (dtype == 0)
        hipLaunchKernelGGL(switch_generic_kernel<float>, grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(switch_generic_kernel<uint16_t>, grid, dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace dlm
