// Token-level top-2 pre-gate (AdaFuse digest, section 2-ga: a lightweight
// top-2 router at the first layer fixes each token's expert set, which every
// later layer reuses).
//
// One wave64 per token.  Each lane accumulates the E logits over its share of
// the columns in binary64 (the products of fp32 or bf16 operands are exact in
// binary64), a fixed butterfly sums the 64 partials, then lane e holds logit e
// and a cross-lane reduction over the wave takes the top two (ties -> lower
// index); lane 0 stores them and the renormalised pair of weights
// g0 = 1/(1+exp(l1-l0)), g1 = exp(l1-l0)/(1+exp(l1-l0)).
#include "dlm.h"
#include "gfx950.hpp"
#include "internal.hpp"

namespace dlm {
namespace {

template <typename T> __device__ __forceinline__ double ldv(const T* p, int64_t i);
template <> __device__ __forceinline__ double ldv<float>(const float* p, int64_t i) {
    return (double)p[i];
}
template <> __device__ __forceinline__ double ldv<uint16_t>(const uint16_t* p, int64_t i) {
    return (double)bf_to_f(p[i]);
}

constexpr int kTokPerBlock = 4;

// Index of the largest key over the wave, equal keys resolved to the lower
// index, by a xor butterfly: every lane ends with the same winner whatever
// order the pairs meet in, since "larger key, then lower index" is a total
// order on the (key, index) pairs.
__device__ __forceinline__ int wave_argmax(double key, int i) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double k2 = __shfl_xor(key, o, kWave);
        const int i2 = __shfl_xor(i, o, kWave);
        if (k2 > key || (k2 == key && i2 < i)) {
            key = k2;
            i = i2;
        }
    }
    return i;
}

// Top two of the logits held one per lane (lane e < E holds expert e's) by two
// wave argmax rounds, then lane 0 stores them and the renormalised weights.
// The keys make each round a strict '>' scan from its lowest candidate index
// (expert 0 for slot 0, the lowest expert other than slot 0's for slot 1):
// equal logits keep the lower index, and a NaN logit is kept where the scan
// starts (the largest key there) and never taken elsewhere (the smallest key),
// so the indices stay in range and distinct.  Lanes past E, and slot 0's lane
// in the second round, carry indices above every expert's and lose every tie.
__device__ __forceinline__ void wave_top2_store(double l, int E, int64_t t, int32_t* idx, float* g) {
    const int lane = lane_id();
    const double inf = __builtin_huge_val();
    const bool nan = l != l;
    const bool on = lane < E;
    const double k0 = !on ? -inf : (nan ? (lane == 0 ? inf : -inf) : l);
    const int i0 = uniform(wave_argmax(k0, on ? lane : kWave + lane));
    const int j0 = i0 == 0 ? 1 : 0;
    const bool on1 = on && lane != i0;
    const double k1 = !on1 ? -inf : (nan ? (lane == j0 ? inf : -inf) : l);
    const int i1 = uniform(wave_argmax(k1, on1 ? lane : kWave + lane));
    const double l0 = __shfl(l, i0, kWave), l1 = __shfl(l, i1, kWave);
    if (lane == 0) {
        const double q = exp(l1 - l0);  // <= 1
        idx[2 * t] = i0;
        idx[2 * t + 1] = i1;
        g[2 * t] = (float)(1.0 / (1.0 + q));
        g[2 * t + 1] = (float)(q / (1.0 + q));
    }
}

// Sum each logit over the wave (fixed butterfly), then the wave's top two.
template <int EMAX>
__device__ __forceinline__ void top2(double (&acc)[EMAX], int E, int64_t t, int32_t* idx, float* g) {
    const int lane = lane_id();
    double mine = 0.0;
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
        if (e < E) {
            acc[e] = wave_sum(acc[e]);
            if (lane == e) mine = acc[e];
        }
    wave_top2_store(mine, E, t, idx, g);
}

template <typename T, int EMAX>
__global__ __launch_bounds__(kTokPerBlock* kWave) void pregate_kernel(
    const T* __restrict__ x, const T* __restrict__ Wr, int64_t n_tok, int64_t d, int E,
    int32_t* __restrict__ idx, float* __restrict__ g) {
    const int64_t t = (int64_t)blockIdx.x * kTokPerBlock + wave_id();
    if (t >= n_tok) return;
    const int lane = lane_id();
    double acc[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;
    const T* xr = x + t * d;
    for (int64_t j = lane; j < d; j += kWave) {
        const double xv = ldv(xr, j);
        const T* w = Wr + j * E;
#pragma unroll
        for (int e = 0; e < EMAX; ++e)
            if (e < E) acc[e] = fma(xv, ldv(w, e), acc[e]);
    }
    top2<EMAX>(acc, E, t, idx, g);
}

// bf16 with d and E multiples of 8 (16-byte aligned rows): one workgroup of
// kVecWaves waves per token.  Lane j of wave w takes the 8 consecutive columns
// of chunks c = j + 64 (w + kVecWaves i); x comes in one 16-byte load and each
// Wr row in E/8 (two chunks' loads in flight at a time for E <= 16).  The
// waves' sums are added in wave order.
constexpr int kVecWaves = 4;
template <int EMAX>
__global__ __launch_bounds__(kVecWaves* kWave) void pregate_bf16_vec(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ Wr, int64_t n_tok, int64_t d, int E,
    int32_t* __restrict__ idx, float* __restrict__ g) {
    const int64_t t = blockIdx.x;
    const int lane = lane_id(), w = wave_id();
    __shared__ double s_part[kVecWaves][EMAX];
    double acc[EMAX];
#pragma unroll
    for (int e = 0; e < EMAX; ++e) acc[e] = 0.0;
    const uint16_t* xr = x + t * d;
    const int64_t nc = d / 8;
    auto chunk = [&](const u32x4& xv, const u32x4 (&wv)[8][EMAX / 8]) {
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) {
            const double xj = (double)(jj & 1 ? bf_hi(xv[jj >> 1]) : bf_lo(xv[jj >> 1]));
#pragma unroll
            for (int e = 0; e < EMAX; ++e) {
                if (e >= E) continue;
                const uint32_t wp = wv[jj][e >> 3][(e & 7) >> 1];
                acc[e] = fma(xj, (double)(e & 1 ? bf_hi(wp) : bf_lo(wp)), acc[e]);
            }
        }
    };
    auto load = [&](int64_t c, u32x4& xv, u32x4 (&wv)[8][EMAX / 8]) {
        xv = ld128(xr + 8 * c);
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
#pragma unroll
            for (int e8 = 0; e8 < EMAX / 8; ++e8) {
                // experts past E (E < EMAX) re-read the row's first 8, unused
                const u32x4 v = ld128(Wr + (8 * c + jj) * E + (8 * e8 < E ? 8 * e8 : 0));
                wv[jj][e8] = 8 * e8 < E ? v : u32x4{0u, 0u, 0u, 0u};
            }
    };
    constexpr int64_t kStep = (int64_t)kVecWaves * kWave;
    int64_t c = lane + (int64_t)kWave * w;
    if constexpr (EMAX <= 16) {  // two chunks in flight (registers allow it)
        for (; c + kStep < nc; c += 2 * kStep) {
            u32x4 xa, xb, wa[8][EMAX / 8], wb[8][EMAX / 8];
            load(c, xa, wa);
            load(c + kStep, xb, wb);
            __builtin_amdgcn_sched_barrier(0);  // both chunks' loads issue before any use
            chunk(xa, wa);
            chunk(xb, wb);
        }
    }
    for (; c < nc; c += kStep) {
        u32x4 xa, wa[8][EMAX / 8];
        load(c, xa, wa);
        __builtin_amdgcn_sched_barrier(0);
        chunk(xa, wa);
    }
#pragma unroll
    for (int e = 0; e < EMAX; ++e)
        if (e < E) acc[e] = wave_sum(acc[e]);
    if (lane == 0) {
#pragma unroll
        for (int e = 0; e < EMAX; ++e) s_part[w][e] = acc[e];
    }
    __syncthreads();
    if (w != 0) return;
    // lane e: logit e, the waves' sums added in wave order; then the top two
    double l = 0.0;
    if (lane < E) {
        l = s_part[0][lane];
#pragma unroll
        for (int q = 1; q < kVecWaves; ++q) l += s_part[q][lane];
    }
    wave_top2_store(l, E, t, idx, g);
}

// Nearest-centroid pre-gate (the ARIADNE page: training-free routing by the
// proximity of the input embedding to centroids of each adapter's training
// data; the closest adapter is chosen).  One workgroup of kVecWaves waves per
// token.  The E*J centroids (C [E][J][d], adapter-major) are taken kCGroup at a
// time: each lane sums (x_k - c_k)^2 in binary64 over the columns
// k = lane + 64 (w + kVecWaves i) (fp32 or bf16 inputs: the differences and
// their squares are exact in binary64), the wave sums are added in wave order,
// and each adapter keeps the smallest of its centroids' distances.  Thread 0
// then takes the nearest adapter (strict '<': ties keep the lower index) for
// slot 0 with weight 1; slot 1 is empty (-1, 0).  A NaN distance never
// compares smaller, so the index stays in range.
constexpr int kCGroup = 8;

// VEC (bf16, d a multiple of 8, 16-byte aligned rows): a lane takes 8
// consecutive columns per step, one 16-byte load of x and of each centroid of
// the group, all issued before any arithmetic.
template <typename T, bool VEC>
__global__ __launch_bounds__(kVecWaves* kWave) void pregate_centroid_kernel(
    const T* __restrict__ x, const T* __restrict__ C, int64_t d, int E, int J, int32_t* __restrict__ idx,
    float* __restrict__ g) {
    const int64_t t = blockIdx.x;
    const int lane = lane_id(), w = wave_id();
    __shared__ double s_part[kVecWaves][kCGroup];
    __shared__ double s_de[DLM_MAX_EXPERTS];
    const int EJ = E * J;
    const T* xr = x + t * d;
    for (int c0 = 0; c0 < EJ; c0 += kCGroup) {
        double acc[kCGroup];
#pragma unroll
        for (int q = 0; q < kCGroup; ++q) acc[q] = 0.0;
        if constexpr (VEC) {
            const int64_t nc = d / 8;
            for (int64_t c = lane + (int64_t)kWave * w; c < nc; c += (int64_t)kVecWaves * kWave) {
                const u32x4 xv = ld128((const uint16_t*)xr + 8 * c);
                u32x4 cv[kCGroup];
#pragma unroll
                for (int q = 0; q < kCGroup; ++q)  // centroids past E*J re-read the group's first, unused
                    cv[q] = ld128((const uint16_t*)C + (int64_t)(c0 + q < EJ ? c0 + q : c0) * d + 8 * c);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) {
                    const double xj = (double)(jj & 1 ? bf_hi(xv[jj >> 1]) : bf_lo(xv[jj >> 1]));
#pragma unroll
                    for (int q = 0; q < kCGroup; ++q) {
                        const uint32_t cw = cv[q][jj >> 1];
                        const double df = xj - (double)(jj & 1 ? bf_hi(cw) : bf_lo(cw));
                        acc[q] = fma(df, df, acc[q]);
                    }
                }
            }
        } else {
            for (int64_t k = lane + (int64_t)kWave * w; k < d; k += (int64_t)kVecWaves * kWave) {
                const double xv = ldv(xr, k);
#pragma unroll
                for (int q = 0; q < kCGroup; ++q) {
                    if (c0 + q >= EJ) break;
                    const double df = xv - ldv(C + (int64_t)(c0 + q) * d, k);
                    acc[q] = fma(df, df, acc[q]);
                }
            }
        }
#pragma unroll
        for (int q = 0; q < kCGroup; ++q) acc[q] = wave_sum(acc[q]);
        if (lane == 0) {
#pragma unroll
            for (int q = 0; q < kCGroup; ++q) s_part[w][q] = acc[q];
        }
        __syncthreads();
        if (threadIdx.x == 0) {
            for (int q = 0; q < kCGroup && c0 + q < EJ; ++q) {
                double s = s_part[0][q];
#pragma unroll
                for (int p = 1; p < kVecWaves; ++p) s += s_part[p][q];
                const int e = (c0 + q) / J;
                if ((c0 + q) % J == 0 || s < s_de[e]) s_de[e] = s;
            }
        }
        __syncthreads();
    }
    if (threadIdx.x != 0) return;
    int eb = 0;
    for (int e = 1; e < E; ++e)
        if (s_de[e] < s_de[eb]) eb = e;
    idx[2 * t] = eb;
    idx[2 * t + 1] = -1;
    g[2 * t] = 1.0f;
    g[2 * t + 1] = 0.0f;
}

template <typename T>
hipError_t launch_t(const void* x, const void* Wr, int64_t T_, int64_t d, int E, int32_t* idx,
                    float* g, hipStream_t s) {
    if (!grid_fits((T_ + kTokPerBlock - 1) / kTokPerBlock, kTokPerBlock * kWave))
        return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)((T_ + kTokPerBlock - 1) / kTokPerBlock));
    const dim3 block(kTokPerBlock * kWave);
    const T* xp = (const T*)x;
    const T* wp = (const T*)Wr;
    if (E <= 8)
        hipLaunchKernelGGL((pregate_kernel<T, 8>), grid, block, 0, s, xp, wp, T_, d, E, idx, g);
    else if (E <= 16)
        hipLaunchKernelGGL((pregate_kernel<T, 16>), grid, block, 0, s, xp, wp, T_, d, E, idx, g);
    else
        hipLaunchKernelGGL((pregate_kernel<T, 32>), grid, block, 0, s, xp, wp, T_, d, E, idx, g);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_pregate_centroid(const void* x, const void* C, int64_t T, int64_t d, int E, int J, int dtype,
                                   int32_t* idx, float* g, hipStream_t s) {
    if (T == 0) return hipSuccess;
    if (!grid_fits(T, kVecWaves * kWave)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)T), block(kVecWaves * kWave);
    const bool vec = dtype == 1 && d % 8 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)C & 15) == 0;
    if (dtype == 0)
        hipLaunchKernelGGL((pregate_centroid_kernel<float, false>), grid, block, 0, s, (const float*)x,
                           (const float*)C, d, E, J, idx, g);
    else if (vec)
        hipLaunchKernelGGL((pregate_centroid_kernel<uint16_t, true>), grid, block, 0, s, (const uint16_t*)x,
                           (const uint16_t*)C, d, E, J, idx, g);
    else
        hipLaunchKernelGGL((pregate_centroid_kernel<uint16_t, false>), grid, block, 0, s, (const uint16_t*)x,
                           (const uint16_t*)C, d, E, J, idx, g);
    return hipGetLastError();
}

hipError_t launch_pregate(const void* x, const void* Wr, int64_t T, int64_t d, int E, int dtype,
                          int32_t* idx, float* g, hipStream_t s) {
    if (dtype == 0) return launch_t<float>(x, Wr, T, d, E, idx, g, s);
    const bool vec = d % 8 == 0 && E % 8 == 0 && ((uintptr_t)x & 15) == 0 && ((uintptr_t)Wr & 15) == 0;
    if (!vec) return launch_t<uint16_t>(x, Wr, T, d, E, idx, g, s);
    if (!grid_fits(T, kVecWaves * kWave)) return hipErrorInvalidConfiguration;
    const dim3 grid((unsigned)T);
    const dim3 block(kVecWaves * kWave);
    const uint16_t* xp = (const uint16_t*)x;
    const uint16_t* wp = (const uint16_t*)Wr;
    if (E <= 8)
        hipLaunchKernelGGL((pregate_bf16_vec<8>), grid, block, 0, s, xp, wp, T, d, E, idx, g);
    else if (E <= 16)
        hipLaunchKernelGGL((pregate_bf16_vec<16>), grid, block, 0, s, xp, wp, T, d, E, idx, g);
    else
        hipLaunchKernelGGL((pregate_bf16_vec<32>), grid, block, 0, s, xp, wp, T, d, E, idx, g);
    return hipGetLastError();
}

}  // namespace dlm
