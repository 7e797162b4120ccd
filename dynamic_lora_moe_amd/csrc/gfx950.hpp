// gfx950 (CDNA4) device helpers shared by the kernels of this library:
// bf16 <-> fp32 conversion, 128-bit global access, the bf16 MFMA shapes used,
// and wave64 reductions.  Compiled for gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dlm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// A bf16 is the upper half of an fp32: widening is a shift / mask.
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf_to_f(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
    bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint16_t f_to_bf(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

// Global-memory accesses go through address_space(1) pointers so they compile
// to global_* instructions.  Generic pointers (e.g. read from a descriptor
// table) would give flat_* instructions, which also count against the LDS
// wait counter: every LDS wait would then drain all in-flight HBM loads.
template <typename T> using gptr = __attribute__((address_space(1))) T*;
template <typename T> using gcptr = __attribute__((address_space(1))) const T*;

template <typename T> __device__ __forceinline__ T gld(const T* p) { return *(gcptr<T>)p; }
template <typename T> __device__ __forceinline__ void gst(T* p, T v) { *(gptr<T>)p = v; }

// 128-bit global load/store.  `nt` marks streaming data that is touched once
// (weights being switched or multiplied, x rows, y rows) so it does not evict
// reused adapter slices from L2.
__device__ __forceinline__ u32x4 ld128(const void* p) { return *(gcptr<u32x4>)p; }
__device__ __forceinline__ u32x4 ld128_nt(const void* p) {
    return __builtin_nontemporal_load((gcptr<u32x4>)p);
}
__device__ __forceinline__ void st128(void* p, u32x4 v) { *(gptr<u32x4>)p = v; }
__device__ __forceinline__ void st128_nt(void* p, u32x4 v) {
    __builtin_nontemporal_store(v, (gptr<u32x4>)p);
}

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies row (l % 32) of A and column (l % 32) of B, 8 consecutive k
// each (the two half-waves cover the two k halves).  Output register a of lane
// l holds D[8*(a/4) + 4*(l/32) + a%4][l % 32].
__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Direct global -> LDS copy, 16 bytes per lane (global_load_lds_dwordx4): lane
// L's 16 bytes land at lds + 16 L, so one wave instruction fills 1 KB of LDS.
// `lds` must be the same for every lane.  The copy is a vector-memory
// instruction: its data is in LDS once the wave's vmcnt has passed it.
__device__ __forceinline__ void copy16_to_lds(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((gcptr<void>)g, (__attribute__((address_space(3))) void*)lds, 16, 0, 0);
}
// The same for data read once (the nt cache policy, so it does not displace
// data that is reused from L2).
__device__ __forceinline__ void copy16_to_lds_nt(const void* g, void* lds) {
    __builtin_amdgcn_global_load_lds((gcptr<void>)g, (__attribute__((address_space(3))) void*)lds, 16, 0, 2);
}

// Wait until at most N vector-memory instructions of this wave are in flight.
// gfx9 s_waitcnt immediate: vmcnt in bits [3:0] and [15:14], expcnt [6:4] and
// lgkmcnt [11:8] left at their maxima (not waited for).  Vector-memory loads,
// stores and LDS copies retire from vmcnt in issue order.
template <int N> __device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same for a wave-uniform count known only at run time, n <= NMAX.
template <int NMAX> __device__ __forceinline__ void wait_vmcnt_le(int n) {
    if constexpr (NMAX == 0) {
        wait_vmcnt<0>();
    } else {
        if (n >= NMAX) wait_vmcnt<NMAX>();
        else wait_vmcnt_le<NMAX - 1>(n);
    }
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }
// Wave index within the workgroup, marked wave-uniform (an SGPR): control flow
// that depends on it stays scalar instead of running under exec masks.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x / kWave); }

// A value every lane of the wave holds identically (e.g. read from LDS),
// moved to an SGPR so loops and branches on it stay scalar.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Butterfly sum over the 64 lanes; every lane gets the total, in the same
// fixed order on every run.
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

}  // namespace dlm
