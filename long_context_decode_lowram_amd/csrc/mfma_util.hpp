// Device helpers shared by the MFMA kernels (gfx950, wave64,
// v_mfma_f32_16x16x32_bf16, direct global -> LDS copies).
#pragma once

#include <math.h>

#include "common.hpp"

namespace lowram {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ bf16x8 pack8(const f32x4& lo, const f32x4& hi) {
    bf16x8 r;
    r[0] = (__bf16)lo[0]; r[1] = (__bf16)lo[1]; r[2] = (__bf16)lo[2]; r[3] = (__bf16)lo[3];
    r[4] = (__bf16)hi[0]; r[5] = (__bf16)hi[1]; r[6] = (__bf16)hi[2]; r[7] = (__bf16)hi[3];
    return r;
}

// s_waitcnt on the vector-memory counter alone (gfx9 encoding: vmcnt in
// bits 3:0 and 15:14; expcnt and lgkmcnt at their maxima mean "no wait").
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt out of range");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4)); }
// s_waitcnt on the LDS/scalar-memory counter alone (lgkmcnt in bits 11:8).
template <int N>
__device__ __forceinline__ void wait_lgkmcnt() {
    static_assert(N >= 0 && N < 16, "lgkmcnt out of range");
    __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4) | (N << 8));
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Workgroup barrier for the main loop. __syncthreads() would also wait for
// every direct-to-LDS load still in flight (they count as LDS stores), which
// includes the next chunk's A rows; here the caller has already waited for
// the loads the other waves need, so only this wave's LDS operations are
// drained. The empty asm statements keep the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
    wait_lgkmcnt0();
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Direct global -> LDS copy of 16 bytes per lane: lane i's bytes land at
// lds + 16 i (in lane order), read from byte voff + soff of the buffer;
// reads past the buffer's end produce zeros.
// POLICY is the load's cache-policy field; kNonTemporal marks data read once.
constexpr int kNonTemporal = 2;
template <int POLICY = 0>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds, 16, voff, soff, 0, POLICY);
}

// Read of one 16-byte LDS piece at byte offset `off` of `base`.
__device__ __forceinline__ bf16x8 lds16(const void* base, uint32_t off) {
    return as_bf16x8(*reinterpret_cast<const u32x4*>(static_cast<const unsigned char*>(base) + off));
}

// The normal tail Q(a) = 1 - Phi(a) for a in [0, 6] (clamped): log2 Q(a) is a
// degree-4 polynomial in a (gelu_tail_fit.py derives the constants; GELU from
// it is within 6.4e-6 of the exact one).
__device__ __forceinline__ float normal_tail(float a) {
    constexpr float c0 = -1.0004796981811523f, c1 = -1.1473716497421265f, c2 = -0.4680161774158478f,
                    c3 = -0.04407823458313942f, c4 = 0.003866035956889391f;
    a = __builtin_amdgcn_fmed3f(a, 0.0f, 6.0f);
    float p = fmaf(c4, a, c3);
    p = fmaf(p, a, c2);
    p = fmaf(p, a, c1);
    p = fmaf(p, a, c0);
    return __builtin_amdgcn_exp2f(p);
}

// GELU(x) = x Phi(x) = max(x, 0) - |x| Q(|x|) with the normal tail
// Q(a) = 1 - Phi(a). Here log2 Q(a) is a degree-3 polynomial in a whose cubic
// coefficient is negative (a weighted near-minimax fit on [0, 6];
// gelu_tail_fit.py derives the constants and bounds the float32 evaluation:
// |error| < 5.6e-5 over [-12, 12], below the bf16 rounding the result goes
// through next). Past 6 the polynomial keeps falling, so |x| 2^P(|x|) stays
// below 3e-9 with no clamp. Per element: three multiply-adds on |x| (a source
// modifier), one exp2, one v_med3 for max(x, 0) (finite inputs; it needs none
// of the quieting steps an IEEE max would add) and one multiply-add.
__device__ __forceinline__ void gelu_tail16(f32x4 (&z)[4]) {
    constexpr float c0 = -1.0035271644592285f, c1 = -1.129267930984497f, c2 = -0.49879294633865356f,
                    c3 = -0.024894719943404198f;
    // Sixteen independent chains, evaluated step by step so their latencies overlap.
    float p[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) p[k] = fmaf(c3, fabsf(z[k >> 2][k & 3]), c2);
#pragma unroll
    for (int k = 0; k < 16; ++k) p[k] = fmaf(p[k], fabsf(z[k >> 2][k & 3]), c1);
#pragma unroll
    for (int k = 0; k < 16; ++k) p[k] = fmaf(p[k], fabsf(z[k >> 2][k & 3]), c0);
#pragma unroll
    for (int k = 0; k < 16; ++k) p[k] = __builtin_amdgcn_exp2f(p[k]);
#pragma unroll
    for (int k = 0; k < 16; ++k)
        z[k >> 2][k & 3] = fmaf(-fabsf(z[k >> 2][k & 3]), p[k], __builtin_amdgcn_fmed3f(z[k >> 2][k & 3], 0.0f, 3.0e38f));
}

}  // namespace lowram
