// Shared device helpers for the liblowram kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowram {

enum : int { DT_F32 = 0, DT_BF16 = 1, DT_I8 = 2, DT_I2 = 3 };

// Residual encodings that carry a per-row scale (int8 codes, 2-bit codes).
constexpr bool res_scaled(int dt) { return dt == DT_I8 || dt == DT_I2; }

constexpr int kHeadDim = 128;   // head_dim the kernels are built for
constexpr int kBlock = 64;      // tokens per cache block
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 bits, round to nearest even (NaN kept quiet). Written
// with selects, not branches, so a wave never splits on it.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    const uint32_t rounded = (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    return static_cast<uint16_t>((u & 0x7fffffffu) > 0x7f800000u ? ((u >> 16) | 0x40u) : rounded);
}

// binary64 -> bfloat16 bits with one round-to-nearest-even step: first to
// float32 with round-to-odd (truncate, then set the last bit if anything was
// dropped), then float32 -> bfloat16 nearest-even. Float32 keeps 16 more
// bits than bfloat16 at every exponent, so the two steps round exactly like
// one.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
    const float f = static_cast<float>(x);
    const double back = static_cast<double>(f);
    const uint32_t u = __float_as_uint(f);
    const uint32_t odd = (u - (fabs(back) > fabs(x) ? 1u : 0u)) | 1u;
    return f32_to_bf16_bits(__uint_as_float(back != x && x == x ? odd : u));
}

// Element load of a stored tensor as float (int8 returns the raw code).
template <int DT> __device__ __forceinline__ float ld(const void* p, int64_t i);
template <> __device__ __forceinline__ float ld<DT_F32>(const void* p, int64_t i) {
    return static_cast<const float*>(p)[i];
}
template <> __device__ __forceinline__ float ld<DT_BF16>(const void* p, int64_t i) {
    return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
}
template <> __device__ __forceinline__ float ld<DT_I8>(const void* p, int64_t i) {
    return static_cast<float>(static_cast<const int8_t*>(p)[i]);
}
// 2-bit codes, four per byte (element i in bits 2(i mod 4) of byte i / 4):
// returns the unscaled level q - 1.5.
template <> __device__ __forceinline__ float ld<DT_I2>(const void* p, int64_t i) {
    const unsigned b = static_cast<const uint8_t*>(p)[i >> 2];
    return static_cast<float>((b >> (2 * (i & 3))) & 3u) - 1.5f;
}

template <int DT> __device__ __forceinline__ void st(void* p, int64_t i, float v);
template <> __device__ __forceinline__ void st<DT_F32>(void* p, int64_t i, float v) {
    static_cast<float*>(p)[i] = v;
}
template <> __device__ __forceinline__ void st<DT_BF16>(void* p, int64_t i, float v) {
    static_cast<uint16_t*>(p)[i] = f32_to_bf16_bits(v);
}

// A raw buffer descriptor over [base, base + bytes): loads at offsets past
// the end return zeros instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ float gelu_erf(float x) {
    return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f));
}

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Per-call constants shared by the decode kernels (passed by value).
struct DecodeParams {
    int batch, ctx_len, n_q, n_kv, group, rank, hidden, n_res, n_blocks, win_len, win_cap;
    int part_stride;       // floats per partial record: 2 + hidden + head_dim, rounded up
    int n_split;           // partial records per (b, query head)
    int blocks_per_split;  // attended blocks folded into one partial record
    float scale;           // 1/sqrt(head_dim)
    const void* q; const void* a; const float* a_scale; const void* b_l;
    const void* w_lin; const void* w1; const void* b1; const void* w2; const void* b2;
    const int32_t* res_idx; const void* res_val; const float* res_scale; const int32_t* res_ptr;
    const int32_t* sel; const uint8_t* keep; const void* win_k; const void* win_v;
    void* out; int32_t* stats;
    // workspace
    int32_t* att_list;     // [B, n_blocks]
    int32_t* att_count;    // [B]
    float* partials;       // [B, Hq, n_split, part_stride]
    int32_t* counts;       // [B, Hkv, n_split, 2]
    int n_sel;
    int att_direct;        // no eviction flags: the attended blocks are sel (or all blocks) as given
    const int32_t* win_len_dev;   // window length read at run time (clamped to [0, win_len]), or null
    uint32_t* check_flags;        // validate mode: defect bits are ORed in here, else null
};

// Window tokens attended by this call: win_len, or the device-held count
// clamped to [0, win_len] (win_len is then the capacity the host checked).
__device__ __forceinline__ int window_len(const DecodeParams& p) {
    if (p.win_len_dev == nullptr) return p.win_len;
    return min(max(*p.win_len_dev, 0), p.win_len);
}

// Attended block i of sequence b, or -1 for an entry outside the cache. With
// eviction flags the assembly kernel has compacted the kept blocks into
// att_list; without them the list is the selection itself (every block when
// there is none), read in place.
__device__ __forceinline__ int attended_block(const DecodeParams& p, int b, int i) {
    if (p.att_direct) {
        const int blk = p.sel ? p.sel[(int64_t)b * p.n_sel + i] : i;
        return (blk >= 0 && blk < p.n_blocks) ? blk : -1;
    }
    return p.att_list[(int64_t)b * p.n_blocks + i];
}
__device__ __forceinline__ int attended_count(const DecodeParams& p, int b) {
    return p.att_direct ? (p.sel ? p.n_sel : p.n_blocks) : p.att_count[b];
}

}  // namespace lowram
