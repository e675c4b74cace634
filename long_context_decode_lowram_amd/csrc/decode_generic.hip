// Generic fp32 SIMT decode kernel: every dtype combination, scalar FMA math.
// It is the float32 path (fp32 activations) and the cross-check for the
// MFMA kernel on bf16 data. One workgroup per (attended block, KV head, b).
#include <math.h>

#include "kernels.hpp"

namespace lowram {

namespace {
constexpr int kThreads = 256;
constexpr int kChunk = 32;           // rank columns per LDS stage
constexpr int kKtStride = kBlock + 1;
constexpr int kAsStride = kChunk + 1;
constexpr int kMaxGroup = 8;
}  // namespace

template <int ACT, int ADT, int RDT>
__global__ __launch_bounds__(kThreads) void decode_generic_kernel(DecodeParams p) {
    const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
    const int G = p.group, H = p.hidden, S = p.part_stride, R = p.rank;
    const int lane = tid & 63, w = tid >> 6;

    auto rec = [&](int jj) -> float* {
        return p.partials + (((int64_t)b * p.n_q + h * G + jj) * p.n_split + i) * (int64_t)S;
    };
    int32_t* cnt_rec = p.counts + (((int64_t)b * p.n_kv + h) * p.n_split + i) * 2;

    const int blk = i < attended_count(p, b) ? attended_block(p, b, i) : -1;
    if (blk < 0) {
        for (int jj = 0; jj < G; ++jj)
            for (int f = tid; f < S; f += kThreads) rec(jj)[f] = (f == 0) ? -INFINITY : 0.f;
        if (tid == 0) { cnt_rec[0] = 0; cnt_rec[1] = 0; }
        return;
    }
    const int t0 = blk * kBlock;
    const int nt = min(kBlock, p.ctx_len - t0);

    __shared__ float smem[kHeadDim * kKtStride + kBlock * kAsStride + kHeadDim * kAsStride];
    float* KT = smem;                                 // [128][65]  K^T of the block, this head
    float* As = KT + kHeadDim * kKtStride;            // [64][33]   A chunk
    float* Bs = As + kBlock * kAsStride;              // [128][33]  B_l chunk (head rows)
    float* Qs = As;                                   // [G][128]   after the K loop
    float* Ps = Qs + kMaxGroup * kHeadDim;            // [G][64]
    __shared__ float mrow[kMaxGroup], lrow[kMaxGroup];

    // 1. K = A_blk . B_l for this head's 128 columns, fp32 accumulation.
    {
        const int tt = tid & 63, ng = tid >> 6;
        float acc[32];
#pragma unroll
        for (int n = 0; n < 32; ++n) acc[n] = 0.f;
        for (int c0 = 0; c0 < R; c0 += kChunk) {
            for (int e = tid; e < kBlock * kChunk; e += kThreads) {
                const int rr = e / kChunk, cc = e % kChunk;
                float v = 0.f;
                if (rr < nt) {
                    const int64_t t = (int64_t)b * p.ctx_len + t0 + rr;
                    v = ld<ADT>(p.a, t * R + c0 + cc);
                    if (ADT == DT_I8) v *= p.a_scale[t];
                }
                As[rr * kAsStride + cc] = v;
            }
            for (int e = tid; e < kHeadDim * kChunk; e += kThreads) {
                const int nn = e / kChunk, cc = e % kChunk;
                Bs[nn * kAsStride + cc] =
                    ld<ACT>(p.b_l, ((int64_t)b * p.n_kv * kHeadDim + h * kHeadDim + nn) * R + c0 + cc);
            }
            __syncthreads();
            for (int cc = 0; cc < kChunk; ++cc) {
                const float av = As[tt * kAsStride + cc];
#pragma unroll
                for (int n = 0; n < 32; ++n) acc[n] += av * Bs[(ng * 32 + n) * kAsStride + cc];
            }
            __syncthreads();
        }
#pragma unroll
        for (int n = 0; n < 32; ++n) KT[(ng * 32 + n) * kKtStride + tt] = acc[n];
    }
    for (int e = tid; e < G * kHeadDim; e += kThreads)
        Qs[e] = ld<ACT>(p.q, ((int64_t)b * p.n_q + h * G) * kHeadDim + e);
    __syncthreads();

    // 2. Scores and the block-local softmax statistics, one wave per query head.
    for (int jj = w; jj < G; jj += kThreads / kWave) {
        float s = -INFINITY;
        if (lane < nt) {
            float a = 0.f;
            for (int n = 0; n < kHeadDim; ++n) a += Qs[jj * kHeadDim + n] * KT[n * kKtStride + lane];
            s = a * p.scale;
        }
        const float m = wave_max(s);
        const float e = (lane < nt) ? expf(s - m) : 0.f;
        const float l = wave_sum(e);
        Ps[jj * kBlock + lane] = e;
        if (lane == 0) { mrow[jj] = m; lrow[jj] = l; }
    }
    __syncthreads();

    // Residual slots of this block (clamped so garbage pointers stay in range).
    const int64_t ptr_row = ((int64_t)b * p.n_kv + h) * (p.n_blocks + 1);
    int lo = p.res_ptr[ptr_row + blk], hi = p.res_ptr[ptr_row + blk + 1];
    lo = max(0, min(lo, p.n_res));
    hi = max(lo, min(hi, p.n_res));
    const int64_t res_row = ((int64_t)b * p.n_kv + h) * p.n_res;

    // 3. Predictor features per token, p-weighted over the block:
    //    f < H      : gelu(k . W1[f] + b1[f])
    //    f >= H     : k . W_lin[f - H]  plus the stored residuals.
    for (int f = tid; f < H + kHeadDim; f += kThreads) {
        const bool is_g = f < H;
        const int64_t wrow = is_g ? (((int64_t)b * p.n_kv + h) * H + f) * kHeadDim
                                  : (((int64_t)b * p.n_kv + h) * kHeadDim + (f - H)) * kHeadDim;
        const void* W = is_g ? p.w1 : p.w_lin;
        float z[kBlock];
#pragma unroll
        for (int t = 0; t < kBlock; ++t) z[t] = 0.f;
        for (int n = 0; n < kHeadDim; ++n) {
            const float wv = ld<ACT>(W, wrow + n);
#pragma unroll
            for (int t = 0; t < kBlock; ++t) z[t] += KT[n * kKtStride + t] * wv;
        }
        if (is_g) {
            const float bb = p.b1 ? ld<ACT>(p.b1, ((int64_t)b * p.n_kv + h) * H + f) : 0.f;
#pragma unroll
            for (int t = 0; t < kBlock; ++t) z[t] = gelu_erf(z[t] + bb);
        }
        for (int jj = 0; jj < G; ++jj) {
            float o = 0.f;
#pragma unroll
            for (int t = 0; t < kBlock; ++t) o += Ps[jj * kBlock + t] * z[t];
            if (!is_g) {
                for (int q = lo; q < hi; ++q) {
                    const int tl = p.res_idx[res_row + q] - t0;
                    if (tl < 0 || tl >= nt) continue;
                    float rv = ld<RDT>(p.res_val, (res_row + q) * kHeadDim + (f - H));
                    if (res_scaled(RDT)) rv *= p.res_scale[res_row + q];
                    o += Ps[jj * kBlock + tl] * rv;
                }
            }
            rec(jj)[2 + f] = o;
        }
    }
    if (tid < G) {
        rec(tid)[0] = mrow[tid];
        rec(tid)[1] = lrow[tid];
    }
    if (tid == 0) {
        int applied = 0;
        for (int q = lo; q < hi; ++q) {
            const int tl = p.res_idx[res_row + q] - t0;
            applied += (tl >= 0 && tl < nt) ? 1 : 0;
        }
        cnt_rec[0] = nt;
        cnt_rec[1] = applied;
    }
}

template <int ACT, int ADT>
static hipError_t launch_r(const DecodeParams& p, int rdt, hipStream_t s) {
    const dim3 grid(p.n_split, p.n_kv, p.batch);
    switch (rdt) {
        case DT_F32: hipLaunchKernelGGL((decode_generic_kernel<ACT, ADT, DT_F32>), grid, dim3(kThreads), 0, s, p); break;
        case DT_BF16: hipLaunchKernelGGL((decode_generic_kernel<ACT, ADT, DT_BF16>), grid, dim3(kThreads), 0, s, p); break;
        case DT_I8: hipLaunchKernelGGL((decode_generic_kernel<ACT, ADT, DT_I8>), grid, dim3(kThreads), 0, s, p); break;
        default: hipLaunchKernelGGL((decode_generic_kernel<ACT, ADT, DT_I2>), grid, dim3(kThreads), 0, s, p); break;
    }
    return hipGetLastError();
}

template <int ACT>
static hipError_t launch_a(const DecodeParams& p, int adt, int rdt, hipStream_t s) {
    switch (adt) {
        case DT_F32: return launch_r<ACT, DT_F32>(p, rdt, s);
        case DT_BF16: return launch_r<ACT, DT_BF16>(p, rdt, s);
        default: return launch_r<ACT, DT_I8>(p, rdt, s);
    }
}

hipError_t launch_decode_generic(const DecodeParams& p, int act, int adt, int rdt, hipStream_t s) {
    return act == DT_F32 ? launch_a<DT_F32>(p, adt, rdt, s) : launch_a<DT_BF16>(p, adt, rdt, s);
}

}  // namespace lowram
