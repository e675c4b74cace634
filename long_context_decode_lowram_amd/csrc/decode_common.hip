// Attended-set assembly and the split-K combine of the decode step.
#include <math.h>

#include "kernels.hpp"

namespace lowram {

// For each sequence: the selected blocks (all when sel is NULL) that keep
// marks kept, in the order given, compacted into att_list[b]. Entries outside
// [0, n_blocks) are dropped, so later kernels never index past the cache.
__global__ __launch_bounds__(256) void assemble_kernel(DecodeParams p) {
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int n_cand = p.sel ? p.n_sel : p.n_blocks;
    __shared__ int wave_tot[4];
    int base = 0;
    for (int c0 = 0; c0 < n_cand; c0 += 256) {
        const int c = c0 + tid;
        int blk = -1;
        bool ok = false;
        if (c < n_cand) {
            blk = p.sel ? p.sel[(int64_t)b * p.n_sel + c] : c;
            ok = blk >= 0 && blk < p.n_blocks &&
                 (p.keep == nullptr || p.keep[(int64_t)b * p.n_blocks + blk] != 0);
        }
        const unsigned long long m = __ballot(ok);
        const int pre = __popcll(m & ((1ull << lane) - 1ull));
        if (lane == 0) wave_tot[w] = __popcll(m);
        __syncthreads();
        int off = base;
        for (int i = 0; i < w; ++i) off += wave_tot[i];
        if (ok) p.att_list[(int64_t)b * p.n_blocks + off + pre] = blk;
        base += wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
        __syncthreads();
    }
    if (tid == 0) p.att_count[b] = base;
}

hipError_t launch_assemble(const DecodeParams& p, hipStream_t s) {
    hipLaunchKernelGGL(assemble_kernel, dim3(p.batch), dim3(256), 0, s, p);
    return hipGetLastError();
}

__device__ __forceinline__ float block_reduce(float v, float* red, bool is_max) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    v = is_max ? wave_max(v) : wave_sum(v);
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float r = red[0];
    for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = is_max ? fmaxf(r, red[i]) : r + red[i];
    return r;
}

// One workgroup per (query head j, sequence b). A partial record is
// (m, l, O[0:hidden], O[hidden:hidden+d]) where m is the running max of the
// scaled scores, l = sum exp(s - m) over its tokens, O[0:hidden] the
// p-weighted sum of the predictor's hidden activations gelu(k W1 + b1) and
// O[hidden:] the p-weighted sum of k W_lin plus residuals. The output is
//   (O_G W2 + O_V + L b2 + sum_window p v) / (L + L_window)
// after rescaling every record to the common max; W2 and b2 are linear and
// the weights p sum to L, so applying them after the weighted sum gives the
// predictor's value for every token exactly (up to rounding).
template <int ACT>
__global__ __launch_bounds__(256) void combine_kernel(DecodeParams p) {
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int h = j / p.group, H = p.hidden, S = p.part_stride;
    const int nsplit = min(p.n_split, (p.att_count[b] + p.blocks_per_split - 1) / p.blocks_per_split);
    const int nw = p.win_len;
    const float* P = p.partials + ((int64_t)b * p.n_q + j) * p.n_split * (int64_t)S;
    extern __shared__ float sm[];
    float* es = sm;                       // [n_split]
    float* sw = es + p.n_split;           // [win_len]
    float* oc = sw + nw;                  // [H + 128]
    float* qs = oc + H + kHeadDim;        // [128]
    float* red = qs + kHeadDim;           // [8 + 128]: block reductions, then the second half-sums

    for (int f = tid; f < kHeadDim; f += blockDim.x)
        qs[f] = ld<ACT>(p.q, ((int64_t)b * p.n_q + j) * kHeadDim + f);
    __syncthreads();

    float mx = -INFINITY;
    for (int s = tid; s < nsplit; s += blockDim.x) mx = fmaxf(mx, P[(int64_t)s * S]);
    for (int u = tid; u < nw; u += blockDim.x) {
        const int64_t row = (((int64_t)b * p.win_cap + u) * p.n_kv + h) * kHeadDim;
        float acc = 0.f;
        for (int n = 0; n < kHeadDim; ++n) acc += qs[n] * ld<ACT>(p.win_k, row + n);
        acc *= p.scale;
        sw[u] = acc;
        mx = fmaxf(mx, acc);
    }
    const float M = block_reduce(mx, red, true);

    const int64_t out_row = ((int64_t)b * p.n_q + j) * kHeadDim;
    if (M == -INFINITY) {   // nothing attended for this sequence
        for (int f = tid; f < kHeadDim; f += blockDim.x) st<ACT>(p.out, out_row + f, 0.f);
    } else {
        float lt = 0.f, lw = 0.f;
        for (int s = tid; s < nsplit; s += blockDim.x) {
            const float m = P[(int64_t)s * S];
            const float e = (m == -INFINITY) ? 0.f : expf(m - M);
            es[s] = e;
            lt += e * P[(int64_t)s * S + 1];
        }
        for (int u = tid; u < nw; u += blockDim.x) {
            const float e = expf(sw[u] - M);
            sw[u] = e;
            lw += e;
        }
        const float Lt = block_reduce(lt, red, false);
        const float Lw = block_reduce(lw, red, false);
        for (int f = tid; f < H + kHeadDim; f += blockDim.x) {
            float acc = 0.f;
            for (int s = 0; s < nsplit; ++s) acc += es[s] * P[(int64_t)s * S + 2 + f];
            oc[f] = acc;
        }
        __syncthreads();
        // out[f] = (sum_i O_G[i] W2[f][i] + O_V[f] + L b2[f] + window) / (L + L_w):
        // two threads per output feature, each half of the W2 row in 16-byte loads.
        const float inv = 1.0f / (Lt + Lw);
        const int f = tid & (kHeadDim - 1), half = tid >> 7;      // blockDim.x == 256
        const int64_t w2row = (((int64_t)b * p.n_kv + h) * kHeadDim + f) * H;
        const int i0 = half * (H / 2), i1 = i0 + H / 2;
        float y = 0.f;
        if (ACT == DT_BF16) {
            const uint4* wv = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.w2) + w2row + i0);
            for (int c = 0; c < (i1 - i0) / 8; ++c) {
                const uint4 u = wv[c];
                const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int i = i0 + 8 * c + 2 * k;
                    y += oc[i] * __uint_as_float(wd[k] << 16) + oc[i + 1] * __uint_as_float(wd[k] & 0xffff0000u);
                }
            }
        } else {
            for (int i = i0; i < i1; ++i) y += oc[i] * ld<ACT>(p.w2, w2row + i);
        }
        if (half == 1) {
            y += oc[H + f];
            if (p.b2) y += Lt * ld<ACT>(p.b2, ((int64_t)b * p.n_kv + h) * kHeadDim + f);
            for (int u = 0; u < nw; ++u)
                y += sw[u] * ld<ACT>(p.win_v, (((int64_t)b * p.win_cap + u) * p.n_kv + h) * kHeadDim + f);
            red[8 + f] = y;
        }
        __syncthreads();
        if (half == 0) st<ACT>(p.out, out_row + f, (y + red[8 + f]) * inv);
    }
    if (p.stats != nullptr && j % p.group == 0 && tid == 0) {
        int tok = 0, res = 0;
        const int32_t* c = p.counts + ((int64_t)b * p.n_kv + h) * p.n_split * 2;
        for (int s = 0; s < nsplit; ++s) {
            tok += c[2 * s];
            res += c[2 * s + 1];
        }
        p.stats[((int64_t)b * p.n_kv + h) * 2 + 0] = tok + nw;
        p.stats[((int64_t)b * p.n_kv + h) * 2 + 1] = res;
    }
}

size_t combine_smem_bytes(const DecodeParams& p) {
    return sizeof(float) * ((size_t)p.n_split + p.win_len + p.hidden + 3 * kHeadDim + 8);
}

hipError_t launch_combine(const DecodeParams& p, int act, hipStream_t s) {
    const size_t smem = combine_smem_bytes(p);
    if (act == DT_F32)
        hipLaunchKernelGGL(combine_kernel<DT_F32>, dim3(p.n_q, p.batch), dim3(256), smem, s, p);
    else
        hipLaunchKernelGGL(combine_kernel<DT_BF16>, dim3(p.n_q, p.batch), dim3(256), smem, s, p);
    return hipGetLastError();
}

}  // namespace lowram
