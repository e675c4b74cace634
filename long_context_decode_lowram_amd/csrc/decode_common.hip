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

// Validate mode: one workgroup per (b, KV head) row of the residual store,
// plus one per sequence for its selection row (blockIdx.y == 1) and the
// window count. Every read stays inside the documented shapes; a defect ORs
// its bit into *check_flags (only defective threads write).
__device__ __forceinline__ void flag(uint32_t* f, uint32_t bit) {
    __hip_atomic_fetch_or(f, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__global__ __launch_bounds__(256) void validate_kernel(DecodeParams p) {
    const int tid = threadIdx.x;
    if (blockIdx.y == 1) {
        const int b = blockIdx.x;
        if (b >= p.batch) return;
        if (b == 0 && tid == 0 && p.win_len_dev != nullptr) {
            const int w = *p.win_len_dev;
            if (w < 0 || w > p.win_len) flag(p.check_flags, kCheckWinLen);
        }
        if (p.sel == nullptr) return;
        // In-range entries strictly ascending, padding (outside [0, nb))
        // anywhere: each in-range entry is compared with the previous one.
        const int32_t* row = p.sel + (int64_t)b * p.n_sel;
        bool bad = false;
        for (int i = tid; i < p.n_sel; i += blockDim.x) {
            const int cur = row[i];
            if (cur < 0 || cur >= p.n_blocks) continue;
            int prev = -1;
            for (int k = i - 1; k >= 0; --k) {
                const int v = row[k];
                if (v >= 0 && v < p.n_blocks) { prev = v; break; }
            }
            bad |= prev >= cur;
        }
        if (bad) flag(p.check_flags, kCheckSelOrder);
        return;
    }
    const int bh = blockIdx.x;                  // b * n_kv + h
    const int32_t* idx = p.res_idx + (int64_t)bh * p.n_res;
    const int32_t* ptr = p.res_ptr + (int64_t)bh * (p.n_blocks + 1);
    uint32_t bits = 0;
    for (int s = tid; s < p.n_res; s += blockDim.x) {
        const int t = idx[s];
        if (t < 0 || t >= p.ctx_len) { bits |= kCheckResRange; continue; }
        if (s > 0 && idx[s - 1] >= t) bits |= kCheckResOrder;
        const int blk = t / kBlock;
        if (!(ptr[blk] <= s && s < ptr[blk + 1])) bits |= kCheckResPtr;
    }
    for (int i = tid; i <= p.n_blocks; i += blockDim.x) {
        const int v = ptr[i];
        if ((i == 0 && v != 0) || (i == p.n_blocks && v != p.n_res) || (i > 0 && ptr[i - 1] > v))
            bits |= kCheckResPtr;
    }
    if (bits) flag(p.check_flags, bits);
}

hipError_t launch_validate(const DecodeParams& p, hipStream_t s) {
    const int rows = p.batch * p.n_kv;
    hipLaunchKernelGGL(validate_kernel, dim3((unsigned)max(rows, p.batch), 2), dim3(256), 0, s, p);
    return hipGetLastError();
}

// Window append: workgroup l copies the new rows of layer l (all sequences)
// into slot win_len_dev[l] of its buffers, then advances the count. The
// count is read once, before the barrier, by every thread; one thread writes
// it after the barrier, so no thread of the workgroup reads the new value.
__global__ __launch_bounds__(256) void window_append_kernel(WindowParams p) {
    const int l = blockIdx.x;
    const int pos = p.win_len[l];
    __syncthreads();
    if (pos < 0 || pos >= p.win_cap) return;     // full (or bad) buffer: nothing written, count kept
    const int pieces = p.width * p.elem_bytes / 16;           // 16-byte pieces per row
    const int64_t n = (int64_t)p.batch * pieces;
    const uint4* nk = reinterpret_cast<const uint4*>(static_cast<const char*>(p.new_k) + (int64_t)l * p.batch * p.width * p.elem_bytes);
    const uint4* nv = reinterpret_cast<const uint4*>(static_cast<const char*>(p.new_v) + (int64_t)l * p.batch * p.width * p.elem_bytes);
    uint4* wk = reinterpret_cast<uint4*>(static_cast<char*>(p.win_k) + (int64_t)l * p.batch * p.win_cap * p.width * p.elem_bytes);
    uint4* wv = reinterpret_cast<uint4*>(static_cast<char*>(p.win_v) + (int64_t)l * p.batch * p.win_cap * p.width * p.elem_bytes);
    for (int64_t e = threadIdx.x; e < n; e += blockDim.x) {
        const int64_t b = e / pieces, c = e % pieces;
        const int64_t dst = (b * p.win_cap + pos) * pieces + c;
        wk[dst] = nk[e];
        wv[dst] = nv[e];
    }
    if (threadIdx.x == 0) p.win_len[l] = pos + 1;
}

hipError_t launch_window_append(const WindowParams& p, hipStream_t s) {
    hipLaunchKernelGGL(window_append_kernel, dim3(p.n_layers), dim3(256), 0, s, p);
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
constexpr int kCombWaves = 8;
constexpr int kCombThreads = kCombWaves * 64;

template <int ACT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(DecodeParams p) {
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    const int h = j / p.group, H = p.hidden, S = p.part_stride, nf = H + kHeadDim;
    const int nsplit = min(p.n_split, (attended_count(p, b) + p.blocks_per_split - 1) / p.blocks_per_split);
    const int nw = window_len(p);         // at most p.win_len, which sizes sw
    const float* P = p.partials + ((int64_t)b * p.n_q + j) * p.n_split * (int64_t)S;
    extern __shared__ float sm[];
    float* sw = sm;                       // [win_len]
    float* oc = sw + p.win_len;           // [H + 128]
    float* red = oc + nf + kHeadDim;      // [8 + 3 * 128]: block reductions, then the W2 quarter sums
    float* part = red + 8 + 3 * kHeadDim; // [8][H + 128]: the waves' record sums
    float* wml = part + kCombWaves * nf;  // [8][2]: each wave's max and weight sum

    // out[f] takes four threads, a quarter of the W2 row each; the first 256
    // bytes of that quarter are loaded now, before anything they wait on.
    const int f_out = tid & (kHeadDim - 1), quarter = tid >> 7;
    const int64_t w2row = (((int64_t)b * p.n_kv + h) * kHeadDim + f_out) * H;
    const int i0 = quarter * (H / 4), n_c = (H / 4) / 8;       // 16-byte pieces of the quarter
    const bool w2_vec = ACT == DT_BF16 && H % 32 == 0;
    const uint4* w2v = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(p.w2) + w2row + i0);
    uint4 w2pre[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) w2pre[c] = (w2_vec && c < n_c) ? w2v[c] : make_uint4(0u, 0u, 0u, 0u);

    // Records: wave wv merges the splits wv, wv+8, ... eight at a time, with
    // a running max (every sum is rescaled to it as it grows), so the loads of
    // a batch's maxima, weight sums and O rows are in flight together. Lane
    // takes the features lane + 64 i, six at a time: each load of the wave
    // reads 256 consecutive bytes of one record.
    for (int f0 = 0; f0 < nf; f0 += 64 * 6) {
        float mrun = -INFINITY, lrun = 0.f;
        float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s0 = wv; s0 < nsplit; s0 += kCombWaves * 8) {
            float mb[8], lb[8], v[8][6];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int sp = s0 + kCombWaves * u;
                const bool ok = sp < nsplit;
                const float* rec = P + (int64_t)(ok ? sp : 0) * S;
                mb[u] = ok ? rec[0] : -INFINITY;
                lb[u] = ok ? rec[1] : 0.f;
#pragma unroll
                for (int i = 0; i < 6; ++i) {
                    const int fi = f0 + lane + 64 * i;
                    v[u][i] = (ok && fi < nf) ? rec[2 + fi] : 0.f;
                }
            }
            float mnew = mrun;
#pragma unroll
            for (int u = 0; u < 8; ++u) mnew = fmaxf(mnew, mb[u]);
            const float r = mrun == -INFINITY ? 0.f : expf(mrun - mnew);
            lrun *= r;
#pragma unroll
            for (int i = 0; i < 6; ++i) acc[i] *= r;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const float e = mb[u] == -INFINITY ? 0.f : expf(mb[u] - mnew);
                lrun += e * lb[u];
#pragma unroll
                for (int i = 0; i < 6; ++i) acc[i] += e * v[u][i];
            }
            mrun = mnew;
        }
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int fi = f0 + lane + 64 * i;
            if (fi < nf) part[wv * nf + fi] = acc[i];
        }
        if (lane == 0 && f0 == 0) {
            wml[2 * wv] = mrun;
            wml[2 * wv + 1] = lrun;
        }
    }

    // Window tokens: exact keys and values, scored here. Wave wv scores the
    // tokens wv, wv + 8, ..., two at a time: lane l holds features 2l and
    // 2l + 1 of the query and reads the same two of each key row (the wave
    // reads a row's 128 features in one coalesced pass), then the wave sums.
    const int64_t q_row = ((int64_t)b * p.n_q + j) * kHeadDim;
    const float q0 = ld<ACT>(p.q, q_row + 2 * lane), q1 = ld<ACT>(p.q, q_row + 2 * lane + 1);
    // Eight tokens per batch: their sixteen loads are issued before any sum,
    // so the batch waits for memory once.
    float mx = -INFINITY;
    constexpr int kWinBatch = 8;
    for (int u0 = wv; u0 < nw; u0 += kWinBatch * kCombWaves) {
        float k0[kWinBatch], k1[kWinBatch];
#pragma unroll
        for (int i = 0; i < kWinBatch; ++i) {
            const int u = u0 + i * kCombWaves;
            const int64_t row = (((int64_t)b * p.win_cap + (u < nw ? u : u0)) * p.n_kv + h) * kHeadDim + 2 * lane;
            k0[i] = ld<ACT>(p.win_k, row);
            k1[i] = ld<ACT>(p.win_k, row + 1);
        }
#pragma unroll
        for (int i = 0; i < kWinBatch; ++i) {
            const int u = u0 + i * kCombWaves;
            const float sc = wave_sum(q0 * k0[i] + q1 * k1[i]) * p.scale;
            if (u < nw) {
                if (lane == 0) sw[u] = sc;
                mx = fmaxf(mx, sc);
            }
        }
    }
    float M = block_reduce(mx, red, true);     // its barriers also publish part, wml and sw
    for (int w8 = 0; w8 < kCombWaves; ++w8) M = fmaxf(M, wml[2 * w8]);

    const int64_t out_row = ((int64_t)b * p.n_q + j) * kHeadDim;
    if (M == -INFINITY) {   // nothing attended for this sequence
        for (int f = tid; f < kHeadDim; f += blockDim.x) st<ACT>(p.out, out_row + f, 0.f);
    } else {
        float scl[kCombWaves], Lt = 0.f;
#pragma unroll
        for (int w8 = 0; w8 < kCombWaves; ++w8) {
            scl[w8] = wml[2 * w8] == -INFINITY ? 0.f : expf(wml[2 * w8] - M);
            Lt += scl[w8] * wml[2 * w8 + 1];
        }
        float lw = 0.f;
        for (int u = tid; u < nw; u += blockDim.x) {
            const float e = expf(sw[u] - M);
            sw[u] = e;
            lw += e;
        }
        const float Lw = block_reduce(lw, red, false);
        for (int f = tid; f < nf; f += blockDim.x) {
            float v = 0.f;
#pragma unroll
            for (int w8 = 0; w8 < kCombWaves; ++w8) v += scl[w8] * part[w8 * nf + f];
            oc[f] = v;
        }
        __syncthreads();
        // out[f] = (sum_i O_G[i] W2[f][i] + O_V[f] + L b2[f] + window) / (L + L_w).
        const float inv = 1.0f / (Lt + Lw);
        const int f = f_out;
        float y = 0.f;
        if (w2_vec) {
            auto piece = [&](int c, const uint4 u) {
                const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int i = i0 + 8 * c + 2 * k;
                    y += oc[i] * __uint_as_float(wd[k] << 16) + oc[i + 1] * __uint_as_float(wd[k] & 0xffff0000u);
                }
            };
#pragma unroll
            for (int c = 0; c < 8; ++c)
                if (c < n_c) piece(c, w2pre[c]);
            for (int c = 8; c < n_c; ++c) piece(c, w2v[c]);
        } else {
            const int i1 = quarter == 3 ? H : i0 + H / 4;
            for (int i = i0; i < i1; ++i) y += oc[i] * ld<ACT>(p.w2, w2row + i);
        }
        // Window values: quarter q takes the tokens u = q (mod 4); each token's
        // row is read by 128 threads, coalesced; eight rows' loads in flight
        // together.
        for (int u0 = quarter; u0 < nw; u0 += 4 * kWinBatch) {
            float vv[kWinBatch];
#pragma unroll
            for (int i = 0; i < kWinBatch; ++i) {
                const int u = u0 + 4 * i;
                vv[i] = u < nw ? ld<ACT>(p.win_v, (((int64_t)b * p.win_cap + u) * p.n_kv + h) * kHeadDim + f) : 0.f;
            }
#pragma unroll
            for (int i = 0; i < kWinBatch; ++i) {
                const int u = u0 + 4 * i;
                if (u < nw) y += sw[u] * vv[i];
            }
        }
        if (quarter == 3) {
            y += oc[H + f];
            if (p.b2) y += Lt * ld<ACT>(p.b2, ((int64_t)b * p.n_kv + h) * kHeadDim + f);
        }
        if (quarter > 0) red[8 + (quarter - 1) * kHeadDim + f] = y;
        __syncthreads();
        if (quarter == 0)
            st<ACT>(p.out, out_row + f, (((y + red[8 + f]) + red[8 + kHeadDim + f]) + red[8 + 2 * kHeadDim + f]) * inv);
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
    return sizeof(float) * ((size_t)p.win_len + (kCombWaves + 1) * ((size_t)p.hidden + kHeadDim) + 4 * kHeadDim + 8 +
                            2 * kCombWaves);
}

hipError_t launch_combine(const DecodeParams& p, int act, hipStream_t s) {
    const size_t smem = combine_smem_bytes(p);
    if (act == DT_F32)
        hipLaunchKernelGGL(combine_kernel<DT_F32>, dim3(p.n_q, p.batch), dim3(kCombThreads), smem, s, p);
    else
        hipLaunchKernelGGL(combine_kernel<DT_BF16>, dim3(p.n_q, p.batch), dim3(kCombThreads), smem, s, p);
    return hipGetLastError();
}

}  // namespace lowram
