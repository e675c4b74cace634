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

// One workgroup per (query head j, sequence b). A partial record is
// (m, l, O[0:hidden], O[hidden:hidden+d]) where m is the running max of the
// scaled scores, l = sum exp(s - m) over its tokens, O[0:hidden] the
// p-weighted sum of the predictor's hidden activations gelu(k W1 + b1) and
// O[hidden:] the p-weighted sum of k W_lin plus residuals. The output is
//   (O_G W2 + O_V + L b2 + sum_window p v) / (L + L_window)
// after rescaling every record to the common max; W2 and b2 are linear and
// the weights p sum to L, so applying them after the weighted sum gives the
// predictor's value for every token exactly (up to rounding).
//
// The kernel is a short chain of dependent steps, so every load it needs is
// issued at the start, in one round trip: the records of its wave's first
// batch, the window rows of its first window batch, then this thread's W2
// pieces (needed last, so the records merge while they land). Each wave folds
// its records and its window tokens into running (max, weight sum, sums)
// pairs, the window tokens as one more record whose hidden part is zero (their
// values are exact), and two barriers merge the eight waves.
constexpr int kCombWaves = 8;
constexpr int kCombThreads = kCombWaves * 64;
constexpr int kCombWin = 16;          // window tokens per wave per batch

// Features 2 lane and 2 lane + 1 of a row, as stored (bf16 pair in .x, or two floats).
template <int ACT> __device__ __forceinline__ uint2 ld_pair_raw(const void* base, int64_t elem) {
    if constexpr (ACT == DT_F32) return *reinterpret_cast<const uint2*>(static_cast<const float*>(base) + elem);
    else return make_uint2(*reinterpret_cast<const uint32_t*>(static_cast<const uint16_t*>(base) + elem), 0u);
}
template <int ACT> __device__ __forceinline__ float2 pair_f(uint2 r) {
    if constexpr (ACT == DT_F32) return make_float2(__uint_as_float(r.x), __uint_as_float(r.y));
    else return make_float2(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u));
}
// Values of lane ^ 1 and lane ^ 2 (DPP quad permutations, no LDS traffic).
__device__ __forceinline__ float quad_xor1(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
// One step of a transposing butterfly: a lane carries 2n partial sums and
// keeps the half that bit `o` of its lane index selects, adding the partner's
// (lane ^ o) partial of the same values; the partner keeps the other half.
template <int N>
__device__ __forceinline__ void fold_half(const float (&in)[2 * N], float (&out)[N], int lane, int o) {
    const bool hi = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < N; ++i) {
        const float keep = hi ? in[N + i] : in[i], send = hi ? in[i] : in[N + i];
        out[i] = keep + __shfl_xor(send, o, kWave);
    }
}

// sum_e oc[e] w[e] over the elements of one 16-byte W2 piece.
template <int ACT> __device__ __forceinline__ float dot_piece(const uint4 u, const float* oc) {
    const uint32_t wd[4] = {u.x, u.y, u.z, u.w};
    float y = 0.f;
    if constexpr (ACT == DT_F32) {
#pragma unroll
        for (int k = 0; k < 4; ++k) y += oc[k] * __uint_as_float(wd[k]);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            y += oc[2 * k] * __uint_as_float(wd[k] << 16) + oc[2 * k + 1] * __uint_as_float(wd[k] & 0xffff0000u);
    }
    return y;
}

template <int ACT>
__global__ __launch_bounds__(kCombThreads) void combine_kernel(DecodeParams p) {
    const int j = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wv = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int h = j / p.group, H = p.hidden, S = p.part_stride, nf = H + kHeadDim;
    const int nsplit = min(p.n_split, (attended_count(p, b) + p.blocks_per_split - 1) / p.blocks_per_split);
    const int nw = window_len(p);
    const float* P = p.partials + ((int64_t)b * p.n_q + j) * p.n_split * (int64_t)S;
    extern __shared__ float sm[];
    float* part = sm;                              // [8][nf]: the waves' record sums
    float* wpart = part + kCombWaves * nf;         // [8][d]: the waves' window value sums
    float* oc = wpart + kCombWaves * kHeadDim;     // [nf]: the merged sums
    float* wml = oc + nf;                          // [8][4]: record max and weight sum, window max and weight sum

    // Issue order: the first record batch, the first window batch, then the
    // W2 pieces, b2 and the query. Loads complete in issue order, so the
    // records merge while the W2 rows (cold in every cache) are still in
    // flight; W2 is first needed after both barriers.
    //
    // Records: wave wv merges the splits wv, wv+8, ... eight at a time, with
    // a running max (every sum is rescaled to it as it grows), so the loads of
    // a batch's maxima, weight sums and O rows are in flight together. Lane
    // takes the features f0 + lane + 64 i, six at a time: each load of the
    // wave reads 256 consecutive bytes of one record.
    // rec_load issues plain loads only: a split past the last reads split 0
    // (written by this call whenever nsplit >= 1) and a feature past the
    // record reads its last one, and rec_use gives those entries weight
    // zero. Loads feeding a select under the split test made the compiler
    // wait for each record before issuing the next one's.
    auto rec_load = [&](int f0, int s0, float2 (&ml)[8], float (&v)[8][6]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int sp = s0 + kCombWaves * u;
            const float* rec = P + (int64_t)(sp < nsplit ? sp : 0) * S;
            ml[u] = *reinterpret_cast<const float2*>(rec);
#pragma unroll
            for (int i = 0; i < 6; ++i) v[u][i] = rec[2 + min(f0 + lane + 64 * i, nf - 1)];
        }
    };
    auto rec_use = [&](int s0, const float2 (&ml)[8], const float (&v)[8][6], float& mrun, float& lrun, float (&acc)[6]) {
        float mb[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) mb[u] = s0 + kCombWaves * u < nsplit ? ml[u].x : -INFINITY;
        float mnew = mrun;
#pragma unroll
        for (int u = 0; u < 8; ++u) mnew = fmaxf(mnew, mb[u]);
        const float r = mrun == -INFINITY ? 0.f : __expf(mrun - mnew);
        lrun *= r;
#pragma unroll
        for (int i = 0; i < 6; ++i) acc[i] *= r;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const float e = mb[u] == -INFINITY ? 0.f : __expf(mb[u] - mnew);
            lrun += e * ml[u].y;
#pragma unroll
            for (int i = 0; i < 6; ++i) acc[i] += e * v[u][i];
        }
        mrun = mnew;
    };
    auto rec_store = [&](int f0, const float (&acc)[6], float mrun, float lrun) {
#pragma unroll
        for (int i = 0; i < 6; ++i) {
            const int fi = f0 + lane + 64 * i;
            if (fi < nf) part[wv * nf + fi] = acc[i];
        }
        if (lane == 0 && f0 == 0) {
            wml[4 * wv] = mrun;
            wml[4 * wv + 1] = lrun;
        }
    };
    float2 ml0[8];
    float v0[8][6];
    if (nsplit > 0) rec_load(0, wv, ml0, v0);     // none: split 0 may hold stale data
    __builtin_amdgcn_sched_barrier(0);

    // Window tokens: batch u0 gives wave wv the tokens u0 + 16 wv + i; lane
    // holds features 2 lane and 2 lane + 1 of the query and of each row.
    // A wave with no token in the batch loads nothing (the buffers may be
    // absent when the window is empty); otherwise every row load is
    // unconditional, tokens past the window reading the last one (win_use
    // ignores them).
    auto win_load = [&](int u0, uint2 (&kr)[kCombWin], uint2 (&vr)[kCombWin]) {
        if (u0 + kCombWin * wv >= nw) return;
#pragma unroll
        for (int i = 0; i < kCombWin; ++i) {
            const int u = min(u0 + kCombWin * wv + i, nw - 1);
            const int64_t row = (((int64_t)b * p.win_cap + u) * p.n_kv + h) * kHeadDim + 2 * lane;
            kr[i] = ld_pair_raw<ACT>(p.win_k, row);
            vr[i] = ld_pair_raw<ACT>(p.win_v, row);
        }
    };
    uint2 kr[kCombWin], vr[kCombWin];
    win_load(0, kr, vr);

    // W2 rows: out[f] takes the 32 lanes of one half-wave, so every load reads
    // whole rows (coalesced). Pass k covers the rows f = 16 k + tid / 32; lane
    // l32 of the half takes the 16-byte pieces l32 + 32 m of its row; the
    // pieces of m = 0 are loaded here.
    constexpr int kEpp = ACT == DT_F32 ? 4 : 8;    // W2 elements per 16-byte piece
    const int n_pc = H / kEpp;                     // pieces per row (H is a multiple of 16)
    const int l32 = tid & 31, g16 = tid >> 5;
    const int64_t head = (int64_t)b * p.n_kv + h;
    const uint4* w2g = reinterpret_cast<const uint4*>(static_cast<const char*>(p.w2) +
                                                      head * kHeadDim * H * (int64_t)(ACT == DT_F32 ? 4 : 2));
    uint4 w2pre[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const int f = 16 * k + g16;
        w2pre[k] = w2g[(int64_t)f * n_pc + min(l32, n_pc - 1)];   // lanes past the row: unused duplicate
    }
    // The row sums end in lane group k_own of the half (see below); b2 of that
    // row, kept as stored and converted where it is used.
    const int k_own = 4 * ((lane >> 4) & 1) + 2 * ((lane >> 3) & 1) + ((lane >> 2) & 1);
    const int f_own = 16 * k_own + g16;
    // Without b2 the load reads the query instead (no branch, whose join
    // would make the compiler wait for every load issued so far) and the
    // value is dropped where it is used.
    const bool has_b2 = p.b2 != nullptr;
    const void* const b2src = has_b2 ? p.b2 : p.q;
    const int64_t b2i = has_b2 ? head * kHeadDim + f_own : 0;
    uint32_t b2_raw;
    if constexpr (ACT == DT_F32) b2_raw = static_cast<const uint32_t*>(b2src)[b2i];
    else b2_raw = static_cast<const uint16_t*>(b2src)[b2i];
    const int64_t q_row = ((int64_t)b * p.n_q + j) * kHeadDim;
    const float2 qq = pair_f<ACT>(ld_pair_raw<ACT>(p.q, q_row + 2 * lane));
    __builtin_amdgcn_sched_barrier(0);

    float wm = -INFINITY, wl = 0.f, wa0 = 0.f, wa1 = 0.f;   // this wave's window max, weight sum, value sums
    auto win_use = [&](int u0, const uint2 (&kr)[kCombWin], const uint2 (&vr)[kCombWin]) {
        if (u0 + kCombWin * wv >= nw) return;       // no token of this batch is the wave's
        // q . k of the wave's 16 tokens: the lanes' products, then a
        // transposing butterfly (17 shuffles in place of 16 wave sums); lane
        // ends with the sum of token 8 b5 + 4 b4 + 2 b3 + b2 (bits of its
        // index), which lane 32 b5 + 16 b4 + 8 b3 + 4 b2 then hands out.
        float v16[16], v8[8], v4[4], v2[2], v1[1];
#pragma unroll
        for (int i = 0; i < kCombWin; ++i) {
            const float2 kk = pair_f<ACT>(kr[i]);
            v16[i] = qq.x * kk.x + qq.y * kk.y;
        }
        fold_half<8>(v16, v8, lane, 32);
        fold_half<4>(v8, v4, lane, 16);
        fold_half<2>(v4, v2, lane, 8);
        fold_half<1>(v2, v1, lane, 4);
        float tsum = v1[0] + quad_xor2(v1[0]);
        tsum += quad_xor1(tsum);
        float sc[kCombWin];
        float mnew = wm;
#pragma unroll
        for (int i = 0; i < kCombWin; ++i) {
            const int src = 32 * ((i >> 3) & 1) + 16 * ((i >> 2) & 1) + 8 * ((i >> 1) & 1) + 4 * (i & 1);
            sc[i] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(tsum), src)) * p.scale;
            if (u0 + kCombWin * wv + i < nw) mnew = fmaxf(mnew, sc[i]);
        }
        if (mnew == -INFINITY) return;             // no token of this batch is the wave's
        const float r = wm == -INFINITY ? 0.f : __expf(wm - mnew);
        wl *= r;
        wa0 *= r;
        wa1 *= r;
#pragma unroll
        for (int i = 0; i < kCombWin; ++i) {
            if (u0 + kCombWin * wv + i < nw) {
                const float e = __expf(sc[i] - mnew);
                const float2 vv = pair_f<ACT>(vr[i]);
                wl += e;
                wa0 += e * vv.x;
                wa1 += e * vv.y;
            }
        }
        wm = mnew;
    };

    // Features 0 .. 383 with the first batch already loaded (straight-line,
    // so its wait covers only the loads issued before the window and W2),
    // then any further feature slices.
    {
        float mrun = -INFINITY, lrun = 0.f;
        float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        if (nsplit > 0) rec_use(wv, ml0, v0, mrun, lrun, acc);
        for (int s0 = wv + kCombWaves * 8; s0 < nsplit; s0 += kCombWaves * 8) {
            rec_load(0, s0, ml0, v0);
            rec_use(s0, ml0, v0, mrun, lrun, acc);
        }
        rec_store(0, acc, mrun, lrun);
    }
    for (int f0 = 64 * 6; f0 < nf; f0 += 64 * 6) {
        float mrun = -INFINITY, lrun = 0.f;
        float acc[6] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int s0 = wv; s0 < nsplit; s0 += kCombWaves * 8) {
            rec_load(f0, s0, ml0, v0);
            rec_use(s0, ml0, v0, mrun, lrun, acc);
        }
        rec_store(f0, acc, mrun, lrun);
    }

    // The window batches: the first was loaded with the records; the others
    // (windows above 128 tokens) load and fold one at a time.
    win_use(0, kr, vr);
    for (int u0 = kCombWin * kCombWaves; u0 < nw; u0 += kCombWin * kCombWaves) {
        win_load(u0, kr, vr);
        win_use(u0, kr, vr);
    }
    wpart[wv * kHeadDim + 2 * lane] = wa0;
    wpart[wv * kHeadDim + 2 * lane + 1] = wa1;
    if (lane == 0) {
        wml[4 * wv + 2] = wm;
        wml[4 * wv + 3] = wl;
    }
    __syncthreads();

    // Merge the waves at the common max: oc = the rescaled record sums, and
    // on the value part the rescaled window sums.
    float M = -INFINITY;
#pragma unroll
    for (int w8 = 0; w8 < kCombWaves; ++w8) M = fmaxf(M, fmaxf(wml[4 * w8], wml[4 * w8 + 2]));
    const int64_t out_row = ((int64_t)b * p.n_q + j) * kHeadDim;
    if (M == -INFINITY) {   // nothing attended for this sequence (uniform branch)
        for (int f = tid; f < kHeadDim; f += blockDim.x) st<ACT>(p.out, out_row + f, 0.f);
    } else {
        float sr[kCombWaves], sw[kCombWaves], Lt = 0.f, Lw = 0.f;
#pragma unroll
        for (int w8 = 0; w8 < kCombWaves; ++w8) {
            sr[w8] = wml[4 * w8] == -INFINITY ? 0.f : __expf(wml[4 * w8] - M);
            sw[w8] = wml[4 * w8 + 2] == -INFINITY ? 0.f : __expf(wml[4 * w8 + 2] - M);
            Lt += sr[w8] * wml[4 * w8 + 1];
            Lw += sw[w8] * wml[4 * w8 + 3];
        }
        for (int f = tid; f < nf; f += blockDim.x) {
            float v = 0.f;
#pragma unroll
            for (int w8 = 0; w8 < kCombWaves; ++w8) v += sr[w8] * part[w8 * nf + f];
            if (f >= H) {
#pragma unroll
                for (int w8 = 0; w8 < kCombWaves; ++w8) v += sw[w8] * wpart[w8 * kHeadDim + (f - H)];
            }
            oc[f] = v;
        }
        __syncthreads();
        // out[f] = (sum_i O_G[i] W2[f][i] + O_V[f] + window + L b2[f]) / (L + L_w)
        const float inv = 1.0f / (Lt + Lw);
        float y8[8], y4[4], y2[2], y1[1];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int f = 16 * k + g16;
            float y = l32 < n_pc ? dot_piece<ACT>(w2pre[k], oc + l32 * kEpp) : 0.f;
            for (int pc = l32 + 32; pc < n_pc; pc += 32) y += dot_piece<ACT>(w2g[(int64_t)f * n_pc + pc], oc + pc * kEpp);
            y8[k] = y;
        }
        // Row sums over the 32 lanes of the half, transposed as they fold:
        // lane group (b4, b3, b2) ends with pass k_own's full sum.
        fold_half<4>(y8, y4, lane, 16);
        fold_half<2>(y4, y2, lane, 8);
        fold_half<1>(y2, y1, lane, 4);
        float y = y1[0] + quad_xor2(y1[0]);
        y += quad_xor1(y);
        const float b2_own = has_b2 ? __uint_as_float(ACT == DT_F32 ? b2_raw : b2_raw << 16) : 0.f;
        if ((lane & 3) == 0) st<ACT>(p.out, out_row + f_own, (y + oc[H + f_own] + Lt * b2_own) * inv);
    }
    // Exact stats: the first wave sums the per-split counts, a split per lane
    // (every load in flight at once; integer sums, so the order is free).
    if (p.stats != nullptr && j % p.group == 0 && wv == 0) {
        int tok = 0, res = 0;
        const int32_t* c = p.counts + ((int64_t)b * p.n_kv + h) * p.n_split * 2;
        for (int s = lane; s < nsplit; s += kWave) {
            tok += c[2 * s];
            res += c[2 * s + 1];
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            tok += __shfl_xor(tok, o, kWave);
            res += __shfl_xor(res, o, kWave);
        }
        if (lane == 0) {
            p.stats[((int64_t)b * p.n_kv + h) * 2 + 0] = tok + nw;
            p.stats[((int64_t)b * p.n_kv + h) * 2 + 1] = res;
        }
    }
}

size_t combine_smem_bytes(const DecodeParams& p) {
    const size_t nf = (size_t)p.hidden + kHeadDim;
    return sizeof(float) * ((kCombWaves + 1) * nf + (size_t)kCombWaves * kHeadDim + 4 * kCombWaves);
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
