// Prefill-side residual ranking: error, exact top-k select, ordered
// compaction with the block CSR, and the residual gather/encode.
// Built with -ffp-contract=off: the error sum must be one binary64 rounding
// per multiply and per add, in index order, to match the float64 definition.
#include <math.h>

#include "kernels.hpp"

#pragma clang fp contract(off)

namespace lowram {

namespace {
constexpr int kRows = 64;            // rows per wave iteration of the error kernel

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };

}  // namespace

// Element k of a staged 16-byte piece as binary64 (exact widening).
template <int DT> __device__ __forceinline__ double piece_elem(const uint4& u, int k);
template <> __device__ __forceinline__ double piece_elem<DT_F32>(const uint4& u, int k) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    return static_cast<double>(__uint_as_float(w[k]));
}
template <> __device__ __forceinline__ double piece_elem<DT_BF16>(const uint4& u, int k) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
    const uint32_t x = w[k >> 1];
    return static_cast<double>(__uint_as_float((k & 1) ? (x & 0xffff0000u) : (x << 16)));
}

// One wave per workgroup. A batch is 64 consecutive rows of V and V_hat;
// lane l sums row l in index order. Rows go through LDS one 128-byte segment
// at a time (64 rows x 128 bytes per tensor, coalesced 16-byte loads), which
// keeps the LDS footprint at 18 KB so two waves share each SIMD and hide the
// latency of the sequential binary64 chain. Two segments are in flight in
// registers (buffer loads: pieces past the last row read as zero) while one
// is summed. Rows are (slice, token, head) in storage order; the error goes to
// err[slice, head, token].
template <int DT>
__global__ __launch_bounds__(64, 2) void rank_error_kernel(RankParams p, int64_t n_rows) {
    constexpr int RB = kHeadDim * Elem<DT>::bytes;   // bytes per row
    constexpr int SEG = 128;                         // bytes per row segment
    constexpr int NSEG = RB / SEG;                   // 2 (bf16) or 4 (f32)
    constexpr int LS = SEG + 16;                     // padded LDS row stride
    constexpr int PIECES = kRows * SEG / (kWave * 16);   // 16-byte pieces per lane per tensor: 8
    constexpr int EPP = 16 / Elem<DT>::bytes;        // elements per piece
    __shared__ __attribute__((aligned(16))) unsigned char sv[kRows * LS];
    __shared__ __attribute__((aligned(16))) unsigned char sh[kRows * LS];
    const int lane = threadIdx.x;
    const int64_t n_batches = (n_rows + kRows - 1) / kRows;
    const int64_t g = gridDim.x;
    const int64_t my_batches = blockIdx.x < n_batches ? (n_batches - 1 - blockIdx.x) / g + 1 : 0;
    const int64_t n_items = my_batches * NSEG;       // (batch, segment) pairs of this wave
    const unsigned char* gv = static_cast<const unsigned char*>(p.v);
    const unsigned char* gh = static_cast<const unsigned char*>(p.v_hat);
    // Piece c of this lane: row (c*64 + lane) / 8, 16-byte column (c*64 + lane) % 8.
    auto load = [&](int64_t it, uint4 (&rv)[PIECES], uint4 (&rh)[PIECES]) {
        const int64_t bt = blockIdx.x + (it / NSEG) * g;
        const int sg = (int)(it % NSEG);
        const int64_t byte0 = bt * kRows * RB;
        const int64_t left = (n_rows - bt * kRows) * RB;
        const uint32_t nbytes = (uint32_t)(left < kRows * RB ? left : kRows * RB);
        const __amdgpu_buffer_rsrc_t bv = buffer_rsrc(gv + byte0, nbytes);
        const __amdgpu_buffer_rsrc_t bh = buffer_rsrc(gh + byte0, nbytes);
#pragma unroll
        for (int c = 0; c < PIECES; ++c) {
            const int q = c * kWave + lane;
            const uint32_t off = (uint32_t)((q >> 3) * RB + sg * SEG + (q & 7) * 16);
            rv[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bv, off, 0, 0));
            rh[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bh, off, 0, 0));
        }
    };
    auto stage = [&](const uint4 (&rv)[PIECES], const uint4 (&rh)[PIECES]) {
#pragma unroll
        for (int c = 0; c < PIECES; ++c) {
            const int q = c * kWave + lane;
            *reinterpret_cast<uint4*>(sv + (q >> 3) * LS + (q & 7) * 16) = rv[c];
            *reinterpret_cast<uint4*>(sh + (q >> 3) * LS + (q & 7) * 16) = rh[c];
        }
    };
    double e = 0.0;
    // Continue row `lane`'s sum over the staged segment; after the last
    // segment of a batch, store it.
    auto consume = [&](int64_t it) {
        const int sg = (int)(it % NSEG);
        if (sg == 0) e = 0.0;
#pragma unroll 2
        for (int c = 0; c < SEG / 16; ++c) {
            const uint4 uv = *reinterpret_cast<const uint4*>(sv + lane * LS + c * 16);
            const uint4 uh = *reinterpret_cast<const uint4*>(sh + lane * LS + c * 16);
            double sq[EPP];
#pragma unroll
            for (int k = 0; k < EPP; ++k) {
                const double dlt = piece_elem<DT>(uv, k) - piece_elem<DT>(uh, k);
                sq[k] = dlt * dlt;
            }
#pragma unroll
            for (int k = 0; k < EPP; ++k) e = e + sq[k];
        }
        if (sg == NSEG - 1) {
            const int64_t row = (blockIdx.x + (it / NSEG) * g) * kRows + lane;
            if (row < n_rows) {
                const int64_t per_slice = (int64_t)p.ctx_len * p.n_kv;
                const int64_t sl = row / per_slice, rem = row % per_slice;
                const int64_t t = rem / p.n_kv, h = rem % p.n_kv;
                p.err[(sl * p.n_kv + h) * p.ctx_len + t] = e;
            }
        }
    };
    uint4 av[PIECES], ah[PIECES], bv[PIECES], bh[PIECES];
    if (n_items > 0) load(0, av, ah);
    if (n_items > 1) load(1, bv, bh);
    for (int64_t it = 0; it < n_items; it += 2) {     // two register sets with fixed roles
        stage(av, ah);
        __syncthreads();
        if (it + 2 < n_items) load(it + 2, av, ah);
        consume(it);
        __syncthreads();
        if (it + 1 >= n_items) break;
        stage(bv, bh);
        __syncthreads();
        if (it + 3 < n_items) load(it + 3, bv, bh);
        consume(it + 1);
        __syncthreads();
    }
}

hipError_t launch_rank_error(const RankParams& p, hipStream_t s) {
    const int64_t n_rows = (int64_t)p.n_slices * p.ctx_len * p.n_kv;
    const int64_t n_batches = (n_rows + kRows - 1) / kRows;
    const int grid = (int)(n_batches < 256 * 8 ? n_batches : 256 * 8);   // one resident wave per slot: 8 per CU
    if (p.in_dtype == DT_F32)
        hipLaunchKernelGGL(rank_error_kernel<DT_F32>, dim3(grid), dim3(64), 0, s, p, n_rows);
    else
        hipLaunchKernelGGL(rank_error_kernel<DT_BF16>, dim3(grid), dim3(64), 0, s, p, n_rows);
    return hipGetLastError();
}

// Exact k-th largest key per (slice, head) by an 8-pass radix select on the
// binary64 bit patterns (non-negative doubles order like their bits). It
// leaves the threshold key and how many tokens equal to it are taken
// (lowest indices first).
__global__ __launch_bounds__(1024) void rank_select_kernel(RankParams p) {
    const int seg = blockIdx.x, tid = threadIdx.x, w = tid >> 6;
    const unsigned long long* keys =
        reinterpret_cast<const unsigned long long*>(p.err) + (int64_t)seg * p.ctx_len;
    __shared__ unsigned int hist[16][256];
    __shared__ unsigned long long s_prefix;
    __shared__ int s_krem;
    if (p.n_res == 0) {
        if (tid == 0) { p.thr[seg] = ~0ull; p.n_eq[seg] = 0; }
        return;
    }
    unsigned long long prefix = 0, mask = 0;
    int krem = p.n_res;
    for (int pass = 0; pass < 8; ++pass) {
        const int shift = 56 - 8 * pass;
        for (int e = tid; e < 16 * 256; e += 1024) (&hist[0][0])[e] = 0;
        __syncthreads();
        for (int t = tid; t < p.ctx_len; t += 1024) {
            const unsigned long long key = keys[t];
            if ((key & mask) == prefix) atomicAdd(&hist[w][(key >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid < 256) {
            unsigned int c = 0;
            for (int i = 0; i < 16; ++i) c += hist[i][tid];
            hist[0][tid] = c;
        }
        __syncthreads();
        if (tid == 0) {
            int cum = 0;
            for (int d = 255; d >= 0; --d) {
                const int c = (int)hist[0][d];
                if (cum + c >= krem) {
                    s_prefix = prefix | ((unsigned long long)d << shift);
                    s_krem = krem - cum;
                    break;
                }
                cum += c;
            }
        }
        __syncthreads();
        prefix = s_prefix;
        krem = s_krem;
        mask |= 0xffull << shift;
        __syncthreads();
    }
    if (tid == 0) { p.thr[seg] = prefix; p.n_eq[seg] = krem; }
}

hipError_t launch_rank_select(const RankParams& p, hipStream_t s) {
    hipLaunchKernelGGL(rank_select_kernel, dim3(p.n_slices * p.n_kv), dim3(1024), 0, s, p);
    return hipGetLastError();
}

// Ordered compaction per (slice, head): token t is taken when its key is above
// the threshold, or equal to it and among the first n_eq such tokens. Slots
// follow ascending t; ptr[i] counts taken tokens below 64*i.
__global__ __launch_bounds__(1024) void rank_compact_kernel(RankParams p) {
    const int seg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const unsigned long long* keys =
        reinterpret_cast<const unsigned long long*>(p.err) + (int64_t)seg * p.ctx_len;
    const unsigned long long thr = p.thr[seg];
    const int neq = p.n_eq[seg];
    __shared__ int wsel[16], weq[16];
    int run_sel = 0, run_eq = 0;
    int32_t* idx = p.res_idx + (int64_t)seg * p.n_res;
    int32_t* ptr = p.res_ptr + (int64_t)seg * (p.n_blocks + 1);
    const unsigned long long lt_mask = (1ull << lane) - 1ull;
    for (int c0 = 0; c0 < p.ctx_len; c0 += 1024) {
        const int t = c0 + tid;
        const bool valid = t < p.ctx_len;
        const unsigned long long key = valid ? keys[t] : 0ull;
        const bool gt = valid && key > thr;
        const bool eq = valid && key == thr && p.n_res > 0;
        const unsigned long long meq = __ballot(eq);
        if (lane == 0) weq[w] = __popcll(meq);
        __syncthreads();
        int off_eq = 0, tot_eq = 0;
        for (int i = 0; i < 16; ++i) { tot_eq += weq[i]; if (i < w) off_eq += weq[i]; }
        const bool take = eq && (run_eq + off_eq + __popcll(meq & lt_mask) < neq);
        const bool sel = gt || take;
        const unsigned long long msel = __ballot(sel);
        if (lane == 0) wsel[w] = __popcll(msel);
        __syncthreads();
        int off_sel = 0, tot_sel = 0;
        for (int i = 0; i < 16; ++i) { tot_sel += wsel[i]; if (i < w) off_sel += wsel[i]; }
        const int before = run_sel + off_sel + __popcll(msel & lt_mask);
        if (sel && before < p.n_res) idx[before] = t;
        if (valid && (t % kBlock) == 0) ptr[t / kBlock] = before;
        run_sel += tot_sel;
        run_eq += tot_eq;
        __syncthreads();
    }
    if (tid == 0) ptr[p.n_blocks] = run_sel < p.n_res ? run_sel : p.n_res;
}

hipError_t launch_rank_compact(const RankParams& p, hipStream_t s) {
    hipLaunchKernelGGL(rank_compact_kernel, dim3(p.n_slices * p.n_kv), dim3(1024), 0, s, p);
    return hipGetLastError();
}

// binary64 -> bfloat16 bits with one round-to-nearest-even step: first to
// float32 with round-to-odd (truncate, then set the last bit if anything was
// dropped), then float32 -> bfloat16 nearest-even. Float32 keeps 16 more
// bits than bfloat16 at every exponent, so the two steps round exactly like
// one.
__device__ __forceinline__ uint16_t f64_to_bf16_bits(double x) {
    float f = static_cast<float>(x);
    const double back = static_cast<double>(f);
    if (back != x && x == x) {
        uint32_t u = __float_as_uint(f);
        if (fabs(back) > fabs(x)) u -= 1u;
        u |= 1u;
        f = __uint_as_float(u);
    }
    return f32_to_bf16_bits(f);
}

// Sixteen lanes per stored residual: lane j of a group owns elements
// 8j .. 8j+7 of the row (16-byte loads of bf16, 32 of f32). R = V - V_hat at
// the chosen token, exact in binary64, then encoded. A wave holds four
// groups and takes two slots per group per iteration (eight rows' loads in
// flight), walking the slots with a grid stride.
template <int IDT>
__device__ __forceinline__ void load_row8(const void* base, int64_t e0, double (&d)[8], const void* base_h) {
    if (IDT == DT_BF16) {
        const uint4 u = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e0);
        const uint4 w = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base_h) + e0);
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = piece_elem<DT_BF16>(u, k) - piece_elem<DT_BF16>(w, k);
    } else {
        const uint4* pv = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + e0);
        const uint4* ph = reinterpret_cast<const uint4*>(static_cast<const float*>(base_h) + e0);
        const uint4 u0 = pv[0], u1 = pv[1], w0 = ph[0], w1 = ph[1];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            d[k] = piece_elem<DT_F32>(u0, k) - piece_elem<DT_F32>(w0, k);
            d[4 + k] = piece_elem<DT_F32>(u1, k) - piece_elem<DT_F32>(w1, k);
        }
    }
}

template <int RDT>
__device__ __forceinline__ void store_res8(const RankParams& p, int64_t gid, int j, const double (&d)[8]) {
    const int64_t o = gid * kHeadDim + 8 * j;
    if (RDT == DT_F32) {
        float4* dst = reinterpret_cast<float4*>(static_cast<float*>(p.res_val) + o);
        dst[0] = make_float4((float)d[0], (float)d[1], (float)d[2], (float)d[3]);
        dst[1] = make_float4((float)d[4], (float)d[5], (float)d[6], (float)d[7]);
    } else if (RDT == DT_BF16) {
        uint32_t w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            w[k] = (uint32_t)f64_to_bf16_bits(d[2 * k]) | ((uint32_t)f64_to_bf16_bits(d[2 * k + 1]) << 16);
        *reinterpret_cast<uint4*>(static_cast<uint16_t*>(p.res_val) + o) = make_uint4(w[0], w[1], w[2], w[3]);
    } else {
        double amax = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmax(amax, fabs(d[k]));
        for (int off = 8; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off, kWave));
        const float s = static_cast<float>(amax / 127.0);
        const double s64 = static_cast<double>(s);
        uint32_t w[2] = {0u, 0u};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            int8_t c = 0;
            if (s64 > 0.0) {
                double q = rint(d[k] / s64);
                q = q > 127.0 ? 127.0 : (q < -127.0 ? -127.0 : q);
                c = static_cast<int8_t>(q);
            }
            w[k >> 2] |= (uint32_t)(uint8_t)c << (8 * (k & 3));
        }
        *reinterpret_cast<uint2*>(static_cast<int8_t*>(p.res_val) + o) = make_uint2(w[0], w[1]);
        if (j == 0) p.res_scale[gid] = s;
    }
}

template <int IDT, int RDT>
__global__ __launch_bounds__(256) void rank_gather_kernel(RankParams p, int64_t n_slots) {
    const int lane = threadIdx.x & 63, grp = lane >> 4, j = lane & 15;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t stride = (int64_t)gridDim.x * 4 * 8;     // slots per grid step
    auto row_of = [&](int64_t gid) {
        const int64_t seg = gid / p.n_res;
        const int64_t sl = seg / p.n_kv, h = seg % p.n_kv;
        int t = p.res_idx[gid];
        t = t < 0 ? 0 : (t >= p.ctx_len ? p.ctx_len - 1 : t);
        return ((sl * p.ctx_len + t) * p.n_kv + h) * kHeadDim + 8 * j;
    };
    for (int64_t base = wave * 8; base < n_slots; base += stride) {
        const int64_t g0 = base + grp, g1 = base + 4 + grp;    // a group's two slots (uniform per group)
        double d0[8], d1[8];
        if (g0 < n_slots) load_row8<IDT>(p.v, row_of(g0), d0, p.v_hat);
        if (g1 < n_slots) load_row8<IDT>(p.v, row_of(g1), d1, p.v_hat);
        if (g0 < n_slots) store_res8<RDT>(p, g0, j, d0);
        if (g1 < n_slots) store_res8<RDT>(p, g1, j, d1);
    }
}

hipError_t launch_rank_gather(const RankParams& p, hipStream_t s) {
    const int64_t n_slots = (int64_t)p.n_slices * p.n_kv * p.n_res;
    if (n_slots == 0) return hipSuccess;
    const int64_t want = (n_slots + 31) / 32;                 // one step per workgroup covers 32 slots
    const dim3 grid((unsigned)(want < 8192 ? want : 8192));
    if (p.in_dtype == DT_F32) {
        if (p.res_dtype == DT_F32) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_F32>), grid, dim3(256), 0, s, p, n_slots);
        else if (p.res_dtype == DT_BF16) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_BF16>), grid, dim3(256), 0, s, p, n_slots);
        else hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_I8>), grid, dim3(256), 0, s, p, n_slots);
    } else {
        if (p.res_dtype == DT_F32) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_F32>), grid, dim3(256), 0, s, p, n_slots);
        else if (p.res_dtype == DT_BF16) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_BF16>), grid, dim3(256), 0, s, p, n_slots);
        else hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_I8>), grid, dim3(256), 0, s, p, n_slots);
    }
    return hipGetLastError();
}

}  // namespace lowram
