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
// Cache policy of the error kernel's loads: V and V_hat are read exactly once,
// so they are marked non-temporal ("nt"); measured on the 32x131072x8x128
// shape, that cuts the whole ranking call by about 7%.
constexpr int kNonTemporal = 2;

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
// registers (non-temporal buffer loads: pieces past the last row read as
// zero) while one is summed. Rows are (slice, token, head) in storage order; the error goes to
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
            rv[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bv, off, 0, kNonTemporal));
            rh[c] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(bh, off, 0, kNonTemporal));
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

// Exact k-th largest key per (slice, head) by radix select on the binary64
// bit patterns (non-negative doubles order like their bits). It leaves the
// threshold key and how many tokens equal to it are taken (lowest indices
// first).
//   1. One pass finds the smallest and largest key; the bits they share are
//      shared by every key, so the digits start below them (errors span a few
//      dozen binades: the top exponent bits carry no information and would
//      pile every key into one bin).
//   2. Passes over 11-bit digits with a private histogram per wave, a block
//      scan from the top bin, and the bin holding the k-th key.
//   3. Once that bin holds at most kCand keys, they are copied to LDS and the
//      remaining digits are resolved there.
namespace {
constexpr int kDigit = 11, kBins = 1 << kDigit, kSelWaves = 16, kCand = 2048;
}

__global__ __launch_bounds__(1024) void rank_select_kernel(RankParams p) {
    const int seg = blockIdx.x, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const unsigned long long* keys =
        reinterpret_cast<const unsigned long long*>(p.err) + (int64_t)seg * p.ctx_len;
    __shared__ unsigned int hist[kSelWaves][kBins];           // 128 KB
    __shared__ unsigned long long cand[kCand];                // 16 KB
    __shared__ unsigned long long red_lo[kSelWaves], red_hi[kSelWaves];
    __shared__ unsigned int wtot[kSelWaves];
    __shared__ unsigned int s_bin, s_above, s_cnt, s_ncand;
    if (p.n_res == 0) {
        if (tid == 0) { p.thr[seg] = ~0ull; p.n_eq[seg] = 0; }
        return;
    }
    // f(key) for every key of src[0, n); eight loads per thread in flight.
    auto for_keys = [&](const unsigned long long* src, int n, auto&& f) {
        for (int t0 = 0; t0 < n; t0 += 8 * 1024) {
            unsigned long long kk[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int t = t0 + j * 1024 + tid;
                kk[j] = t < n ? src[t] : 0ull;
            }
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (t0 + j * 1024 + tid < n) f(kk[j]);
        }
    };
    // 1. common leading bits of all keys
    unsigned long long lo = ~0ull, hi = 0ull;
    for_keys(keys, p.ctx_len, [&](unsigned long long k) {
        lo = k < lo ? k : lo;
        hi = k > hi ? k : hi;
    });
    for (int o = 32; o > 0; o >>= 1) {
        const unsigned long long l2 = __shfl_xor(lo, o, kWave), h2 = __shfl_xor(hi, o, kWave);
        lo = l2 < lo ? l2 : lo;
        hi = h2 > hi ? h2 : hi;
    }
    if (lane == 0) { red_lo[w] = lo; red_hi[w] = hi; }
    __syncthreads();
    lo = red_lo[0]; hi = red_hi[0];
    for (int i = 1; i < kSelWaves; ++i) {
        lo = red_lo[i] < lo ? red_lo[i] : lo;
        hi = red_hi[i] > hi ? red_hi[i] : hi;
    }
    int shift = lo == hi ? 0 : 64 - __clzll(lo ^ hi);        // bits still undecided
    unsigned long long mask = shift == 64 ? 0ull : (~0ull << shift);
    unsigned long long prefix = lo & mask;
    unsigned int krem = (unsigned int)p.n_res;

    // 2./3. digit passes over the global keys, then over the LDS candidates
    const unsigned long long* src = keys;
    int n_src = p.ctx_len;
    while (shift > 0) {
        const int d = shift < kDigit ? shift : kDigit;
        shift -= d;
        for (int e = tid; e < kSelWaves * kBins; e += 1024) (&hist[0][0])[e] = 0u;
        __syncthreads();
        for_keys(src, n_src, [&](unsigned long long k) {
            if ((k & mask) == prefix) atomicAdd(&hist[w][(unsigned)(k >> shift) & (kBins - 1)], 1u);
        });
        __syncthreads();
        // Thread t owns bins 2047-2t and 2046-2t (descending order); sum the
        // wave copies, then an exclusive scan gives the count above each bin.
        const int b0 = kBins - 1 - 2 * tid, b1 = b0 - 1;
        unsigned int c0 = 0, c1 = 0;
        for (int i = 0; i < kSelWaves; ++i) { c0 += hist[i][b0]; c1 += hist[i][b1]; }
        unsigned int incl = c0 + c1;
        for (int o = 1; o < kWave; o <<= 1) {
            const unsigned int v = __shfl_up(incl, o, kWave);
            if (lane >= o) incl += v;
        }
        if (lane == kWave - 1) wtot[w] = incl;
        __syncthreads();
        unsigned int above = incl - (c0 + c1);
        for (int i = 0; i < w; ++i) above += wtot[i];
        if (above < krem && krem <= above + c0) { s_bin = b0; s_above = above; s_cnt = c0; }
        else if (above + c0 < krem && krem <= above + c0 + c1) { s_bin = b1; s_above = above + c0; s_cnt = c1; }
        __syncthreads();
        const unsigned int bin = s_bin, cnt = s_cnt;
        krem -= s_above;
        prefix |= (unsigned long long)bin << shift;
        mask |= (unsigned long long)(kBins - 1 >> (kDigit - d)) << shift;
        if (shift > 0 && src == keys && cnt <= (unsigned)kCand) {
            if (tid == 0) s_ncand = 0;
            __syncthreads();
            for_keys(keys, n_src, [&](unsigned long long k) {
                if ((k & mask) == prefix) cand[atomicAdd(&s_ncand, 1u)] = k;
            });
            __syncthreads();
            src = cand;
            n_src = (int)s_ncand;
        }
        __syncthreads();
    }
    if (tid == 0) { p.thr[seg] = prefix; p.n_eq[seg] = (int)krem; }
}

hipError_t launch_rank_select(const RankParams& p, hipStream_t s) {
    hipLaunchKernelGGL(rank_select_kernel, dim3(p.n_slices * p.n_kv), dim3(1024), 0, s, p);
    return hipGetLastError();
}

// Ordered compaction per (slice, head): token t is taken when its key is above
// the threshold, or equal to it and among the first n_eq such tokens. Slots
// follow ascending t; ptr[i] counts taken tokens below 64*i. Each thread
// takes 8 consecutive tokens per step (8192 per workgroup step); a block
// scan of the per-thread counts orders them.
__device__ __forceinline__ unsigned int block_excl_scan_1024(unsigned int v, unsigned int* wtot, unsigned int& total) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    unsigned int incl = v;
    for (int o = 1; o < kWave; o <<= 1) {
        const unsigned int u = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += u;
    }
    if (lane == kWave - 1) wtot[w] = incl;
    __syncthreads();
    unsigned int before = incl - v;
    total = 0;
    for (int i = 0; i < 16; ++i) {
        if (i < w) before += wtot[i];
        total += wtot[i];
    }
    __syncthreads();
    return before;
}

__global__ __launch_bounds__(1024) void rank_compact_kernel(RankParams p) {
    const int seg = blockIdx.x, tid = threadIdx.x;
    const unsigned long long* keys =
        reinterpret_cast<const unsigned long long*>(p.err) + (int64_t)seg * p.ctx_len;
    const unsigned long long thr = p.thr[seg];
    const unsigned int neq = (unsigned int)p.n_eq[seg];
    __shared__ unsigned int wtot[16];
    unsigned int run_sel = 0, run_eq = 0;
    int32_t* idx = p.res_idx + (int64_t)seg * p.n_res;
    int32_t* ptr = p.res_ptr + (int64_t)seg * (p.n_blocks + 1);
    for (int t0 = 0; t0 < p.ctx_len; t0 += 8 * 1024) {
        const int tb = t0 + 8 * tid;
        unsigned long long kk[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) kk[j] = tb + j < p.ctx_len ? keys[tb + j] : 0ull;
        unsigned int n_gt = 0, n_eq = 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const bool valid = tb + j < p.ctx_len;
            n_gt += valid && kk[j] > thr;
            n_eq += valid && kk[j] == thr && p.n_res > 0;
        }
        unsigned int tot_eq;
        unsigned int eq_before = run_eq + block_excl_scan_1024(n_eq, wtot, tot_eq);
        // taken tokens of this thread: all above, and the equal ones still within n_eq
        unsigned int n_take = n_gt;
        {
            unsigned int e = eq_before;
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (tb + j < p.ctx_len && kk[j] == thr && p.n_res > 0) { n_take += e < neq; ++e; }
        }
        unsigned int tot_sel;
        unsigned int before = run_sel + block_excl_scan_1024(n_take, wtot, tot_sel);
        unsigned int e = eq_before;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const int t = tb + j;
            if (t >= p.ctx_len) break;
            if (t % kBlock == 0) ptr[t / kBlock] = (int32_t)before;
            bool take = kk[j] > thr;
            if (kk[j] == thr && p.n_res > 0) { take = e < neq; ++e; }
            if (take) {
                if (before < (unsigned int)p.n_res) idx[before] = t;
                ++before;
            }
        }
        run_sel += tot_sel;
        run_eq += tot_eq;
    }
    if (tid == 0) ptr[p.n_blocks] = run_sel < (unsigned int)p.n_res ? (int32_t)run_sel : p.n_res;
}

hipError_t launch_rank_compact(const RankParams& p, hipStream_t s) {
    hipLaunchKernelGGL(rank_compact_kernel, dim3(p.n_slices * p.n_kv), dim3(1024), 0, s, p);
    return hipGetLastError();
}


// Sixteen lanes per stored residual: lane j of a group owns elements
// 8j .. 8j+7 of the row (16-byte loads of bf16, 32 of f32). R = V - V_hat at
// the chosen token, exact in binary64, then encoded. A wave holds four
// groups and takes four slots per group per iteration, walking the slots
// with a grid stride: the iteration loads its 16 token indices, then the
// 16 rows of V and of V_hat, then encodes, so it costs two memory round
// trips. Slots past the end read the last slot (nothing is stored for
// them): loads under a slot test made the compiler wait for each slot's
// index and rows in turn.
template <int IDT> struct RowRaw { uint4 v[IDT == DT_F32 ? 2 : 1], h[IDT == DT_F32 ? 2 : 1]; };
template <int IDT>
__device__ __forceinline__ RowRaw<IDT> load_row8_raw(const void* base, int64_t e0, const void* base_h) {
    RowRaw<IDT> r;
    if constexpr (IDT == DT_BF16) {
        r.v[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base) + e0);
        r.h[0] = *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(base_h) + e0);
    } else {
        const uint4* pv = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + e0);
        const uint4* ph = reinterpret_cast<const uint4*>(static_cast<const float*>(base_h) + e0);
        r.v[0] = pv[0]; r.v[1] = pv[1]; r.h[0] = ph[0]; r.h[1] = ph[1];
    }
    return r;
}
template <int IDT>
__device__ __forceinline__ void row8_diff(const RowRaw<IDT>& r, double (&d)[8]) {
    if constexpr (IDT == DT_BF16) {
#pragma unroll
        for (int k = 0; k < 8; ++k) d[k] = piece_elem<DT_BF16>(r.v[0], k) - piece_elem<DT_BF16>(r.h[0], k);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            d[k] = piece_elem<DT_F32>(r.v[0], k) - piece_elem<DT_F32>(r.h[0], k);
            d[4 + k] = piece_elem<DT_F32>(r.v[1], k) - piece_elem<DT_F32>(r.h[1], k);
        }
    }
}

template <int RDT>
__device__ __forceinline__ void store_res8(const RankParams& p, int64_t gid, int j, const double (&d)[8]) {
    const int64_t o = gid * kHeadDim + 8 * j;
    if (RDT == DT_I2) {
        // Symmetric mid-rise 4-level code: s = f32(amax / 1.5),
        // q = clamp(rint(r / s + 1.5), 0, 3) in binary64; a zero row is level 2.
        double amax = 0.0;
#pragma unroll
        for (int k = 0; k < 8; ++k) amax = fmax(amax, fabs(d[k]));
        for (int off = 8; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off, kWave));
        const float s = static_cast<float>(amax / 1.5);
        const double s64 = static_cast<double>(s);
        uint32_t w = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            double q = 2.0;
            if (s64 > 0.0) {
                q = rint(d[k] / s64 + 1.5);
                q = q > 3.0 ? 3.0 : (q < 0.0 ? 0.0 : q);
            }
            w |= (uint32_t)q << (2 * k);
        }
        *reinterpret_cast<uint16_t*>(static_cast<uint8_t*>(p.res_val) + gid * (kHeadDim / 4) + 2 * j) = (uint16_t)w;
        if (j == 0) p.res_scale[gid] = s;
    } else if (RDT == DT_F32) {
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
    constexpr int U = 4;                                        // slots per group per iteration
    const int lane = threadIdx.x & 63, grp = lane >> 4, j = lane & 15;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const int64_t stride = (int64_t)gridDim.x * 4 * 4 * U;     // slots per grid step
    const bool small = n_slots <= 0x7fffffff;                   // 32-bit divisions suffice
    const int64_t tok_stride = (int64_t)p.n_kv * kHeadDim;     // elements between tokens of a slice
    // Element offset of token 0 of slot g's (slice, head), plus this lane's 8 elements.
    auto seg_base = [&](int64_t g) {
        int64_t sl, h;
        if (small) {
            const uint32_t seg = (uint32_t)g / (uint32_t)p.n_res;
            sl = seg / (uint32_t)p.n_kv;
            h = seg % (uint32_t)p.n_kv;
        } else {
            const int64_t seg = g / p.n_res;
            sl = seg / p.n_kv;
            h = seg % p.n_kv;
        }
        return (sl * p.ctx_len * p.n_kv + h) * kHeadDim + 8 * j;
    };
    for (int64_t base = wave * (4 * U); base < n_slots; base += stride) {
        int64_t gid[U], rb[U];
        int tk[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            gid[u] = base + grp + 4 * u;                        // uniform per group
            rb[u] = seg_base(gid[u] < n_slots ? gid[u] : n_slots - 1);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) tk[u] = p.res_idx[gid[u] < n_slots ? gid[u] : n_slots - 1];
        __builtin_amdgcn_sched_barrier(0);
        RowRaw<IDT> raw[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tk[u] < 0 ? 0 : (tk[u] >= p.ctx_len ? p.ctx_len - 1 : tk[u]);
            raw[u] = load_row8_raw<IDT>(p.v, rb[u] + (int64_t)t * tok_stride, p.v_hat);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (gid[u] < n_slots) {
                double d[8];
                row8_diff<IDT>(raw[u], d);
                store_res8<RDT>(p, gid[u], j, d);
            }
        }
    }
}

hipError_t launch_rank_gather(const RankParams& p, hipStream_t s) {
    const int64_t n_slots = (int64_t)p.n_slices * p.n_kv * p.n_res;
    if (n_slots == 0) return hipSuccess;
    const int64_t want = (n_slots + 63) / 64;                 // one step per workgroup covers 64 slots
    const dim3 grid((unsigned)(want < 8192 ? want : 8192));
    if (p.in_dtype == DT_F32) {
        if (p.res_dtype == DT_F32) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_F32>), grid, dim3(256), 0, s, p, n_slots);
        else if (p.res_dtype == DT_BF16) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_BF16>), grid, dim3(256), 0, s, p, n_slots);
        else if (p.res_dtype == DT_I8) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_I8>), grid, dim3(256), 0, s, p, n_slots);
        else hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_I2>), grid, dim3(256), 0, s, p, n_slots);
    } else {
        if (p.res_dtype == DT_F32) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_F32>), grid, dim3(256), 0, s, p, n_slots);
        else if (p.res_dtype == DT_BF16) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_BF16>), grid, dim3(256), 0, s, p, n_slots);
        else if (p.res_dtype == DT_I8) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_I8>), grid, dim3(256), 0, s, p, n_slots);
        else hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_I2>), grid, dim3(256), 0, s, p, n_slots);
    }
    return hipGetLastError();
}

}  // namespace lowram
