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

template <int DT> __device__ __forceinline__ double ld64(const void* base, int64_t i);
template <> __device__ __forceinline__ double ld64<DT_F32>(const void* base, int64_t i) {
    return static_cast<double>(static_cast<const float*>(base)[i]);
}
template <> __device__ __forceinline__ double ld64<DT_BF16>(const void* base, int64_t i) {
    return static_cast<double>(bf16_bits_to_f32(static_cast<const uint16_t*>(base)[i]));
}
}  // namespace

// One wave per workgroup; each iteration stages 64 consecutive rows of V and
// V_hat through LDS with 16-byte coalesced loads, then lane l sums row l in
// index order. Rows are (slice, token, head) in storage order; the error
// goes to err[slice, head, token].
template <int DT>
__global__ __launch_bounds__(64) void rank_error_kernel(RankParams p, int64_t n_rows) {
    constexpr int RB = kHeadDim * Elem<DT>::bytes;   // bytes per row
    constexpr int LS = RB + 16;                      // padded LDS row stride
    constexpr int PER_LANE = RB / 16;                // 16-byte pieces per lane per tensor
    __shared__ __attribute__((aligned(16))) unsigned char sv[kRows * LS];
    __shared__ __attribute__((aligned(16))) unsigned char sh[kRows * LS];
    const int lane = threadIdx.x;
    const int64_t n_batches = (n_rows + kRows - 1) / kRows;
    const unsigned char* gv = static_cast<const unsigned char*>(p.v);
    const unsigned char* gh = static_cast<const unsigned char*>(p.v_hat);
    for (int64_t bt = blockIdx.x; bt < n_batches; bt += gridDim.x) {
        const int64_t row0 = bt * kRows;
        const int64_t byte0 = row0 * RB;
        const int64_t bytes_left = (n_rows - row0) * RB;
        uint4 rv[PER_LANE], rh[PER_LANE];
#pragma unroll
        for (int c = 0; c < PER_LANE; ++c) {
            const int64_t off = (int64_t)(c * kWave + lane) * 16;
            if (off < bytes_left) {
                rv[c] = *reinterpret_cast<const uint4*>(gv + byte0 + off);
                rh[c] = *reinterpret_cast<const uint4*>(gh + byte0 + off);
            } else {
                rv[c] = make_uint4(0, 0, 0, 0);
                rh[c] = make_uint4(0, 0, 0, 0);
            }
        }
#pragma unroll
        for (int c = 0; c < PER_LANE; ++c) {
            const int off = (c * kWave + lane) * 16;
            const int r = off / RB, col = off % RB;
            *reinterpret_cast<uint4*>(sv + r * LS + col) = rv[c];
            *reinterpret_cast<uint4*>(sh + r * LS + col) = rh[c];
        }
        __syncthreads();
        const int64_t row = row0 + lane;
        if (row < n_rows) {
            double e = 0.0;
            const void* pv = sv + lane * LS;
            const void* ph = sh + lane * LS;
#pragma unroll 8
            for (int i = 0; i < kHeadDim; ++i) {
                const double dlt = ld64<DT>(pv, i) - ld64<DT>(ph, i);
                const double sq = dlt * dlt;
                e = e + sq;
            }
            const int64_t per_slice = (int64_t)p.ctx_len * p.n_kv;
            const int64_t sl = row / per_slice, rem = row % per_slice;
            const int64_t t = rem / p.n_kv, h = rem % p.n_kv;
            p.err[(sl * p.n_kv + h) * p.ctx_len + t] = e;
        }
        __syncthreads();
    }
}

hipError_t launch_rank_error(const RankParams& p, hipStream_t s) {
    const int64_t n_rows = (int64_t)p.n_slices * p.ctx_len * p.n_kv;
    const int64_t n_batches = (n_rows + kRows - 1) / kRows;
    const int grid = (int)(n_batches < 256 * 16 ? n_batches : 256 * 16);
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

// One wave per stored residual: R = V - V_hat at the chosen token, exact in
// binary64, then encoded. Lane l owns elements 2l and 2l+1.
template <int IDT, int RDT>
__global__ __launch_bounds__(256) void rank_gather_kernel(RankParams p) {
    const int lane = threadIdx.x & 63;
    const int64_t gid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t n_slots = (int64_t)p.n_slices * p.n_kv * p.n_res;
    if (gid >= n_slots) return;
    const int64_t seg = gid / p.n_res;
    const int64_t sl = seg / p.n_kv, h = seg % p.n_kv;
    int t = p.res_idx[gid];
    t = t < 0 ? 0 : (t >= p.ctx_len ? p.ctx_len - 1 : t);
    const int64_t row = ((sl * p.ctx_len + t) * p.n_kv + h) * kHeadDim;
    const double d0 = ld64<IDT>(p.v, row + 2 * lane) - ld64<IDT>(p.v_hat, row + 2 * lane);
    const double d1 = ld64<IDT>(p.v, row + 2 * lane + 1) - ld64<IDT>(p.v_hat, row + 2 * lane + 1);
    const int64_t o = gid * kHeadDim + 2 * lane;
    if (RDT == DT_F32) {
        static_cast<float*>(p.res_val)[o] = static_cast<float>(d0);
        static_cast<float*>(p.res_val)[o + 1] = static_cast<float>(d1);
    } else if (RDT == DT_BF16) {
        static_cast<uint16_t*>(p.res_val)[o] = f64_to_bf16_bits(d0);
        static_cast<uint16_t*>(p.res_val)[o + 1] = f64_to_bf16_bits(d1);
    } else {
        double amax = fmax(fabs(d0), fabs(d1));
        for (int off = 32; off > 0; off >>= 1) amax = fmax(amax, __shfl_xor(amax, off, kWave));
        const float s = static_cast<float>(amax / 127.0);
        const double s64 = static_cast<double>(s);
        auto code = [&](double dv) -> int8_t {
            if (!(s64 > 0.0)) return 0;
            double q = rint(dv / s64);
            q = q > 127.0 ? 127.0 : (q < -127.0 ? -127.0 : q);
            return static_cast<int8_t>(q);
        };
        static_cast<int8_t*>(p.res_val)[o] = code(d0);
        static_cast<int8_t*>(p.res_val)[o + 1] = code(d1);
        if (lane == 0) p.res_scale[gid] = s;
    }
}

hipError_t launch_rank_gather(const RankParams& p, hipStream_t s) {
    const int64_t n_slots = (int64_t)p.n_slices * p.n_kv * p.n_res;
    if (n_slots == 0) return hipSuccess;
    const dim3 grid((unsigned)((n_slots + 3) / 4));
    if (p.in_dtype == DT_F32) {
        if (p.res_dtype == DT_F32) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_F32>), grid, dim3(256), 0, s, p);
        else if (p.res_dtype == DT_BF16) hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_BF16>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((rank_gather_kernel<DT_F32, DT_I8>), grid, dim3(256), 0, s, p);
    } else {
        if (p.res_dtype == DT_F32) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_F32>), grid, dim3(256), 0, s, p);
        else if (p.res_dtype == DT_BF16) hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_BF16>), grid, dim3(256), 0, s, p);
        else hipLaunchKernelGGL((rank_gather_kernel<DT_BF16, DT_I8>), grid, dim3(256), 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace lowram
