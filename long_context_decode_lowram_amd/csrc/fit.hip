// Test-time fit of the per-head value predictor's nonlinear branch.
//
// explainer, Slim Attention paragraph: the predictor starts from the linear
// pseudoinverse map and a small nonlinear branch learns the rest from the
// current context; explainer, cost paragraph: the fit takes gradient steps
// per context at prefill. Loss L = (1 / T) sum_t ||v_hat_t - v_t||^2, plain
// gradient descent on W1, b1, W2, b2 (W_lin fixed). Per step and problem
// (layer, KV head), with weights stored output-major:
//   H = gelu(K W1^T + b1)                              fit_nt_kernel<kEpiZ>
//   G = (2 / T)(K W_lin^T + H W2^T + b2 - V)           fit_nt_kernel<kEpiG>   (+ loss, sum_t G)
//   dZ = (G W2) * gelu'(K W1^T + b1)                   fit_nt_kernel<kEpiDz>  (+ sum_t dZ; the
//                                                      pre-activations are recomputed, not stored)
//   dW2 = G^T H, dW1 = dZ^T K                          fit_tn_kernel (token chunks)
//   theta -= lr dL/dtheta                              fit_update_kernel
// Products on bf16 MFMA with fp32 sums; the parameters are fp32 masters with
// bf16 copies for the products.
#include <hip/hip_runtime.h>
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace lowram {

constexpr int kFM = 128;                 // tokens per tile (MFMA B operand rows)
constexpr int kFN = 128;                 // outputs per tile (MFMA A operand rows)
constexpr int kFK = 64;                  // contraction step
constexpr int kFRowB = kFK * 2;          // 128-byte LDS rows
constexpr int kFOp0 = kFN * kFRowB;      // 16 KB
constexpr int kFStage = (kFN + kFM) * kFRowB;   // 32 KB
constexpr int kFThreads = 512;
enum : int { kEpiZ = 0, kEpiG = 1, kEpiDz = 2 };

__device__ __forceinline__ uint32_t fslot(int row, int piece) {
    return (uint32_t)(row * kFRowB + ((piece ^ (row & 7)) << 4));
}

// GELU and its derivative from the normal tail fit (normal_tail): with
// a = |z|, gelu(z) = max(z, 0) - a Q(a) and gelu'(z) = Phi(z) + z phi(z),
// Phi(z) = 1 - Q(a) for z >= 0, Q(a) below; phi(z) = 2^(-z^2 / (2 ln 2)) / sqrt(2 pi).
__device__ __forceinline__ float gelu_f(float z) {
    const float a = fabsf(z);
    return fmaxf(z, 0.0f) - a * normal_tail(a);
}
__device__ __forceinline__ float gelu_grad_f(float z) {
    const float q = normal_tail(fabsf(z));
    const float phi = __builtin_amdgcn_exp2f(-0.72134752044448170f * z * z) * 0.39894228040143268f;
    return (z >= 0.0f ? 1.0f - q : q) + z * phi;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f32_to_bf16_bits(a) | ((uint32_t)f32_to_bf16_bits(b) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// One segment of a contraction: op1 rows are tokens of `a` (row stride lda
// elements), op0 rows are outputs of `b` (row stride ldb), kdim contiguous.
struct NtSeg {
    const __bf16* a; int lda;
    const __bf16* b; int ldb;
    int kdim;
};

// NT product over up to two segments for a 128-token x 128-output tile of
// problem blockIdx.y, then the fused epilogue. Grid (m_tiles * n_tiles, P);
// 64 KB of LDS (two workgroups per CU), 32 KB for EPI_Z (three). Eight
// waves: wave w covers
// outputs 64 (w & 1) .. and tokens 32 (w >> 1) ..; lane (l16, g4) ends with
// outputs n .. n + 3 (n = 4 g4 + 16 nt) of token l16 + 16 tt of its block.
template <int EPI>
__global__ __launch_bounds__(kFThreads, 2) void fit_nt_kernel(FitParams p) {
    // EPI_Z (two contraction steps) keeps one stage buffer: 32 KB of LDS, so
    // three workgroups share a CU (its 65 registers allow three as well) and
    // hide each other's load latency, which pays more than overlapping its
    // second copy with its first step (measured: the fit call 118.6 -> 113.5
    // ms). The others double-buffer.
    constexpr int kNst = EPI == kEpiZ ? 1 : 2;
    __shared__ __attribute__((aligned(16))) unsigned char stg[kNst * kFStage];
    unsigned char* const st0 = stg;
    unsigned char* const st1 = stg + (kNst - 1) * kFStage;
    __shared__ float red_cs[4][256];
    __shared__ float red_loss[8];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = blockIdx.y;
    const int l = q / p.n_kv, h = q - l * p.n_kv;
    const int d = kHeadDim, H = p.hidden, T = p.ctx_len;
    const int N = EPI == kEpiG ? d : H;
    const int n_tiles = N / kFN;
    // The output tiles of one token tile sit 8 blocks apart, so that they run
    // on the same XCD (blocks go round-robin over the 8) and share its L2
    // copy of the token rows. Blocks past the last token tile exit.
    const int grp = blockIdx.x / (8 * n_tiles), rem = blockIdx.x - grp * 8 * n_tiles;
    const int ntile = rem >> 3, mt = grp * 8 + (rem & 7);
    if (mt >= p.m_tiles) return;
    const int t0 = mt * kFM, n0 = ntile * kFN;
    const int ldkv = p.n_kv * d;
    const __bf16* kq = p.keys + (int64_t)l * T * ldkv + h * d;
    const int64_t th = (int64_t)q * T * H, td = (int64_t)q * T * d;

    // Segments of the contraction; EPI_G sums two into one accumulator,
    // EPI_DZ runs two separate products (pre-activations, then G W2).
    NtSeg seg[2];
    int n_seg = 1;
    const NtSeg zseg = NtSeg{kq, ldkv, p.w1b + (int64_t)q * H * d, d, d};
    if (EPI == kEpiZ) {
        seg[0] = zseg;
    } else if (EPI == kEpiG) {
        seg[0] = NtSeg{kq, ldkv, p.w_lin + (int64_t)q * d * d, d, d};
        seg[1] = NtSeg{p.hb + th, H, p.w2b + (int64_t)q * d * H, H, H};
        n_seg = 2;
    } else {
        seg[0] = NtSeg{p.gb + td, d, p.w2tb + (int64_t)q * H * d, d, d};
    }

    // Direct copies: op0 (128 output rows) and op1 (128 token rows, zeros
    // past T) by 2 copies per wave each; lane i lands in row 8 c + i / 8,
    // slot i % 8, and fetches piece (i % 8) ^ (row % 8).
    const int dma_row = lane >> 3;
    const uint32_t dma_piece = (uint32_t)(((lane & 7) ^ dma_row) * 16);
    auto dma = [&](const NtSeg* sgs, int steps0, int s, unsigned char* stage) {
        const int sg = s < steps0 ? 0 : 1;
        const int k0 = (s - (sg ? steps0 : 0)) * kFK;
        const NtSeg& g = sgs[sg];
        const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(g.b + (int64_t)n0 * g.ldb, (uint32_t)(kFN * g.ldb * 2));
        const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(g.a + (int64_t)t0 * g.lda,
                                                      (uint32_t)((int64_t)max(0, T - t0) * g.lda * 2));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r0 = (w * 2 + c) * 8;
            dma16(rb, stage + r0 * kFRowB, (uint32_t)(((r0 + dma_row) * g.ldb + k0) * 2) + dma_piece, 0u);
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r0 = (w * 2 + c) * 8;
            dma16(ra, stage + kFOp0 + r0 * kFRowB, (uint32_t)(((r0 + dma_row) * g.lda + k0) * 2) + dma_piece, 0u);
        }
    };

    const int l16 = lane & 15, g4 = lane >> 4;
    const int wn = (w & 1) * 64, wt = (w >> 1) * 32;
    auto mma = [&](const unsigned char* stage, f32x4 (&acc)[4][2]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[4], bf[2];
#pragma unroll
            for (int a = 0; a < 4; ++a) af[a] = lds16(stage, fslot(wn + a * 16 + l16, ks * 4 + g4));
#pragma unroll
            for (int b = 0; b < 2; ++b) bf[b] = lds16(stage + kFOp0, fslot(wt + b * 16 + l16, ks * 4 + g4));
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b) acc[a][b] = mfma(af[a], bf[b], acc[a][b]);
        }
    };
    // acc = sum over the segments' contraction, copies one 64-wide step ahead
    // into two static stage buffers.
    auto contract = [&](const NtSeg* sgs, int ns, f32x4 (&acc)[4][2]) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int steps0 = sgs[0].kdim / kFK;
        const int n_steps = steps0 + (ns == 2 ? sgs[1].kdim / kFK : 0);
        dma(sgs, steps0, 0, st0);
        if constexpr (kNst == 1) {
            for (int s = 0; s < n_steps; ++s) {
                wait_vmcnt<0>();
                barrier_lds();
                mma(st0, acc);
                if (s + 1 < n_steps) {
                    barrier_lds();       // every wave is done reading the buffer
                    dma(sgs, steps0, s + 1, st0);
                }
            }
        } else {
            auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
                wait_vmcnt<0>();
                barrier_lds();
                if (s + 1 < n_steps) dma(sgs, steps0, s + 1, nxt);
                mma(cur, acc);
            };
            for (int s = 0; s < n_steps; s += 2) {
                step(s, st0, st1);
                if (s + 1 < n_steps) step(s + 1, st1, st0);
            }
        }
        wait_vmcnt<0>();
    };
    f32x4 acc[4][2], accz[4][2];
    if (EPI == kEpiDz) {
        contract(&zseg, 1, accz);
        barrier_lds();       // every wave is done with the stage buffers
    }
    contract(seg, n_seg, acc);

    // Epilogue.
    float cs[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) cs[a][v] = 0.f;
    float loss = 0.f;
    const float gscale = 2.0f / (float)T;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int t = t0 + wt + b * 16 + l16;
        if (t >= T) continue;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int n = n0 + wn + a * 16 + g4 * 4;
            const f32x4 x = acc[a][b];
            if (EPI == kEpiZ) {
                const float* bb = p.b1 + (int64_t)q * H + n;
                float hv[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) hv[v] = gelu_f(x[v] + bb[v]);
                *reinterpret_cast<u32x2*>(p.hb + th + (int64_t)t * H + n) =
                    u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            } else if (EPI == kEpiG) {
                const float* bb = p.b2 + (int64_t)q * d + n;
                const u32x2 vv = *reinterpret_cast<const u32x2*>(p.v + ((int64_t)l * T + t) * ldkv + h * d + n);
                const float vt[4] = {bf16_lo(vv[0]), bf16_hi(vv[0]), bf16_lo(vv[1]), bf16_hi(vv[1])};
                float g[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float e = x[v] + bb[v] - vt[v];
                    loss = fmaf(e, e, loss);
                    g[v] = gscale * e;
                    cs[a][v] += g[v];
                }
                *reinterpret_cast<u32x2*>(p.gb + td + (int64_t)t * d + n) = u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
            } else {
                const float* bb = p.b1 + (int64_t)q * H + n;
                const f32x4 zx = accz[a][b];
                float dz[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    dz[v] = x[v] * gelu_grad_f(zx[v] + bb[v]);
                    cs[a][v] += dz[v];
                }
                *reinterpret_cast<u32x2*>(p.dzb + th + (int64_t)t * H + n) = u32x2{pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3])};
            }
        }
    }
    if (EPI == kEpiZ) return;
    // Column sums over this tile's tokens: lanes l16 = 0..15 share outputs;
    // the 4 token waves of an output half meet in LDS in a fixed order.
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            float x = cs[a][v];
            for (int off = 1; off < 16; off <<= 1) x += __shfl_xor(x, off, kWave);
            cs[a][v] = x;
        }
    if (l16 == 0) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int v = 0; v < 4; ++v) red_cs[w >> 1][wn + a * 16 + g4 * 4 + v] = cs[a][v];
    }
    if (EPI == kEpiG) {
        for (int off = 32; off > 0; off >>= 1) loss += __shfl_xor(loss, off, kWave);
        if (lane == 0) red_loss[w] = loss;
    }
    __syncthreads();
    if (tid < kFN) {
        const float c = ((red_cs[0][tid] + red_cs[1][tid]) + red_cs[2][tid]) + red_cs[3][tid];
        if (EPI == kEpiG) p.cs_g[((int64_t)q * p.m_tiles + mt) * d + n0 + tid] = c;
        else p.cs_dz[((int64_t)q * p.m_tiles + mt) * H + n0 + tid] = c;
    }
    if (EPI == kEpiG && tid == 0) {
        float sum = 0.f;
        for (int i = 0; i < 8; ++i) sum += red_loss[i];
        p.loss_p[(int64_t)q * p.m_tiles + mt] = sum;
    }
}

// ------------------------------------------------------------------- TN
// C[m][n] = sum over this chunk's tokens of A[t][m] B[t][n], a 128 x 128
// tile, stored transposed: out[n][m]. Both operands are token-major, copied
// untransposed into a 4-stage ring of 32-token steps (256-byte rows, piece p
// of row t in slot p ^ tsw(t)) three steps ahead and read with the
// transposing LDS read (lanes 4r .. 4r+3 of a 16-lane group name row r's 16
// columns, lane j gets column j of the 4 rows). Four waves of 64 x 64.
// role 0: dW2 = G^T H (A = G [T][d], B = H [T][h]); role 1: dW1 = dZ^T K.
constexpr int kTK = 32;
constexpr int kTRowB = 256;
constexpr int kTOp = kTK * kTRowB;       // 8 KB
constexpr int kTStage = 2 * kTOp;

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

__device__ __forceinline__ int tsw(int t) { return 2 * ((t & 3) | (((t >> 3) & 1) << 2)); }

__device__ __forceinline__ bf16x8 tn_frag(const unsigned char* op, uint32_t off) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(op + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(op + off + 4 * kTRowB));
    u32x4 v;
    v[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    v[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    v[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    v[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return as_bf16x8(v);
}

template <int ROLE>
__global__ __launch_bounds__(256, 1) void fit_tn_kernel(FitParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char s0[kTStage];
    __shared__ __attribute__((aligned(16))) unsigned char s1[kTStage];
    __shared__ __attribute__((aligned(16))) unsigned char s2[kTStage];
    __shared__ __attribute__((aligned(16))) unsigned char s3[kTStage];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int q = blockIdx.y;
    const int l = q / p.n_kv, h = q - l * p.n_kv;
    const int d = kHeadDim, H = p.hidden, T = p.ctx_len;
    const int M = ROLE == 0 ? d : H, N = ROLE == 0 ? H : d;
    const int mtn = M / 128, ntn = N / 128;
    const int per_chunk = mtn * ntn;
    const int chunk = blockIdx.x / per_chunk;
    const int tile = blockIdx.x - chunk * per_chunk;
    const int mi = tile / ntn, ni = tile - mi * ntn;
    const int tb0 = chunk * p.chunk_len;
    const int tb1 = min(T, tb0 + p.chunk_len);
    const int n_steps = (tb1 - tb0 + kTK - 1) / kTK;
    const int ldkv = p.n_kv * d;
    const int64_t th = (int64_t)q * T * H, td = (int64_t)q * T * d;
    const __bf16* A;
    const __bf16* B;
    int lda, ldb;
    if (ROLE == 0) { A = p.gb + td; lda = d; B = p.hb + th; ldb = H; }
    else { A = p.dzb + th; lda = H; B = p.keys + (int64_t)l * T * ldkv + h * d; ldb = ldkv; }
    const int rows = tb1 - tb0;
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(A + (int64_t)tb0 * lda + mi * 128, (uint32_t)((int64_t)rows * lda * 2));
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(B + (int64_t)tb0 * ldb + ni * 128, (uint32_t)((int64_t)rows * ldb * 2));
    // Copies: wave w fills rows 8 w .. 8 w + 7 of both operands, 4 rows per
    // instruction (lane i: row 8 w + 4 c + i / 16, slot i % 16).
    uint32_t va[2], vb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int row = w * 8 + c * 4 + (lane >> 4);
        const int piece = (lane & 15) ^ tsw(row);
        va[c] = (uint32_t)(row * lda * 2 + piece * 16);
        vb[c] = (uint32_t)(row * ldb * 2 + piece * 16);
    }
    auto dma = [&](int s, unsigned char* stage) {
        const uint32_t sa = (uint32_t)(s * kTK * lda * 2), sb = (uint32_t)(s * kTK * ldb * 2);
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            dma16(ra, stage + (w * 8 + c * 4) * kTRowB, va[c], sa);
            // B (H or K rows) is read by one workgroup only: non-temporal.
            // A (G or dZ rows) is shared by the two output tiles' workgroups.
            dma16<kNonTemporal>(rb, stage + kTOp + (w * 8 + c * 4) * kTRowB, vb[c], sb);
        }
    };
    const int g = lane >> 4, i16 = lane & 15;
    const int trow = 8 * g + (i16 >> 2);
    const int lane_sw = tsw(trow) | ((i16 & 3) >> 1);
    const uint32_t lane_off = (uint32_t)(trow * kTRowB + ((i16 & 1) << 3));
    auto off = [&](int m0) { return lane_off + ((uint32_t)(((m0 >> 3) ^ lane_sw)) << 4); };

    f32x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
    auto mma = [&](const unsigned char* stage) {
        bf16x8 af[4], bf[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) af[a] = tn_frag(stage, off(wm + a * 16));
#pragma unroll
        for (int b = 0; b < 4; ++b) bf[b] = tn_frag(stage + kTOp, off(wn + b * 16));
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) acc[a][b] = mfma(af[a], bf[b], acc[a][b]);
    };
    if (n_steps > 0) dma(0, s0);
    if (n_steps > 1) dma(1, s1);
    if (n_steps > 2) dma(2, s2);
    auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
        if (s + 2 < n_steps) wait_vmcnt<8>();
        else if (s + 1 < n_steps) wait_vmcnt<4>();
        else wait_vmcnt<0>();
        barrier_lds();
        if (s + 3 < n_steps) dma(s + 3, nxt);
        mma(cur);
    };
    for (int s = 0; s < n_steps; s += 4) {
        step(s, s0, s3);
        if (s + 1 < n_steps) step(s + 1, s1, s0);
        if (s + 2 < n_steps) step(s + 2, s2, s1);
        if (s + 3 < n_steps) step(s + 3, s3, s2);
    }
    wait_vmcnt<0>();
    float* out = (ROLE == 0 ? p.pw2 : p.pw1) + ((int64_t)q * p.n_chunks + chunk) * (int64_t)M * N;
    const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int m = mi * 128 + wm + a * 16 + g4 * 4;
            const int n = ni * 128 + wn + b * 16 + l16;
            *reinterpret_cast<f32x4*>(out + (int64_t)n * M + m) = acc[a][b];
        }
}

// --------------------------------------------------------------- update
// One block per problem. mode 0: loss only (slot `step`); mode 1: gradient
// step `step` (reduces the partials in a fixed order, updates the fp32
// masters, refreshes the bf16 copies); mode 2: bf16 copies only.
__global__ __launch_bounds__(256) void fit_update_kernel(FitParams p, int step, int mode) {
    const int q = blockIdx.x, tid = threadIdx.x;
    const int d = kHeadDim, H = p.hidden;
    float* w1 = p.w1 + (int64_t)q * H * d;
    float* w2 = p.w2 + (int64_t)q * d * H;
    float* b1 = p.b1 + (int64_t)q * H;
    float* b2 = p.b2 + (int64_t)q * d;
    if (mode != 2 && tid == 0 && p.losses) {
        double s = 0.0;
        for (int m = 0; m < p.m_tiles; ++m) s += (double)p.loss_p[(int64_t)q * p.m_tiles + m];
        p.losses[(int64_t)q * (p.n_steps + 1) + step] = (float)(s / (double)p.ctx_len);
    }
    if (mode == 0) return;
    if (mode == 1) {
        const float lr = p.lr;
        const float* pw1 = p.pw1 + (int64_t)q * p.n_chunks * H * d;   // [c][i][u]
        const float* pw2 = p.pw2 + (int64_t)q * p.n_chunks * H * d;   // [c][u][o]
        for (int e = tid; e < H * d; e += 256) {
            const int u = e / d, i = e - u * d;        // w1[u][i]
            float g = 0.f;
            for (int c = 0; c < p.n_chunks; ++c) g += pw1[((int64_t)c * d + i) * H + u];
            w1[e] -= lr * g;
        }
        for (int e = tid; e < d * H; e += 256) {
            const int o = e / H, u = e - o * H;        // w2[o][u]
            float g = 0.f;
            for (int c = 0; c < p.n_chunks; ++c) g += pw2[((int64_t)c * H + u) * d + o];
            w2[e] -= lr * g;
        }
        for (int u = tid; u < H; u += 256) {
            float g = 0.f;
            for (int m = 0; m < p.m_tiles; ++m) g += p.cs_dz[((int64_t)q * p.m_tiles + m) * H + u];
            b1[u] -= lr * g;
        }
        for (int o = tid; o < d; o += 256) {
            float g = 0.f;
            for (int m = 0; m < p.m_tiles; ++m) g += p.cs_g[((int64_t)q * p.m_tiles + m) * d + o];
            b2[o] -= lr * g;
        }
        __syncthreads();
    }
    uint16_t* w1b = reinterpret_cast<uint16_t*>(p.w1b) + (int64_t)q * H * d;
    uint16_t* w2b = reinterpret_cast<uint16_t*>(p.w2b) + (int64_t)q * d * H;
    uint16_t* w2tb = reinterpret_cast<uint16_t*>(p.w2tb) + (int64_t)q * H * d;
    for (int e = tid; e < H * d; e += 256) w1b[e] = f32_to_bf16_bits(w1[e]);
    for (int e = tid; e < d * H; e += 256) {
        const int o = e / H, u = e - o * H;
        const uint16_t v = f32_to_bf16_bits(w2[e]);
        w2b[e] = v;
        w2tb[(int64_t)u * d + o] = v;
    }
}

hipError_t launch_fit(const FitParams& p, void* ev_begin, void* ev_end, hipStream_t s) {
    const unsigned P = (unsigned)p.n_probs;
    const unsigned mt8 = (unsigned)((p.m_tiles + 7) / 8 * 8);
    const dim3 gz(mt8 * (unsigned)(p.hidden / kFN), P), gg(mt8, P);
    const dim3 t2((unsigned)(p.n_chunks * (kHeadDim / 128) * (p.hidden / 128)), P);
    hipError_t e;
    hipLaunchKernelGGL(fit_update_kernel, dim3(P), dim3(256), 0, s, p, 0, 2);
    if (ev_begin && (e = hipEventRecord(static_cast<hipEvent_t>(ev_begin), s)) != hipSuccess) return e;
    for (int it = 0; it < p.n_steps; ++it) {
        hipLaunchKernelGGL((fit_nt_kernel<kEpiZ>), gz, dim3(kFThreads), 0, s, p);
        hipLaunchKernelGGL((fit_nt_kernel<kEpiG>), gg, dim3(kFThreads), 0, s, p);
        hipLaunchKernelGGL((fit_nt_kernel<kEpiDz>), gz, dim3(kFThreads), 0, s, p);
        hipLaunchKernelGGL((fit_tn_kernel<0>), t2, dim3(256), 0, s, p);
        hipLaunchKernelGGL((fit_tn_kernel<1>), t2, dim3(256), 0, s, p);
        hipLaunchKernelGGL(fit_update_kernel, dim3(P), dim3(256), 0, s, p, it, 1);
    }
    if (ev_end && (e = hipEventRecord(static_cast<hipEvent_t>(ev_end), s)) != hipSuccess) return e;
    hipLaunchKernelGGL((fit_nt_kernel<kEpiZ>), gz, dim3(kFThreads), 0, s, p);
    hipLaunchKernelGGL((fit_nt_kernel<kEpiG>), gg, dim3(kFThreads), 0, s, p);
    hipLaunchKernelGGL(fit_update_kernel, dim3(P), dim3(256), 0, s, p, p.n_steps, 0);
    return hipGetLastError();
}

}  // namespace lowram
