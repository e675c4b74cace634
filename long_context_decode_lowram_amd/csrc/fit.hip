// Test-time fit of the per-head value predictor's nonlinear branch.
//
// explainer, Slim Attention paragraph: the predictor starts from the linear
// pseudoinverse map and a small nonlinear branch learns the rest from the
// current context; explainer, cost paragraph: the fit takes gradient steps
// per context at prefill. Loss L = (1 / T) sum_t ||v_hat_t - v_t||^2, plain
// gradient descent on W1, b1, W2, b2 (W_lin fixed). Per step and problem
// (layer, KV head), with weights stored output-major:
//   H = gelu(K W1^T + b1)                              fit_fused_kernel, one workgroup per
//   G = (2 / T)(K W_lin^T + H W2^T + b2 - V)           (problem, 64-token tile) (+ loss, sum_t G,
//   dZ = (G W2) * gelu'(K W1^T + b1)                   sum_t dZ; the pre-activations are recomputed)
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

constexpr int kFN = 128;                 // outputs per product tile (MFMA A operand rows)
constexpr int kFK = 64;                  // contraction step
constexpr int kFRowB = kFK * 2;          // 128-byte LDS rows
constexpr int kFOp0 = kFN * kFRowB;      // 16 KB: a weight stage buffer
constexpr int kFThreads = 512;

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

// --------------------------------------------------------------- fused
// The three token-tile products of a gradient step in one workgroup per
// (problem, 64-token tile), so the tile's keys are read from HBM once and H
// and G are never read back from it:
//   for each 128-wide hidden tile u:  Z_u = K W1_u^T;  H_u = gelu(Z_u + b1_u)
//                                     (stored for dW2, and kept in LDS);
//                                     V_hat += H_u W2_u^T
//   V_hat += K W_lin^T;  G = (2 / T)(V_hat + b2 - V)   (stored, kept in LDS)
//   for each hidden tile u:           dZ_u = (G W2_u) * gelu'(K W1_u^T + b1_u)
// (BACKWARD = false stops after G: the loss after the last step). The keys and
// H_u (then G, in the same place) stay resident in LDS as the token operand
// ([64 tokens][128] bf16, two 64-wide halves in swizzled 128-byte rows); the
// weight rows stream through two 16 KB stage buffers, 64 columns of the
// contraction at a time. 66 KB of LDS, so two workgroups share a CU and hide
// each other's copy latency. Eight waves: wave w covers outputs 64 (w & 1)
// .. + 63 and tokens 16 (w >> 1) .. + 15; lane (l16, g4) ends with outputs
// n .. n + 3 (n = 4 g4 + 16 a) of token l16. H, G, dZ, the column sums and
// the loss partials have the values and layout the weight-gradient products
// and the update read. Workgroups of one problem run on one XCD at a time
// (its L2 then holds the problem's weights): XCD x takes problems x, x + 8,
// ..., each problem's tiles in turn.
constexpr int kFTok = 64;                       // tokens per tile
constexpr int kFHalf = kFTok * kFRowB;          // one 64-wide half of a resident tile: 8 KB

template <bool BACKWARD>
__global__ __launch_bounds__(kFThreads, 2) void fit_fused_kernel(FitParams p, int n_per_xcd) {
    __shared__ __attribute__((aligned(16))) unsigned char kt[2 * kFHalf];   // keys of the tile
    __shared__ __attribute__((aligned(16))) unsigned char ht[2 * kFHalf];   // H_u, then G
    __shared__ __attribute__((aligned(16))) unsigned char ws0[kFOp0], ws1[kFOp0];
    __shared__ float red_cs[4][kFN];
    __shared__ float red_loss[8];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // blockIdx -> (problem, token tile): XCD x = blockIdx % 8 walks its own
    // list of (problem, tile) pairs in order.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= n_per_xcd) return;
    const int q = (local / p.m_tiles) * 8 + xcd;
    const int mt = local - (local / p.m_tiles) * p.m_tiles;
    if (q >= p.n_probs) return;
    const int l = q / p.n_kv, h = q - l * p.n_kv;
    const int d = kHeadDim, H = p.hidden, T = p.ctx_len;
    const int t0 = mt * kFTok;
    const int ldkv = p.n_kv * d;
    const int64_t th = (int64_t)q * T * H, td = (int64_t)q * T * d;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int wn = (w & 1) * 64, wt = (w >> 1) * 16;
    const int dma_row = lane >> 3;
    const uint32_t dma_piece = (uint32_t)(((lane & 7) ^ dma_row) * 16);

    // The keys of the tile, both 64-wide halves (rows past T read as zeros);
    // read once: non-temporal. Wave w copies rows 8 w .. 8 w + 7.
    {
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.keys + (int64_t)l * T * ldkv + h * d + (int64_t)t0 * ldkv,
                                                      (uint32_t)((int64_t)max(0, T - t0) * ldkv * 2));
#pragma unroll
        for (int half = 0; half < 2; ++half)
            dma16<kNonTemporal>(rk, kt + half * kFHalf + w * 8 * kFRowB,
                                (uint32_t)(((w * 8 + dma_row) * ldkv + half * kFK) * 2) + dma_piece, 0u);
    }
    // 128 weight rows (outputs n0 .. n0 + 127 of a row-major matrix with row
    // stride ldw), contraction columns k0 .. k0 + 63, into a stage buffer.
    auto dma_w = [&](const __bf16* wmat, int ldw, int n0, int k0, unsigned char* stage) {
        const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wmat + (int64_t)n0 * ldw, (uint32_t)(kFN * ldw * 2));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r0 = (w * 2 + c) * 8;
            dma16(rw, stage + r0 * kFRowB, (uint32_t)(((r0 + dma_row) * ldw + k0) * 2) + dma_piece, 0u);
        }
    };
    auto mma = [&](const unsigned char* op0, const unsigned char* op1, f32x4 (&acc)[4]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) af[a] = lds16(op0, fslot(wn + a * 16 + l16, ks * 4 + g4));
            const bf16x8 bf = lds16(op1, fslot(wt + l16, ks * 4 + g4));
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[a] = mfma(af[a], bf, acc[a]);
        }
    };
    // acc (+)= W[n0 .. n0 + 127][k0 .. k0 + 127] . tok^T over a resident
    // 128-wide token tile (two halves): two 64-wide steps, weights double
    // buffered. The barriers also publish resident-tile rows written before
    // the call, and on return every wave is done with the stage buffers and
    // with tok.
    auto contract = [&](const __bf16* wmat, int ldw, int n0, int k0, const unsigned char* tok, f32x4 (&acc)[4],
                        bool zero) {
        if (zero) {
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        dma_w(wmat, ldw, n0, k0, ws0);
        dma_w(wmat, ldw, n0, k0 + kFK, ws1);
        wait_vmcnt<2>();                    // this wave's step 0 copies (the older two) have landed
        barrier_lds();                      // (step 1's copies stay in flight)
        mma(ws0, tok, acc);
        wait_vmcnt<0>();
        barrier_lds();
        mma(ws1, tok + kFHalf, acc);
        barrier_lds();
    };
    // Store a lane's four consecutive outputs (as bf16) of token row r into a
    // resident tile: output n lands in half n / 64, piece (n % 64) / 8.
    auto put = [&](unsigned char* tile, int r, int n, u32x2 v) {
        const int hf = n >> 6, nn = n & 63;
        *reinterpret_cast<u32x2*>(tile + hf * kFHalf + fslot(r, nn >> 3) + (nn & 7) * 2) = v;
    };
    // Column sums of a 128-output tile over this tile's tokens, in a fixed
    // order: lanes l16 = 0..15 share outputs, then the 4 token waves of an
    // output half meet in LDS.
    auto colsum = [&](float (&cs)[4][4], float* dst) {
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
        __syncthreads();
        if (tid < kFN) dst[tid] = ((red_cs[0][tid] + red_cs[1][tid]) + red_cs[2][tid]) + red_cs[3][tid];
    };
    const float gscale = 2.0f / (float)T;
    const __bf16* w1b = p.w1b + (int64_t)q * H * d;
    const __bf16* w2b = p.w2b + (int64_t)q * d * H;
    const __bf16* w2tb = p.w2tb + (int64_t)q * H * d;
    const __bf16* wl = p.w_lin + (int64_t)q * d * d;
    const float* b1 = p.b1 + (int64_t)q * H;
    const float* b2 = p.b2 + (int64_t)q * d;
    const int r = wt + l16, t = t0 + r;          // this lane's token row
    f32x4 acc[4], accv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) accv[a] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- forward: H_u and V_hat
    for (int u0 = 0; u0 < H; u0 += kFN) {
        contract(w1b, d, u0, 0, kt, acc, true);                 // Z_u
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int n = wn + a * 16 + g4 * 4;
            u32x2 hv = {0u, 0u};
            if (t < T) {
                float v4[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) v4[v] = gelu_f(acc[a][v] + b1[u0 + n + v]);
                hv = u32x2{pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])};
                *reinterpret_cast<u32x2*>(p.hb + th + (int64_t)t * H + u0 + n) = hv;
            }
            put(ht, r, n, hv);
        }
        contract(w2b, H, 0, u0, ht, accv, false);              // V_hat += H_u W2_u^T
    }
    contract(wl, d, 0, 0, kt, accv, false);                     // V_hat += K W_lin^T

    // ---- G (into the H tile's place: its last reader has passed the barrier
    // that ends the contraction above), loss, column sums of G
    {
        float cs[4][4];
        float loss = 0.f;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int n = wn + a * 16 + g4 * 4;
            u32x2 gv = {0u, 0u};
#pragma unroll
            for (int v = 0; v < 4; ++v) cs[a][v] = 0.f;
            if (t < T) {
                const u32x2 vv = *reinterpret_cast<const u32x2*>(p.v + ((int64_t)l * T + t) * ldkv + h * d + n);
                const float vt[4] = {bf16_lo(vv[0]), bf16_hi(vv[0]), bf16_lo(vv[1]), bf16_hi(vv[1])};
                float g[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float e = accv[a][v] + b2[n + v] - vt[v];
                    loss = fmaf(e, e, loss);
                    g[v] = gscale * e;
                    cs[a][v] = g[v];
                }
                gv = u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
                *reinterpret_cast<u32x2*>(p.gb + td + (int64_t)t * d + n) = gv;
            }
            put(ht, r, n, gv);
        }
        for (int off = 32; off > 0; off >>= 1) loss += __shfl_xor(loss, off, kWave);
        if (lane == 0) red_loss[w] = loss;
        colsum(cs, p.cs_g + ((int64_t)q * p.m_tiles + mt) * d);
        if (tid == 0) {
            float sum = 0.f;
            for (int i = 0; i < 8; ++i) sum += red_loss[i];
            p.loss_p[(int64_t)q * p.m_tiles + mt] = sum;
        }
    }
    if (!BACKWARD) return;

    // ---- backward: dZ_u = (G W2_u) * gelu'(Z_u + b1_u), column sums of dZ
    for (int u0 = 0; u0 < H; u0 += kFN) {
        contract(w1b, d, u0, 0, kt, accv, true);                // Z_u again (cheaper than keeping every tile)
        contract(w2tb, d, u0, 0, ht, acc, true);                // G W2_u
        float cs[4][4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int n = wn + a * 16 + g4 * 4;
#pragma unroll
            for (int v = 0; v < 4; ++v) cs[a][v] = 0.f;
            if (t < T) {
                float dz[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    dz[v] = acc[a][v] * gelu_grad_f(accv[a][v] + b1[u0 + n + v]);
                    cs[a][v] = dz[v];
                }
                *reinterpret_cast<u32x2*>(p.dzb + th + (int64_t)t * H + u0 + n) =
                    u32x2{pack_bf16x2(dz[0], dz[1]), pack_bf16x2(dz[2], dz[3])};
            }
        }
        colsum(cs, p.cs_dz + ((int64_t)q * p.m_tiles + mt) * H + u0);
        __syncthreads();                    // red_cs is free for the next hidden tile
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
// Grid (problem, slice of kUpdSlices). mode 0: loss only (slot `step`, slice
// 0); mode 1: gradient step `step`: each weight's partials reduced in a fixed
// order by the one thread that owns it, which updates the fp32 master and
// writes its bf16 copies; mode 2: bf16 copies only. Threads walk the
// weights in the order of the partials' fastest axis, so the (n_chunks x
// more numerous) partial reads coalesce.
constexpr int kUpdSlices = 8;

__global__ __launch_bounds__(256) void fit_update_kernel(FitParams p, int step, int mode) {
    const int q = blockIdx.x, slice = blockIdx.y, tid = threadIdx.x;
    const int d = kHeadDim, H = p.hidden;
    const int e0 = slice * 256 + tid, es = 256 * kUpdSlices;
    float* w1 = p.w1 + (int64_t)q * H * d;
    float* w2 = p.w2 + (int64_t)q * d * H;
    float* b1 = p.b1 + (int64_t)q * H;
    float* b2 = p.b2 + (int64_t)q * d;
    uint16_t* w1b = reinterpret_cast<uint16_t*>(p.w1b) + (int64_t)q * H * d;
    uint16_t* w2b = reinterpret_cast<uint16_t*>(p.w2b) + (int64_t)q * d * H;
    uint16_t* w2tb = reinterpret_cast<uint16_t*>(p.w2tb) + (int64_t)q * H * d;
    if (mode != 2 && slice == 0 && tid == 0 && p.losses) {
        double s = 0.0;
        for (int m = 0; m < p.m_tiles; ++m) s += (double)p.loss_p[(int64_t)q * p.m_tiles + m];
        p.losses[(int64_t)q * (p.n_steps + 1) + step] = (float)(s / (double)p.ctx_len);
    }
    if (mode == 0) return;
    if (mode == 1) {
        const float lr = p.lr;
        const float* pw1 = p.pw1 + (int64_t)q * p.n_chunks * H * d;   // [c][i][u]
        const float* pw2 = p.pw2 + (int64_t)q * p.n_chunks * H * d;   // [c][u][o]
        for (int e = e0; e < H * d; e += es) {
            const int i = e / H, u = e - i * H;        // w1[u][i]; partials contiguous in u
            float g = 0.f;
            for (int c = 0; c < p.n_chunks; ++c) g += pw1[((int64_t)c * d + i) * H + u];
            const float x = w1[(int64_t)u * d + i] - lr * g;
            w1[(int64_t)u * d + i] = x;
            w1b[(int64_t)u * d + i] = f32_to_bf16_bits(x);
        }
        for (int e = e0; e < d * H; e += es) {
            const int u = e / d, o = e - u * d;        // w2[o][u]; partials contiguous in o
            float g = 0.f;
            for (int c = 0; c < p.n_chunks; ++c) g += pw2[((int64_t)c * H + u) * d + o];
            const float x = w2[(int64_t)o * H + u] - lr * g;
            w2[(int64_t)o * H + u] = x;
            const uint16_t v = f32_to_bf16_bits(x);
            w2b[(int64_t)o * H + u] = v;
            w2tb[e] = v;                               // w2tb[u][o]
        }
        for (int u = e0; u < H; u += es) {
            float g = 0.f;
            for (int m = 0; m < p.m_tiles; ++m) g += p.cs_dz[((int64_t)q * p.m_tiles + m) * H + u];
            b1[u] -= lr * g;
        }
        for (int o = e0; o < d; o += es) {
            float g = 0.f;
            for (int m = 0; m < p.m_tiles; ++m) g += p.cs_g[((int64_t)q * p.m_tiles + m) * d + o];
            b2[o] -= lr * g;
        }
        return;
    }
    for (int e = e0; e < H * d; e += es) w1b[e] = f32_to_bf16_bits(w1[e]);
    for (int e = e0; e < d * H; e += es) {
        const int o = e / H, u = e - o * H;
        const uint16_t v = f32_to_bf16_bits(w2[e]);
        w2b[e] = v;
        w2tb[(int64_t)u * d + o] = v;
    }
}

hipError_t launch_fit(const FitParams& p, void* ev_begin, void* ev_end, hipStream_t s) {
    const unsigned P = (unsigned)p.n_probs;
    const dim3 t2((unsigned)(p.n_chunks * (kHeadDim / 128) * (p.hidden / 128)), P);
    hipError_t e;
    hipLaunchKernelGGL(fit_update_kernel, dim3(P, kUpdSlices), dim3(256), 0, s, p, 0, 2);
    if (ev_begin && (e = hipEventRecord(static_cast<hipEvent_t>(ev_begin), s)) != hipSuccess) return e;
    // Fused token-tile products: (problem, tile) pairs dealt to the 8 XCDs by
    // problem (see fit_fused_kernel).
    const int per_xcd = (int)(((P + 7) / 8) * (unsigned)p.m_tiles);
    const dim3 gf((unsigned)per_xcd * 8u);
    for (int it = 0; it < p.n_steps; ++it) {
        hipLaunchKernelGGL((fit_fused_kernel<true>), gf, dim3(kFThreads), 0, s, p, per_xcd);
        hipLaunchKernelGGL((fit_tn_kernel<0>), t2, dim3(256), 0, s, p);
        hipLaunchKernelGGL((fit_tn_kernel<1>), t2, dim3(256), 0, s, p);
        hipLaunchKernelGGL(fit_update_kernel, dim3(P, kUpdSlices), dim3(256), 0, s, p, it, 1);
    }
    if (ev_end && (e = hipEventRecord(static_cast<hipEvent_t>(ev_end), s)) != hipSuccess) return e;
    hipLaunchKernelGGL((fit_fused_kernel<false>), gf, dim3(kFThreads), 0, s, p, per_xcd);
    hipLaunchKernelGGL(fit_update_kernel, dim3(P, kUpdSlices), dim3(256), 0, s, p, p.n_steps, 0);

    return hipGetLastError();
}

}  // namespace lowram
