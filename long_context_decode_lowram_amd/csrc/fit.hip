// Test-time fit of the per-head value predictor's nonlinear branch.
//
// explainer, Slim Attention paragraph: the predictor starts from the linear
// pseudoinverse map and a small nonlinear branch learns the rest from the
// current context; explainer, cost paragraph: the fit takes gradient steps
// per context at prefill. Loss L = (1 / T) sum_t ||v_hat_t - v_t||^2, plain
// gradient descent on W1, b1, W2, b2 (W_lin fixed). Per step and problem
// (layer, KV head), with weights stored output-major:
//   Z = K W1^T + b1,  H = gelu(Z)
//   E = K W_lin^T + H W2^T + b2 - V                     fit_fwd_kernel (loss partials too)
//   dZ = (E W2) * gelu'(Z)
//   E^T H,  dZ^T K,  sum_t E,  sum_t dZ                 fit_bwd_kernel (Z and H recomputed)
//   theta -= lr (2 / T) (those sums)                    fit_update_kernel
// (dL/dW2 = G^T H with G = (2 / T) E, and so on: every gradient is linear in
// E, so the factor 2 / T is applied once, in the update.) Products on bf16
// MFMA with fp32 sums; the parameters are fp32 masters with bf16 copies for
// the products. Only E goes through HBM between the passes.
#include <hip/hip_runtime.h>
#include <math.h>

#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace lowram {

constexpr int kFitThreads = 512;          // eight waves, two per SIMD
constexpr int kLdsAll = 163840;           // the whole LDS of a CU
constexpr int kFwdMaxHidden = 256;        // widest hidden layer whose weights stay resident in LDS

// GELU and its derivative from the normal tail fit (normal_tail): with
// q = Q(|z|), Phi(z) = 1 - q for z >= 0 and q below; gelu(z) = z Phi(z) and
// gelu'(z) = Phi(z) + z phi(z), phi(z) = 2^(-z^2 / (2 ln 2) + log2(1 / sqrt(2 pi))).
__device__ __forceinline__ float gelu_q(float z, float q) {
    return fmaf(-fabsf(z), q, __builtin_amdgcn_fmed3f(z, 0.0f, 3.0e38f));
}
__device__ __forceinline__ void gelu_and_grad(float z, float& h, float& g) {
    const float q = normal_tail(fabsf(z));
    const float cdf = z >= 0.0f ? 1.0f - q : q;
    const float phi = __builtin_amdgcn_exp2f(fmaf(-0.72134752044448170f * z, z, -1.3257480647361593f));
    h = z * cdf;
    g = fmaf(z, phi, cdf);
}

// Two floats to packed bf16 (round to nearest even, one v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 16-byte piece `piece` of row `row` of an LDS matrix with `row_bytes`-byte
// rows, swizzled: piece p of row r sits in slot p ^ (r & 15). Sixteen lanes
// reading the same logical piece of sixteen consecutive rows then hit
// sixteen different bank groups.
__device__ __forceinline__ uint32_t sw_off(int row, int piece, int row_bytes) {
    return (uint32_t)(row * row_bytes + ((piece ^ (row & 15)) << 4));
}

// ------------------------------------------------------------ forward
// One workgroup per (problem, token range); W1 [h][d], W2 [d][h] and W_lin
// [d][d] stay in LDS for the workgroup's life (160 KB at h = 256, the MFMA A
// operands); each wave takes 32-token tiles in turn (tile w, w + 8, ...) and
// holds the tile's keys as B-operand fragments read straight from HBM, so no
// token data passes through LDS and the waves never wait for each other.
// Per tile and 32 hidden units c:
//   Z^T (2 x 2 tiles of 16) = W1[32 c ..] K^T + b1      16 MFMAs
//   H^T = gelu(Z^T) (gelu_tail16), bf16: lane (token j, g4) holds units
//         4 g4 + i and 16 + 4 g4 + i, the k-slots of one B fragment
//   V_hat^T (8 x 2 tiles) += W2[:, 32 c ..] H^T          16 MFMAs
// W2's columns are stored in LDS in that k-slot order (within every 32
// units, piece g4 holds units 4 g4 .. + 3 and 16 + 4 g4 .. + 3), so its A
// fragments are single 16-byte reads. The V_hat^T accumulators start at b2;
// then V_hat^T += W_lin K^T, and V is subtracted on the matrix pipe too (one
// MFMA per tile pair with a -I fragment against V read like the keys), so E
// comes out of the accumulators; the lane's squared errors go to a per-wave
// loss partial.
template <bool WRITE_E, int NC>                      // NC = h / 32 hidden chunks (4 or 8)
__global__ __launch_bounds__(kFitThreads, 1) void fit_fwd_kernel(FitParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char lds[kLdsAll];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    constexpr int H = 32 * NC;
    const int T = p.ctx_len, d = kHeadDim;
    const int q = blockIdx.x / p.fwd_ranges, rg = blockIdx.x - q * p.fwd_ranges;
    const int l = q / p.n_kv, h = q - l * p.n_kv;
    const int ldkv = p.n_kv * d;
    const int w2row = 2 * H;                          // bytes per W2 row
    unsigned char* const w1s = lds;                   // [h][d]
    unsigned char* const w2s = lds + H * 256;         // [d][h], permuted columns
    unsigned char* const wls = w2s + d * w2row;       // [d][d]

    {
        // all loads first, then the LDS stores (H <= 256: at most 8 W1 and W2
        // pieces and 4 W_lin pieces per thread)
        const u32x4* w1g = reinterpret_cast<const u32x4*>(p.w1b + (int64_t)q * H * d);
        const u32x4* wlg = reinterpret_cast<const u32x4*>(p.w_lin + (int64_t)q * d * d);
        const u32x2* w2g = reinterpret_cast<const u32x2*>(p.w2b + (int64_t)q * d * H);
        const int npc = H / 8;                        // pieces per W2 row
        u32x4 v1[8], vl[4], v2[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = tid + k * kFitThreads;
            if (i < H * 16) v1[k] = w1g[i];
            if (i < d * npc) {
                const int r = i / npc, pc = i - r * npc;      // piece pc = 4 c + gg of row r
                const int c = pc >> 2, gg = pc & 3;
                const u32x2 lo = w2g[(r * H + 32 * c + 4 * gg) >> 2];
                const u32x2 hi = w2g[(r * H + 32 * c + 16 + 4 * gg) >> 2];
                v2[k] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            }
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) vl[k] = wlg[tid + k * kFitThreads];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = tid + k * kFitThreads;
            if (i < H * 16) *reinterpret_cast<u32x4*>(w1s + sw_off(i >> 4, i & 15, 256)) = v1[k];
            if (i < d * npc) *reinterpret_cast<u32x4*>(w2s + sw_off(i / npc, i % npc, w2row)) = v2[k];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = tid + k * kFitThreads;
            *reinterpret_cast<u32x4*>(wls + sw_off(i >> 4, i & 15, 256)) = vl[k];
        }
    }
    __syncthreads();

    const int n_tiles = (T + 31) / 32;
    const int per = (n_tiles + p.fwd_ranges - 1) / p.fwd_ranges;
    const int tb = rg * per, te = min(n_tiles, tb + per);
    const uint32_t kv_bytes = (uint32_t)((int64_t)T * ldkv * 2);   // below 2^31 (checked on the host)
    const uint32_t ldkv_u = (uint32_t)ldkv;                          // offsets of rows past T stay below 2^32
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.keys + (int64_t)l * T * ldkv + h * d, kv_bytes);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(p.v + (int64_t)l * T * ldkv + h * d, kv_bytes);
    const __amdgpu_buffer_rsrc_t rgo = buffer_rsrc(p.gb + (int64_t)q * T * d, (uint32_t)((int64_t)T * d * 2));
    const float* const b1 = p.b1 + (int64_t)q * H;
    const float* const b2 = p.b2 + (int64_t)q * d;
    // -I as A fragments (rows d, k-slots d): neg_eye[e] serves the d tiles with
    // dt % 2 == e against k-step dt / 2; lane (i, g4) holds -1 in slot
    // 16 e + i - 8 g4 when that lies in 0..7.
    bf16x8 neg_eye[2];
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)
            neg_eye[e][jj] = (__bf16)(16 * e + l16 - 8 * g4 == jj ? -1.0f : 0.0f);
    // Keys of a tile as B fragments: kf[tt][s] = K[t0 + 16 tt + l16][32 s + 8 g4 .. + 7]
    // (rows past T read as zeros).
    auto load_k = [&](int tile, bf16x8 (&kf)[2][4]) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                kf[tt][s] = as_bf16x8(__builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rk, ((uint32_t)(tile * 32 + 16 * tt + l16) * ldkv_u + 32 * s + 8 * g4) * 2u, 0, 0)));
    };
    float loss = 0.f;
    bf16x8 kf[2][4];
    for (int tile = tb + w; tile < te; tile += 8) {
        const int t0 = tile * 32;
        // A zero the compiler cannot see through: the W_lin fragments and b2
        // below are the same for every tile, and hoisting their loads out of
        // the loop would hold 160 registers for the kernel's life.
        int zero = 0;
        asm volatile("" : "+v"(zero));
        // Loads in the order they are needed (the counter of outstanding
        // loads drains in order): keys, the first hidden chunks' b1, b2 (the
        // accumulators start at it), V for the last step.
        load_k(tile, kf);
        // b1 of hidden chunks c and c + 1 (loaded two chunks ahead)
        f32x4 bq[3][2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
                bq[c][ht] = *reinterpret_cast<const f32x4*>(b1 + 32 * c + 16 * ht + 4 * g4 + zero);
        f32x4 acc[8][2];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const f32x4 bb = *reinterpret_cast<const f32x4*>(b2 + 16 * dt + 4 * g4 + zero);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[dt][tt] = bb;
        }
        // V as B fragments, like the keys: vf[tt][s] = V[t0 + 16 tt + l16][32 s + 8 g4 .. + 7]
        bf16x8 vf[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int s = 0; s < 4; ++s)
                vf[tt][s] = as_bf16x8(__builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                               rv, ((uint32_t)(t0 + 16 * tt + l16) * ldkv_u + 32 * s + 8 * g4) * 2u, 0, 0)));
        __builtin_amdgcn_sched_barrier(0);            // every load of the tile is in flight before the products
        // Z^T of hidden chunk c: zt[2 ht + tt], started at b1, 16 MFMAs over the keys
        auto zchunk = [&](int c, f32x4 (&zt)[4]) {
#pragma unroll
            for (int ht = 0; ht < 2; ++ht)
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) zt[2 * ht + tt] = bq[c % 3][ht];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int ht = 0; ht < 2; ++ht) {
                    const bf16x8 wf = lds16(w1s, sw_off(32 * c + 16 * ht + l16, 4 * s + g4, 256));
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt) zt[2 * ht + tt] = mfma(wf, kf[tt][s], zt[2 * ht + tt]);
                }
        };
        // Chunks in a software pipeline: the next chunk's Z MFMAs are issued
        // between this chunk's GELU operations, so the matrix pipe and the
        // vector ALU work side by side; then this chunk's W2 products.
        f32x4 zc[4], zn[4];
        zchunk(0, zc);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            if (c + 2 < NC) {
#pragma unroll
                for (int ht = 0; ht < 2; ++ht)
                    bq[(c + 2) % 3][ht] = *reinterpret_cast<const f32x4*>(b1 + 32 * (c + 2) + 16 * ht + 4 * g4);
                __builtin_amdgcn_sched_barrier(0);    // issue the prefetch here, not next to its use
            }
            if (c + 1 < NC) zchunk(c + 1, zn);
            gelu_tail16(zc);                          // H^T in place
            bf16x8 hf[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) hf[tt] = pack8(zc[tt], zc[2 + tt]);
            if (c + 1 < NC) {
                __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);      // the next chunk's W1 fragments
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // then a share of the GELU
                }
            }
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const bf16x8 wf = lds16(w2s, sw_off(16 * dt + l16, 4 * c + g4, w2row));
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) acc[dt][tt] = mfma(wf, hf[tt], acc[dt][tt]);
            }
            if (c + 1 < NC) {
#pragma unroll
                for (int i = 0; i < 4; ++i) zc[i] = zn[i];
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
                const bf16x8 wf = lds16(wls, sw_off(16 * dt + l16, 4 * s + g4, 256) + zero);
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) acc[dt][tt] = mfma(wf, kf[tt][s], acc[dt][tt]);
            }
        // E^T = V_hat^T - V^T: d tile dt meets the k-step dt / 2 of V
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) acc[dt][tt] = mfma(neg_eye[dt & 1], vf[tt][dt >> 1], acc[dt][tt]);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int t = t0 + 16 * tt + l16;
            const bool valid = t < T;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (valid) loss = fmaf(acc[dt][tt][i], acc[dt][tt][i], loss);
                if (WRITE_E)      // rows past T fall outside the descriptor and are dropped
                    __builtin_amdgcn_raw_buffer_store_b64(
                        __builtin_bit_cast(__attribute__((ext_vector_type(2))) unsigned,
                                           u32x2{pack_bf16x2(acc[dt][tt][0], acc[dt][tt][1]),
                                                 pack_bf16x2(acc[dt][tt][2], acc[dt][tt][3])}),
                        rgo, (uint32_t)((t * d + 16 * dt + 4 * g4) * 2), 0, 0);
            }
        }
    }
    loss = wave_sum(loss);
    if (lane == 0) p.loss_p[((int64_t)q * p.fwd_ranges + rg) * 8 + w] = loss;
}

// ------------------------------------------------------ tiled forward
// The forward for hidden layers too wide to keep resident (h > 256): one
// workgroup per (problem, 64-token tile); the keys and H_u stay in LDS as the
// token operand and the weight rows stream through two 16 KB stage buffers,
// 64 columns of the contraction at a time. Eight waves: wave w covers
// outputs 64 (w & 1) .. + 63 and tokens 16 (w >> 1) .. + 15; lane (l16, g4)
// ends with outputs n .. n + 3 (n = 4 g4 + 16 a) of token l16.
constexpr int kTN = 128;                 // outputs per product tile
constexpr int kTK = 64;                  // contraction step
constexpr int kTRowB = kTK * 2;          // 128-byte LDS rows
constexpr int kTOp = kTN * kTRowB;       // 16 KB: a weight stage buffer
constexpr int kTTok = 64;                // tokens per tile
constexpr int kTHalf = kTTok * kTRowB;   // one 64-wide half of a resident tile: 8 KB

__device__ __forceinline__ uint32_t tslot(int row, int piece) {
    return (uint32_t)(row * kTRowB + ((piece ^ (row & 7)) << 4));
}

template <bool WRITE_E>
__global__ __launch_bounds__(kFitThreads, 2) void fit_fwd_tiled_kernel(FitParams p, int n_per_xcd) {
    __shared__ __attribute__((aligned(16))) unsigned char kt[2 * kTHalf];   // keys of the tile
    __shared__ __attribute__((aligned(16))) unsigned char ht[2 * kTHalf];   // H_u
    __shared__ __attribute__((aligned(16))) unsigned char ws0[kTOp], ws1[kTOp];
    __shared__ float red_loss[8];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // blockIdx -> (problem, token tile): XCD x = blockIdx % 8 walks its own
    // problems' tiles in order, so its L2 holds those problems' weights.
    const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
    if (local >= n_per_xcd) return;
    const int q = (local / p.m_tiles) * 8 + xcd;
    const int mt = local - (local / p.m_tiles) * p.m_tiles;
    if (q >= p.n_probs) return;
    const int l = q / p.n_kv, h = q - l * p.n_kv;
    const int d = kHeadDim, H = p.hidden, T = p.ctx_len;
    const int t0 = mt * kTTok;
    const int ldkv = p.n_kv * d;
    const int l16 = lane & 15, g4 = lane >> 4;
    const int wn = (w & 1) * 64, wt = (w >> 1) * 16;
    const int dma_row = lane >> 3;
    const uint32_t dma_piece = (uint32_t)(((lane & 7) ^ dma_row) * 16);

    {
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(p.keys + (int64_t)l * T * ldkv + h * d + (int64_t)t0 * ldkv,
                                                      (uint32_t)((int64_t)max(0, T - t0) * ldkv * 2));
#pragma unroll
        for (int half = 0; half < 2; ++half)
            dma16<kNonTemporal>(rk, kt + half * kTHalf + w * 8 * kTRowB,
                                (uint32_t)(((w * 8 + dma_row) * ldkv + half * kTK) * 2) + dma_piece, 0u);
    }
    auto dma_w = [&](const __bf16* wmat, int ldw, int n0, int k0, unsigned char* stage) {
        const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wmat + (int64_t)n0 * ldw, (uint32_t)(kTN * ldw * 2));
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int r0 = (w * 2 + c) * 8;
            dma16(rw, stage + r0 * kTRowB, (uint32_t)(((r0 + dma_row) * ldw + k0) * 2) + dma_piece, 0u);
        }
    };
    auto mma = [&](const unsigned char* op0, const unsigned char* op1, f32x4 (&acc)[4]) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
            bf16x8 af[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) af[a] = lds16(op0, tslot(wn + a * 16 + l16, ks * 4 + g4));
            const bf16x8 bf = lds16(op1, tslot(wt + l16, ks * 4 + g4));
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[a] = mfma(af[a], bf, acc[a]);
        }
    };
    // acc (+)= W[n0 .. n0 + 127][k0 .. k0 + 127] . tok^T over a resident
    // 128-wide token tile (two halves), weights double buffered. On return
    // every wave is done with the stage buffers and with tok.
    auto contract = [&](const __bf16* wmat, int ldw, int n0, int k0, const unsigned char* tok, f32x4 (&acc)[4],
                        bool zero) {
        if (zero) {
#pragma unroll
            for (int a = 0; a < 4; ++a) acc[a] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        dma_w(wmat, ldw, n0, k0, ws0);
        dma_w(wmat, ldw, n0, k0 + kTK, ws1);
        wait_vmcnt<2>();
        barrier_lds();
        mma(ws0, tok, acc);
        wait_vmcnt<0>();
        barrier_lds();
        mma(ws1, tok + kTHalf, acc);
        barrier_lds();
    };
    auto put = [&](unsigned char* tile, int r, int n, u32x2 v) {
        const int hf = n >> 6, nn = n & 63;
        *reinterpret_cast<u32x2*>(tile + hf * kTHalf + tslot(r, nn >> 3) + (nn & 7) * 2) = v;
    };
    const __bf16* w1b = p.w1b + (int64_t)q * H * d;
    const __bf16* w2b = p.w2b + (int64_t)q * d * H;
    const __bf16* wl = p.w_lin + (int64_t)q * d * d;
    const float* b1 = p.b1 + (int64_t)q * H;
    const float* b2 = p.b2 + (int64_t)q * d;
    const int r = wt + l16, t = t0 + r;
    f32x4 acc[4], accv[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) accv[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int u0 = 0; u0 < H; u0 += kTN) {
        contract(w1b, d, u0, 0, kt, acc, true);                 // Z_u
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const int n = wn + a * 16 + g4 * 4;
            float v4[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float z = acc[a][v] + b1[u0 + n + v];
                v4[v] = gelu_q(z, normal_tail(fabsf(z)));
            }
            put(ht, r, n, u32x2{pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3])});
        }
        contract(w2b, H, 0, u0, ht, accv, false);              // V_hat += H_u W2_u^T
    }
    contract(wl, d, 0, 0, kt, accv, false);                     // V_hat += K W_lin^T
    float loss = 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int n = wn + a * 16 + g4 * 4;
        if (t < T) {
            const u32x2 vv = *reinterpret_cast<const u32x2*>(p.v + ((int64_t)l * T + t) * ldkv + h * d + n);
            const float vt[4] = {bf16_lo(vv[0]), bf16_hi(vv[0]), bf16_lo(vv[1]), bf16_hi(vv[1])};
            float g[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const float e = accv[a][v] + b2[n + v] - vt[v];
                loss = fmaf(e, e, loss);
                g[v] = e;
            }
            if (WRITE_E)
                *reinterpret_cast<u32x2*>(p.gb + ((int64_t)q * T + t) * d + n) =
                    u32x2{pack_bf16x2(g[0], g[1]), pack_bf16x2(g[2], g[3])};
        }
    }
    loss = wave_sum(loss);
    if (lane == 0) red_loss[w] = loss;
    __syncthreads();
    if (tid == 0) {
        float sum = 0.f;
        for (int i = 0; i < 8; ++i) sum += red_loss[i];
        p.loss_p[(int64_t)q * p.m_tiles + mt] = sum;
    }
}

// ------------------------------------------------------------ backward
// One workgroup per (problem, 128-unit hidden slice, token range), 64 tokens
// per iteration. Wave w takes hidden units u0 = 128 slice + 32 (w & 3) .. + 31
// and the 32-token half w >> 2 of each tile, and keeps its rows of the two
// weight-gradient sums, H^T E and dZ^T K (32 x 128 each, up to the factor
// 2 / T), in registers for the whole range. Resident in LDS: the slice's W1
// rows (B operand of Z) and W2^T rows (B operand of E W2). The keys and E of
// each tile arrive by direct global -> LDS copies into two alternating
// buffers, one tile ahead. Per tile:
//   Z  [tok][u] = K W1^T + b1           A = K rows (LDS)        16 MFMAs
//   dH [tok][u] = E W2                  A = E rows (LDS)        16 MFMAs
//   H = gelu(Z), dZ = dH gelu'(Z); lane (unit j, g4) holds tokens 4 g4 + i
//     and 16 + 4 g4 + i of its unit, the k-slots of one A fragment of the
//     token contractions below
//   (H^T E)[u][o] += ...                B = E^T by transposing LDS reads
//   (dZ^T K)[u][i] += ...               B = K^T likewise        32 MFMAs
//   sum_t E (slice 0; wave w sums d tiles 2 (w & 3), + 1) from E^T
//   fragments by bf16 dot products with ones, sum_t dZ from dZ, both in fp32.
// Tokens past T read as zeros: their E and dH vanish, so they add nothing.
// The two token halves write separate partials; the update sums them.
constexpr int kBwdTok = 64;
constexpr int kBwdRing = 2;
constexpr int kBwdTile = kBwdTok * 256;          // 16 KB: 64 rows of 128 bf16
constexpr int kBwdW = 128 * 256;                 // the slice's W1 or W2^T rows: 32 KB
static_assert(kBwdRing * 2 * kBwdTile + 2 * kBwdW <= kLdsAll, "backward LDS layout");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

// Transposing read of a B fragment over a 32-token slab: lane (j, g4) gets
// column c0 + j of slab rows 4 g4 + 0..3 (low half) and 16 + 4 g4 + 0..3
// (high half). Each 16-lane group's lane i names row 4 g4 + i / 4, columns
// c0 + 4 (i % 4) .. + 3 (8 bytes); rows are 256 bytes, swizzled as sw_off.
__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* slab, int c0, int l16, int g4) {
    const int rr = 4 * g4 + (l16 >> 2);
    const int byte = (c0 + 4 * (l16 & 3)) * 2;
    const uint32_t off = sw_off(rr, byte >> 4, 256) + (byte & 15);
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(slab + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(slab + off + 16 * 256));
    u32x4 v;
    v[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
    v[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
    v[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
    v[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
    return as_bf16x8(v);
}

__global__ __launch_bounds__(kFitThreads, 1) void fit_bwd_kernel(FitParams p) {
    // Separate objects, so the compiler's waits for the direct-to-LDS copies
    // into one tile buffer do not hold up reads of the other.
    __shared__ __attribute__((aligned(16))) unsigned char tile0[2 * kBwdTile];
    __shared__ __attribute__((aligned(16))) unsigned char tile1[2 * kBwdTile];
    __shared__ __attribute__((aligned(16))) unsigned char w1s[kBwdW];   // the slice's W1 rows [128][d]
    __shared__ __attribute__((aligned(16))) unsigned char w2s[kBwdW];   // the slice's W2^T rows [128][d]
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int hg = w & 3, th = w >> 2;
    const int H = p.hidden, T = p.ctx_len, d = kHeadDim;
    const int n_sl = H / 128;
    // blockIdx -> (problem, slice, range): XCD x = blockIdx % 8 takes
    // problems x, x + 8, ..., each problem's slices and ranges back to back,
    // so they share the keys and E of a tile in that XCD's L2.
    const int xcd = blockIdx.x & 7, j = blockIdx.x >> 3;
    const int per_q = n_sl * p.bwd_ranges;
    const int q = (j / per_q) * 8 + xcd, sr = j - (j / per_q) * per_q;
    if (q >= p.n_probs) return;
    const int sl = sr / p.bwd_ranges, rg = sr - sl * p.bwd_ranges;
    const int l = q / p.n_kv, hh = q - l * p.n_kv;
    const int ldkv = p.n_kv * d;
    const int u0 = sl * 128 + hg * 32;

    {
        const u32x4* s1 = reinterpret_cast<const u32x4*>(p.w1b + ((int64_t)q * H + sl * 128) * d);
        const u32x4* s2 = reinterpret_cast<const u32x4*>(p.w2tb + ((int64_t)q * H + sl * 128) * d);
        u32x4 v1[4], v2[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            v1[k] = s1[tid + k * kFitThreads];
            v2[k] = s2[tid + k * kFitThreads];
        }
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int i = tid + k * kFitThreads;
            *reinterpret_cast<u32x4*>(w1s + sw_off(i >> 4, i & 15, 256)) = v1[k];
            *reinterpret_cast<u32x4*>(w2s + sw_off(i >> 4, i & 15, 256)) = v2[k];
        }
    }
    const float bb0 = p.b1[(int64_t)q * H + u0 + l16], bb1 = p.b1[(int64_t)q * H + u0 + 16 + l16];

    const int n_all = (T + kBwdTok - 1) / kBwdTok;
    const int per = (n_all + p.bwd_ranges - 1) / p.bwd_ranges;
    const int ib = rg * per, n_it = max(0, min(n_all, ib + per) - ib);
    const __bf16* const kq = p.keys + (int64_t)l * T * ldkv + hh * d;
    const __bf16* const gq = p.gb + (int64_t)q * T * d;
    // Tile i's keys and E rows: wave w copies rows 8 w .. 8 w + 7 of each
    // (two copies of 4 rows; lane L fills row 4 c' + L / 16, slot L % 16 with
    // the piece that the swizzle puts there). Rows past T read as zeros.
    auto issue = [&](int i, unsigned char* const kt) {
        const int t0 = (ib + i) * kBwdTok;
        const int rows = max(0, T - t0);
        const __amdgpu_buffer_rsrc_t rk = buffer_rsrc(kq + (int64_t)t0 * ldkv, (uint32_t)(rows * ldkv * 2));
        const __amdgpu_buffer_rsrc_t rgt = buffer_rsrc(gq + (int64_t)t0 * d, (uint32_t)(rows * d * 2));
        // the lane's offsets are recomputed per tile (a few ALU operations)
        // rather than held in registers for the whole loop
        int ln = lane;
        asm volatile("" : "+v"(ln));
        const int crow = ln >> 4, cslot = ln & 15;
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int row = 8 * w + 4 * c + crow;
            const uint32_t pc = (uint32_t)((cslot ^ (row & 15)) << 4);
            dma16(rk, kt + (8 * w + 4 * c) * 256, (uint32_t)(row * ldkv * 2) + pc, 0u);
            dma16(rgt, kt + kBwdTile + (8 * w + 4 * c) * 256, (uint32_t)(row * 256) + pc, 0u);
        }
    };

    f32x4 dw1[2][8], dw2[2][8];
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) dw1[ht][dt] = dw2[ht][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    float db1a[2] = {0.f, 0.f}, db2a[2] = {0.f, 0.f};
    const bool db2_duty = sl == 0;

    // One tile per step: wait for its copies, the barrier, then the copies of
    // the next tile into the other buffer (whose tile every wave has finished).
    auto step = [&](auto slot_c, int it) {
        constexpr int SLOT = decltype(slot_c)::value;
        wait_vmcnt<0>();                              // this wave's copies of tile `it`
        barrier_lds();                                // and every wave's
        if (it + 1 < n_it) issue(it + 1, SLOT ? tile0 : tile1);
        const unsigned char* const ks = (SLOT ? tile1 : tile0) + th * 32 * 256;     // this wave's 32 rows
        const unsigned char* const gs = ks + kBwdTile;
        int zero = 0;                                 // keeps the weight reads inside the loop (as in the forward)
        asm volatile("" : "+v"(zero));

        f32x4 z[2][2], dh[2][2];                      // [tt][ht]
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            z[tt][0] = f32x4{bb0, bb0, bb0, bb0};
            z[tt][1] = f32x4{bb1, bb1, bb1, bb1};
            dh[tt][0] = dh[tt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            bf16x8 ka[2], ga[2], wb[2], wd[2];
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
                ka[tt] = lds16(ks, sw_off(16 * tt + l16, 4 * s + g4, 256));
                ga[tt] = lds16(gs, sw_off(16 * tt + l16, 4 * s + g4, 256));
            }
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                wb[ht] = lds16(w1s, sw_off(32 * hg + 16 * ht + l16, 4 * s + g4, 256) + zero);
                wd[ht] = lds16(w2s, sw_off(32 * hg + 16 * ht + l16, 4 * s + g4, 256) + zero);
            }
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int ht = 0; ht < 2; ++ht) {
                    z[tt][ht] = mfma(ka[tt], wb[ht], z[tt][ht]);
                    dh[tt][ht] = mfma(ga[tt], wd[ht], dh[tt][ht]);
                }
        }
        bf16x8 hp[2], dzp[2];
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) {
            f32x4 hv[2], dv[2];
            float sdz = 0.f;
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float hz, gz;
                    gelu_and_grad(z[tt][ht][i], hz, gz);
                    hv[tt][i] = hz;
                    dv[tt][i] = dh[tt][ht][i] * gz;
                    sdz += dv[tt][i];
                }
            db1a[ht] += sdz;
            hp[ht] = pack8(hv[0], hv[1]);
            dzp[ht] = pack8(dv[0], dv[1]);
        }
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            const bf16x8 gtr = tr_frag(gs, 16 * dt, l16, g4);
            const bf16x8 ktr = tr_frag(ks, 16 * dt, l16, g4);
#pragma unroll
            for (int ht = 0; ht < 2; ++ht) {
                dw2[ht][dt] = mfma(hp[ht], gtr, dw2[ht][dt]);
                dw1[ht][dt] = mfma(dzp[ht], ktr, dw1[ht][dt]);
            }
        }
        if (db2_duty) {
            // lane (column j, g4): its 8 tokens of columns 16 dt + j, dt = 2 (w & 3) + e,
            // summed in fp32 by bf16 dot products with ones
            typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
            const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const bf16x8 gtr = tr_frag(gs, 16 * (2 * hg + e), l16, g4);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    db2a[e] = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{gtr[2 * k], gtr[2 * k + 1]}, one2, db2a[e], false);
            }
        }
    };
    if (n_it > 0) issue(0, tile0);
    for (int it = 0; it < n_it; it += 2) {
        step(std::integral_constant<int, 0>{}, it);
        if (it + 1 < n_it) step(std::integral_constant<int, 1>{}, it + 1);
    }

    // partials of this (range, token half)
    const int64_t part = (int64_t)q * p.n_parts + rg * 2 + th;
    float* const o1 = p.pw1 + part * H * d;
    float* const o2 = p.pw2 + part * H * d;
#pragma unroll
    for (int ht = 0; ht < 2; ++ht)
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t e = (int64_t)(u0 + 16 * ht + 4 * g4 + i) * d + 16 * dt + l16;
                o1[e] = dw1[ht][dt][i];
                o2[e] = dw2[ht][dt][i];
            }
#pragma unroll
    for (int ht = 0; ht < 2; ++ht) {
        float x = db1a[ht];
        x += __shfl_xor(x, 16, kWave);
        x += __shfl_xor(x, 32, kWave);
        if (g4 == 0) p.pb1[part * H + u0 + 16 * ht + l16] = x;
    }
    if (db2_duty) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float x = db2a[e];
            x += __shfl_xor(x, 16, kWave);
            x += __shfl_xor(x, 32, kWave);
            if (g4 == 0) p.pb2[part * d + 16 * (2 * hg + e) + l16] = x;
        }
    }
}

// --------------------------------------------------------------- update
// Grid (problem, slice of kUpdSlices). mode 0: loss only (slot `step`, slice
// 0); mode 1: gradient step `step`: each weight's partials summed in a fixed
// order by the one thread that owns it, which updates the fp32 master and
// writes its bf16 copies; mode 2: bf16 copies only. W1, b1 and b2 are walked
// along the partials' contiguous axis; W2 ([o][u]) goes in tiles of 32 units
// x 128 outputs through LDS, so that its partials ([part][u][o]) and its
// transposed copy ([u][o]) are walked along o and W2 and its copy along u.
constexpr int kUpdSlices = 8;
constexpr int kUt = 32;                          // hidden units per W2 tile

__global__ __launch_bounds__(256) void fit_update_kernel(FitParams p, int step, int mode) {
    __shared__ float gt[kUt][kHeadDim + 1];      // a tile's W2 gradient, [u][o]
    __shared__ uint16_t nt[kUt][kHeadDim + 2];   // its bf16 values, [u][o]
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
        for (int m = 0; m < p.n_loss_parts; ++m) s += (double)p.loss_p[(int64_t)q * p.n_loss_parts + m];
        p.losses[(int64_t)q * (p.n_steps + 1) + step] = (float)(s / (double)p.ctx_len);
    }
    if (mode == 0) return;
    const float lr = p.lr * (2.0f / (float)p.ctx_len);   // the sums are over E = (T / 2) G
    const int np = p.n_parts;
    if (mode == 1) {
        const float* pw1 = p.pw1 + (int64_t)q * np * H * d;   // [part][u][i]
        for (int e = e0; e < H * d; e += es) {
            float g1 = 0.f;
            for (int c = 0; c < np; ++c) g1 += pw1[(int64_t)c * H * d + e];
            const float x1 = w1[e] - lr * g1;         // w1[u][i], e = u d + i
            w1[e] = x1;
            w1b[e] = f32_to_bf16_bits(x1);
        }
        for (int u = e0; u < H; u += es) {
            float g = 0.f;
            for (int c = 0; c < np; ++c) g += p.pb1[((int64_t)q * np + c) * H + u];
            b1[u] -= lr * g;
        }
        for (int o = e0; o < d; o += es) {
            float g = 0.f;
            for (int c = 0; c < np; ++c) g += p.pb2[((int64_t)q * np + c) * d + o];
            b2[o] -= lr * g;
        }
    } else {
        for (int e = e0; e < H * d; e += es) w1b[e] = f32_to_bf16_bits(w1[e]);
    }
    const float* pw2 = p.pw2 + (int64_t)q * np * H * d;       // [part][u][o]
    constexpr int kPer = kUt * kHeadDim / 256;                 // tile elements per thread
    for (int u0 = slice * kUt; u0 < H; u0 += kUt * kUpdSlices) {
        if (mode == 1) {
#pragma unroll 4
            for (int k = 0; k < kPer; ++k) {
                const int idx = tid + 256 * k, ul = idx / kHeadDim, o = idx % kHeadDim;
                float g2 = 0.f;
                for (int c = 0; c < np; ++c) g2 += pw2[(int64_t)c * H * d + (int64_t)(u0 + ul) * d + o];
                gt[ul][o] = g2;
            }
            __syncthreads();
        }
#pragma unroll 4
        for (int k = 0; k < kPer; ++k) {
            const int idx = tid + 256 * k, o = idx / kUt, ul = idx % kUt;
            const int64_t wi = (int64_t)o * H + u0 + ul;          // w2[o][u]
            float x2 = w2[wi];
            if (mode == 1) {
                x2 = x2 - lr * gt[ul][o];
                w2[wi] = x2;
            }
            const uint16_t v = f32_to_bf16_bits(x2);
            w2b[wi] = v;
            nt[ul][o] = v;
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < kPer; ++k) {
            const int idx = tid + 256 * k, ul = idx / kHeadDim, o = idx % kHeadDim;
            w2tb[(int64_t)(u0 + ul) * d + o] = nt[ul][o];         // w2tb[u][o]
        }
        __syncthreads();
    }
}

hipError_t launch_fit(const FitParams& p, void* ev_begin, void* ev_end, hipStream_t s) {
    const unsigned P = (unsigned)p.n_probs;
    const bool resident = p.hidden <= kFwdMaxHidden, wide = p.hidden > 128;
    const dim3 gf(P * (unsigned)p.fwd_ranges);
    const int per_xcd = (int)(((P + 7) / 8) * (unsigned)p.m_tiles);
    const dim3 gt((unsigned)per_xcd * 8u);
    const dim3 gb(((P + 7) / 8) * 8u * (unsigned)(p.hidden / 128 * p.bwd_ranges));
    hipError_t e;
    hipLaunchKernelGGL(fit_update_kernel, dim3(P, kUpdSlices), dim3(256), 0, s, p, 0, 2);
    if (ev_begin && (e = hipEventRecord(static_cast<hipEvent_t>(ev_begin), s)) != hipSuccess) return e;
    for (int it = 0; it < p.n_steps; ++it) {
        if (resident && wide) hipLaunchKernelGGL((fit_fwd_kernel<true, 8>), gf, dim3(kFitThreads), 0, s, p);
        else if (resident) hipLaunchKernelGGL((fit_fwd_kernel<true, 4>), gf, dim3(kFitThreads), 0, s, p);
        else hipLaunchKernelGGL((fit_fwd_tiled_kernel<true>), gt, dim3(kFitThreads), 0, s, p, per_xcd);
        hipLaunchKernelGGL(fit_bwd_kernel, gb, dim3(kFitThreads), 0, s, p);
        hipLaunchKernelGGL(fit_update_kernel, dim3(P, kUpdSlices), dim3(256), 0, s, p, it, 1);
    }
    if (ev_end && (e = hipEventRecord(static_cast<hipEvent_t>(ev_end), s)) != hipSuccess) return e;
    if (p.losses) {     // the loss after the last step: a forward pass that only sums squared errors
        if (resident && wide) hipLaunchKernelGGL((fit_fwd_kernel<false, 8>), gf, dim3(kFitThreads), 0, s, p);
        else if (resident) hipLaunchKernelGGL((fit_fwd_kernel<false, 4>), gf, dim3(kFitThreads), 0, s, p);
        else hipLaunchKernelGGL((fit_fwd_tiled_kernel<false>), gt, dim3(kFitThreads), 0, s, p, per_xcd);
        hipLaunchKernelGGL(fit_update_kernel, dim3(P, kUpdSlices), dim3(256), 0, s, p, p.n_steps, 0);
    }
    return hipGetLastError();
}

}  // namespace lowram
