// Fused prefill value prediction and residual ranking for gfx950.
//
// The values the predictor would give every cached token are computed in the
// kernel from the cache's own parameters, so ranking reads the true values V
// and never a stored V_hat:
//   K     = A_group . B_l^T                      (keys of layer l, per head)
//   V_hat = K W_lin^T + gelu(K W1^T + b1) W2^T + b2
//   e_t   = sum_i (V[t, i] - V_hat[t, i])^2     (binary64, index order)
// Pass 1 (MODE 0) does this for every token and writes e (and, on request, a
// float32 copy of V_hat). The select and compact kernels of the ranking then
// pick the k worst tokens per (layer, head). Pass 2 (MODE 1) recomputes V_hat
// for the chosen tokens only, with the same instructions in the same order,
// so the values are bit-identical to pass 1, and stores R = V - V_hat.
//
// Work split: one wave per 64 tokens, four waves of one KV head per
// workgroup; B_l chunks and predictor weights go to LDS once per workgroup by
// direct global -> LDS copies. All products are v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation:
//   K^T[n][t]      A = B_l rows (LDS),   B = A rows (LDS, per wave)
//   V_hat^T[o][t]  A = W_lin rows,       B = K (bf16, k-slots = 8 features)
//   Z^T[j][t]      A = W1 rows,          B = K
//   V_hat^T[o][t] += A = W2 rows,        B = gelu(Z) (bf16, k-slots = 8 hidden)
// The D layout of one product is the B layout of the next when both operands
// agree on the k-slot order. The accumulator tiles hold rows 4g..4g+3 and
// 16+4g..16+4g+3 of each 32-row group in one lane, so the B_l rows and the W1
// rows are copied to LDS in the permuted order perm(r) below: the lane's
// eight k-slots are then eight consecutive features (or hidden units), and
// every weight fragment is one plain 16-byte piece of a weight row.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"
#include "mfma_util.hpp"

#pragma clang fp contract(off)

namespace lowram {

namespace {

constexpr int kPw = 4;                       // waves (64-token tiles) per workgroup
constexpr int kPThreads = kPw * kWave;
constexpr int kPKc = 64;                     // rank columns per B_l / A chunk
constexpr int kPRow = kPKc * 2;              // bytes of one row of a rank chunk
constexpr int kBuf = 16384;                  // bytes of one LDS buffer
constexpr int kXcds = 8;
constexpr int kPMaxHidden = 4096;           // the largest hidden width the prefill takes
constexpr uint32_t kOob = 0x80000000u;       // buffer offset past every valid range: reads zero

// LDS row r of a 32-row group holds row perm(r) of the source: accumulator
// rows 4g+i and 16+4g+i (i < 4) of a lane become consecutive features 8g+i
// and 8g+4+i.
__device__ __forceinline__ int perm32(int r) {
    const int m = r & 31;
    return (r & ~31) + 8 * ((m & 15) >> 2) + 4 * (m >> 4) + (m & 3);
}

}  // namespace

template <int MODE, int RDT>
__global__ __launch_bounds__(kPThreads, 1) void prefill_mfma_kernel(PrefillParams p, int n_grp_pad) {
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;
    const int R = p.rank, H = p.hidden, T = p.ctx_len;

    // ---- workgroup -> (layer, head, token group)
    int l, h, grp;
    if (MODE == 0) {       // the heads of one token group on one XCD: they read the same A rows
        const int per_l = n_grp_pad * p.n_kv;
        l = blockIdx.x / per_l;
        const int rem = blockIdx.x % per_l;
        const int xcd = rem % kXcds, slot = rem / kXcds;
        h = slot % p.n_kv;
        grp = (slot / p.n_kv) * kXcds + xcd;
    } else {
        l = blockIdx.x / (n_grp_pad * p.n_kv);
        const int rem = blockIdx.x % (n_grp_pad * p.n_kv);
        h = rem / n_grp_pad;
        grp = rem % n_grp_pad;
    }
    if (grp >= p.n_groups) return;
    const int64_t lh = (int64_t)l * p.n_kv + h;

    // ---- this wave's 64 tokens: row r -> token, or -1
    int my_tok;                                      // token of row `lane`
    if (MODE == 0) {
        const int t = (grp * kPw + w) * kBlock + lane;
        my_tok = t < T ? t : -1;
    } else {
        const int s = (grp * kPw + w) * kBlock + lane;
        my_tok = s < p.n_res ? p.res_idx[lh * p.n_res + s] : -1;
        my_tok = (my_tok >= 0 && my_tok < T) ? my_tok : -1;
    }

    __shared__ __attribute__((aligned(16))) unsigned char buf0[kBuf], buf1[kBuf], buf2[kBuf], buf3[kBuf];
    // The head's biases as float (zero when absent), for the predictor steps.
    __shared__ __attribute__((aligned(16))) float sb1[kPMaxHidden], sb2[kHeadDim];
    // This wave's 64 rows of V (256-byte rows; 16-byte piece p of row r at
    // slot p ^ (r & 15)), copied after the keys so they land during the
    // predictor steps. 128 KB of LDS in all: one workgroup per CU.
    __shared__ __attribute__((aligned(16))) unsigned char sv[kPw * kBlock * 256];

    // The biases are loaded now, with no branch and no arithmetic on them until
    // they are staged after the key loop (a missing bias reads the W_lin row
    // instead and is dropped): loaded where the predictor steps use them, each
    // load made the compiler wait for it, and for the next step's copies in
    // flight, on the spot.
    const bool has_b1 = p.b1 != nullptr, has_b2 = p.b2 != nullptr;
    const uint16_t* const b1src = has_b1 ? static_cast<const uint16_t*>(p.b1) + lh * H : static_cast<const uint16_t*>(p.w_lin);
    const uint16_t* const b2src = has_b2 ? static_cast<const uint16_t*>(p.b2) + lh * kHeadDim : static_cast<const uint16_t*>(p.w_lin);
    uint16_t b1raw[kPMaxHidden / kPThreads];
#pragma unroll
    for (int k = 0; k < kPMaxHidden / kPThreads; ++k) b1raw[k] = b1src[has_b1 ? min(tid + kPThreads * k, H - 1) : 0];
    const uint16_t b2raw = b2src[has_b2 ? (tid & (kHeadDim - 1)) : 0];

    // ---- 1. K^T = B_l(head)^T . A^T over the rank, 64 columns per chunk
    const __amdgpu_buffer_rsrc_t ra = buffer_rsrc(
        static_cast<const unsigned char*>(p.a) + (int64_t)(l / p.group) * T * R * 2, (uint32_t)((int64_t)T * R * 2));
    const __amdgpu_buffer_rsrc_t rb = buffer_rsrc(
        static_cast<const unsigned char*>(p.b_l) + lh * kHeadDim * (int64_t)R * 2, (uint32_t)(kHeadDim * R * 2));
    const int n_chunks = R / kPKc;
    const int dma_row = lane >> 3;
    const uint32_t piece = (uint32_t)(((lane & 7) ^ dma_row) * 16);   // slot lane%8 of an 8-row group
    uint32_t a_off[8];             // instruction q copies A rows 8q .. 8q+7 of this wave
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int t = __shfl(my_tok, q * 8 + dma_row, kWave);
        a_off[q] = (t >= 0 ? (uint32_t)t * (uint32_t)R * 2u : kOob) + piece;
    }
    uint32_t bl_off[4];            // instruction q copies LDS rows 32w + 8q .. +7 of the B_l chunk
#pragma unroll
    for (int q = 0; q < 4; ++q) bl_off[q] = (uint32_t)(perm32(w * 32 + q * 8 + dma_row) * R * 2) + piece;
    unsigned char* const sa_w = ((w >> 1) ? buf3 : buf2) + (w & 1) * (kBlock * kPRow);
    // Copies past the last chunk go to a resource of size zero: they read
    // zeros and touch no memory, so every chunk issues the same copies.
    const __amdgpu_buffer_rsrc_t rnone = buffer_rsrc(p.b_l, 0u);
    auto dma_bl = [&](int c, unsigned char* dst) {
        const __amdgpu_buffer_rsrc_t r = c < n_chunks ? rb : rnone;
#pragma unroll
        for (int q = 0; q < 4; ++q) dma16(r, dst + (w * 32 + q * 8) * kPRow, bl_off[q], (uint32_t)(c * kPRow));
    };
    auto dma_a = [&](int c) {
        const __amdgpu_buffer_rsrc_t r = c < n_chunks ? ra : rnone;
#pragma unroll
        for (int q = 0; q < 8; ++q) dma16(r, sa_w + q * 8 * kPRow, a_off[q], (uint32_t)(c * kPRow));
    };
    const int xs = g4 ^ (l16 & 7);
    const uint32_t rd_off[2] = {(uint32_t)(l16 * kPRow + xs * 16), (uint32_t)(l16 * kPRow + (xs ^ 4) * 16)};

    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[i][tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    // MFMA steps s0 .. s1-1 of one rank chunk (B_l tile st % 8, k-step st / 8),
    // each B_l fragment read two steps ahead; the first two are read by the caller.
    auto mma_part = [&](const unsigned char* sb, const bf16x8 (&a8)[2][4], bf16x8 (&bq)[3], auto s0c, auto s1c) {
        constexpr int s0 = decltype(s0c)::value, s1 = decltype(s1c)::value;
        auto rd = [&](int st) { return lds16(sb, rd_off[st >> 3] + (st & 7) * 16 * kPRow); };
#pragma unroll
        for (int st = s0; st < s1; ++st) {
            if (st + 2 < 16) bq[(st + 2) % 3] = rd(st + 2);
            const int kk = st >> 3, nt_ = st & 7;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[nt_][tt] = mfma(bq[st % 3], a8[kk][tt], acc[nt_][tt]);
        }
        if (s0 == 0) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int st = s0; st < s1; ++st) {
            if (st + 2 < 16) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
    };
    dma_bl(0, buf0);
    dma_a(0);
    wait_vmcnt<8>();
    barrier_lds();
    auto chunk = [&](int c, const unsigned char* cur, unsigned char* nxt) {
        bf16x8 a8[2][4];
        wait_vmcnt<0>();   // this wave's copy of the chunk's A rows (the only copy in flight)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) a8[kk][tt] = lds16(sa_w, rd_off[kk] + tt * 16 * kPRow);
        // The next chunk's B_l copy starts now (the other buffer); its A copy,
        // into the region just read, four MFMA steps in, once the A reads are
        // done (LDS reads complete in order: with two B_l reads issued since,
        // they are).
        dma_bl(c + 1, nxt);
        __builtin_amdgcn_sched_barrier(0);
        bf16x8 bq[3];
        bq[0] = lds16(cur, rd_off[0]);
        bq[1] = lds16(cur, rd_off[0] + 16 * kPRow);
        mma_part(cur, a8, bq, std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
        __builtin_amdgcn_sched_barrier(0);
        wait_lgkmcnt<2>();
        dma_a(c + 1);
        __builtin_amdgcn_sched_barrier(0);
        mma_part(cur, a8, bq, std::integral_constant<int, 4>{}, std::integral_constant<int, 16>{});
        wait_vmcnt<8>();
        barrier_lds();
    };
    for (int c = 0; c < n_chunks; c += 2) {
        chunk(c, buf0, buf1);
        if (c + 1 < n_chunks) chunk(c + 1, buf1, buf0);
    }
    wait_vmcnt<0>();

    // Stage the biases (the first predictor step's barrier publishes them).
#pragma unroll
    for (int k = 0; k < kPMaxHidden / kPThreads; ++k) {
        const int e = tid + kPThreads * k;
        if (e < H) sb1[e] = has_b1 ? __uint_as_float((uint32_t)b1raw[k] << 16) : 0.f;
    }
    if (tid < kHeadDim) sb2[tid] = has_b2 ? __uint_as_float((uint32_t)b2raw << 16) : 0.f;

    // K as the B operand: kf[tt][s] holds features 32s + 8g + (0..7) of token 16tt + l16.
    bf16x8 kf[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[tt][s] = pack8(acc[2 * s][tt], acc[2 * s + 1][tt]);

    // ---- 2. predictor weights through LDS, two 16 KB chunks per step:
    //   step 0: W_lin rows 0..63 and 64..127 (256-byte rows of 128 inputs)
    //   step j (1..H/64): W1 rows 64(j-1) + perm(0..63) (256-byte rows) and
    //           W2[:, 64(j-1) .. 64j) (128-byte rows of 64 hidden units)
    // Even steps use buffers 0/1, odd steps 2/3; the next step's copies run
    // during this step's products.
    const int n_steps = 1 + H / 64;
    const unsigned char* wl = static_cast<const unsigned char*>(p.w_lin) + lh * kHeadDim * kHeadDim * 2;
    const unsigned char* w1 = static_cast<const unsigned char*>(p.w1) + lh * (int64_t)H * kHeadDim * 2;
    const unsigned char* w2 = static_cast<const unsigned char*>(p.w2) + lh * (int64_t)kHeadDim * H * 2;
    auto dma_step = [&](int j, unsigned char* d0, unsigned char* d1) {
        // 256-byte rows: instruction q of wave w fills rows 16w + 4q .. +3,
        // lane i row 16w + 4q + i/16 at slot i%16, which holds piece slot ^ (row & 15).
        const int r256 = lane >> 4;
        if (j == 0) {
            const __amdgpu_buffer_rsrc_t rw = buffer_rsrc(wl, kHeadDim * kHeadDim * 2);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = w * 16 + q * 4 + r256;                 // 0..63
                const uint32_t pc = (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
                dma16(rw, d0 + (w * 16 + q * 4) * 256, (uint32_t)(row * 256) + pc, 0u);
                dma16(rw, d1 + (w * 16 + q * 4) * 256, (uint32_t)((row + 64) * 256) + pc, 0u);
            }
        } else {
            const int hc = j - 1;
            const __amdgpu_buffer_rsrc_t r1 = buffer_rsrc(w1, (uint32_t)(H * kHeadDim * 2));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = w * 16 + q * 4 + r256;                 // LDS row 0..63
                const uint32_t pc = (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
                dma16(r1, d0 + (w * 16 + q * 4) * 256, (uint32_t)((hc * 64 + perm32(row)) * 256) + pc, 0u);
            }
            // 128-byte rows: instruction q of wave w fills rows 32w + 8q .. +7,
            // lane i row 32w + 8q + i/8 at slot i%8, which holds piece slot ^ (row & 7).
            const __amdgpu_buffer_rsrc_t r2 = buffer_rsrc(w2, (uint32_t)(kHeadDim * H * 2));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int row = w * 32 + q * 8 + dma_row;              // output feature 0..127
                dma16(r2, d1 + (w * 32 + q * 8) * 128, (uint32_t)(row * H * 2 + hc * 128) + piece, 0u);
            }
        }
    };

    // V_hat^T accumulators: vacc[ot][tt] holds outputs 16ot + 4g + (0..3) of
    // token 16tt + l16; step 0 starts them at b2.
    f32x4 vacc[8][4];

    // One step: wait for its copies, compute from (s0, s1), then, once every
    // wave is done with them, start the copies of step j + 2 into them.
    auto step = [&](int j, unsigned char* s0, unsigned char* s1) {
        if (j + 1 < n_steps) wait_vmcnt<8>(); else wait_vmcnt<0>();   // this step's 8 copies per wave
        barrier_lds();
        if (j == 0) {
#pragma unroll
            for (int ot = 0; ot < 8; ++ot) {
                const unsigned char* src = ot < 4 ? s0 : s1;
                const int row = (ot & 3) * 16 + l16;
                bf16x8 wf[4];
#pragma unroll
                for (int s = 0; s < 4; ++s) wf[s] = lds16(src, (uint32_t)(row * 256 + (((4 * s + g4) ^ (row & 15)) * 16)));
                const f32x4 bb = *reinterpret_cast<const f32x4*>(sb2 + ot * 16 + 4 * g4);
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    vacc[ot][tt] = bb;
#pragma unroll
                    for (int s = 0; s < 4; ++s) vacc[ot][tt] = mfma(wf[s], kf[tt][s], vacc[ot][tt]);
                }
            }
        } else {
            const int hc = j - 1;
            f32x4 zb[4];             // hidden bias of LDS rows 16ht + 4g + (0..3): four consecutive units
#pragma unroll
            for (int ht = 0; ht < 4; ++ht) zb[ht] = *reinterpret_cast<const f32x4*>(sb1 + hc * 64 + perm32(ht * 16 + 4 * g4));
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f32x4 z[4];
#pragma unroll
                for (int ht = 0; ht < 4; ++ht) {
                    const int row = ht * 16 + l16;
                    z[ht] = zb[ht];
#pragma unroll
                    for (int s = 0; s < 4; ++s)
                        z[ht] = mfma(lds16(s0, (uint32_t)(row * 256 + (((4 * s + g4) ^ (row & 15)) * 16))), kf[tt][s], z[ht]);
                }
                gelu_tail16(z);
                const bf16x8 gb[2] = {pack8(z[0], z[1]), pack8(z[2], z[3])};
#pragma unroll
                for (int ot = 0; ot < 8; ++ot) {
                    const int row = ot * 16 + l16;
#pragma unroll
                    for (int s = 0; s < 2; ++s)
                        vacc[ot][tt] = mfma(lds16(s1, (uint32_t)(row * 128 + (((4 * s + g4) ^ (row & 7)) * 16))), gb[s], vacc[ot][tt]);
                }
            }
        }
        barrier_lds();                      // every wave is done with this step's buffers
        if (j + 2 < n_steps) dma_step(j + 2, s0, s1);
    };
    const int64_t vrow_stride = (int64_t)p.n_kv * kHeadDim;     // elements between tokens of V
    const __bf16* vl = static_cast<const __bf16*>(p.v) + ((int64_t)l * T * p.n_kv + h) * kHeadDim;
    unsigned char* const sv_w = sv + w * (kBlock * 256);
    {
        // Instruction q fills rows 4q .. 4q+3: lane i row 4q + i/16, slot i%16,
        // fetching piece (i%16) ^ (row & 15); rows without a token read zeros.
        const __amdgpu_buffer_rsrc_t rv = buffer_rsrc(vl, (uint32_t)((int64_t)T * vrow_stride * 2));
#pragma unroll
        for (int q = 0; q < 16; ++q) {
            const int row = 4 * q + (lane >> 4);
            const int t = __shfl(my_tok, row, kWave);
            const uint32_t pc = (uint32_t)(((lane & 15) ^ (row & 15)) * 16);
            dma16<kNonTemporal>(rv, sv_w + q * 1024, t >= 0 ? (uint32_t)((int64_t)t * vrow_stride * 2) + pc : kOob, 0u);
        }
    }
    // The V copies are older than the first step's: its wait covers them too.
    dma_step(0, buf0, buf1);
    if (n_steps > 1) dma_step(1, buf2, buf3);
    for (int j = 0; j < n_steps; j += 2) {  // static buffers: even steps in buf0/buf1
        step(j, buf0, buf1);
        if (j + 1 < n_steps) step(j + 1, buf2, buf3);
    }

    // ---- 3. per token: error (pass 1) or residual (pass 2)
    // V elements 16 ot + 4 g4 .. + 3 of row r: bytes 32 ot + 8 g4 of the row,
    // piece 2 ot + g4 / 2 at its swizzled slot.
    auto v4 = [&](int r, int ot) {
        const int pc = 2 * ot + (g4 >> 1);
        return *reinterpret_cast<const u32x2*>(sv_w + r * 256 + ((pc ^ (r & 15)) << 4) + 8 * (g4 & 1));
    };
    if (MODE == 0) {
        // d^2 in binary64, in four 32-feature chunks: every lane forms the
        // squares of its 32 values of the chunk into this wave's 16 KB LDS
        // tile [64 tokens][32] (16-byte pair cp of row r at slot cp ^ (r & 15),
        // so a 16-lane group's row reads hit distinct banks); then lane r adds
        // token r's 32 terms in index order, its sum running across the
        // chunks. All 64 lanes carry a token's chain at once.
        unsigned char* const et = w == 0 ? buf0 : (w == 1 ? buf1 : (w == 2 ? buf2 : buf3));
        if (p.v_hat != nullptr) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int t = __shfl(my_tok, tt * 16 + l16, kWave);
                if (t >= 0) {
#pragma unroll
                    for (int ot = 0; ot < 8; ++ot) {
                        float* vh = p.v_hat + (((int64_t)l * T + t) * p.n_kv + h) * kHeadDim + ot * 16 + 4 * g4;
                        *reinterpret_cast<f32x4*>(vh) = vacc[ot][tt];
                    }
                }
            }
        }
        double e = 0.0;
#pragma unroll
        for (int fc = 0; fc < 4; ++fc) {
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                const int r = tt * 16 + l16;
#pragma unroll
                for (int oo = 0; oo < 2; ++oo) {
                    const int ot = 2 * fc + oo;
                    const u32x2 vv = v4(r, ot);
                    double d2[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const uint32_t word = vv[i >> 1];
                        const float vf = __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
                        const double dl = (double)vf - (double)vacc[ot][tt][i];
                        d2[i] = dl * dl;
                    }
                    const int cp = 8 * oo + 2 * g4;      // pairs of columns 16 oo + 4 g4 .. + 3
                    *reinterpret_cast<double2*>(et + r * 256 + ((cp ^ (r & 15)) << 4)) = double2{d2[0], d2[1]};
                    *reinterpret_cast<double2*>(et + r * 256 + (((cp + 1) ^ (r & 15)) << 4)) = double2{d2[2], d2[3]};
                }
            }
            wait_lgkmcnt0();                          // the wave's LDS operations complete in order
#pragma unroll
            for (int cp = 0; cp < 16; ++cp) {
                const double2 pr = *reinterpret_cast<const double2*>(et + lane * 256 + ((cp ^ (lane & 15)) << 4));
                e = e + pr.x;
                e = e + pr.y;
            }
            wait_lgkmcnt0();                          // before the next chunk overwrites the tile
        }
        if (my_tok >= 0) p.err[lh * T + my_tok] = e;
    } else {
        // R = V - V_hat in binary64, encoded like the ranking's gather.
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int row = tt * 16 + l16;
            const int t = __shfl(my_tok, row, kWave);
            const int s = (grp * kPw + w) * kBlock + row;              // slot in the residual store
            double rr[8][4];
#pragma unroll
            for (int ot = 0; ot < 8; ++ot) {
                const u32x2 vv = v4(row, ot);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const uint32_t word = vv[i >> 1];
                    const float vf = __uint_as_float((i & 1) ? (word & 0xffff0000u) : (word << 16));
                    rr[ot][i] = (double)vf - (double)vacc[ot][tt][i];
                }
            }
            const int64_t o = (lh * p.n_res + s) * kHeadDim + 4 * g4;
            if (RDT == DT_I2) {
                // Symmetric mid-rise 4-level code; the lane's four features
                // 16 ot + 4 g4 .. + 3 are exactly byte 4 ot + g4 of the row.
                double amax = 0.0;
#pragma unroll
                for (int ot = 0; ot < 8; ++ot)
#pragma unroll
                    for (int i = 0; i < 4; ++i) amax = fmax(amax, fabs(rr[ot][i]));
                amax = fmax(amax, __shfl_xor(amax, 16, kWave));
                amax = fmax(amax, __shfl_xor(amax, 32, kWave));
                const float sc = static_cast<float>(amax / 1.5);
                const double s64 = static_cast<double>(sc);
                if (t >= 0) {
                    uint8_t* const dst = static_cast<uint8_t*>(p.res_val) + (lh * p.n_res + s) * (kHeadDim / 4) + g4;
#pragma unroll
                    for (int ot = 0; ot < 8; ++ot) {
                        uint32_t byte = 0u;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            double q = 2.0;
                            if (s64 > 0.0) {
                                q = rint(rr[ot][i] / s64 + 1.5);
                                q = q > 3.0 ? 3.0 : (q < 0.0 ? 0.0 : q);
                            }
                            byte |= (uint32_t)q << (2 * i);
                        }
                        dst[ot * 4] = (uint8_t)byte;
                    }
                    if (g4 == 0) p.res_scale[lh * p.n_res + s] = sc;
                }
            } else if (RDT == DT_I8) {
                double amax = 0.0;
#pragma unroll
                for (int ot = 0; ot < 8; ++ot)
#pragma unroll
                    for (int i = 0; i < 4; ++i) amax = fmax(amax, fabs(rr[ot][i]));
                amax = fmax(amax, __shfl_xor(amax, 16, kWave));
                amax = fmax(amax, __shfl_xor(amax, 32, kWave));
                const float sc = static_cast<float>(amax / 127.0);
                const double s64 = static_cast<double>(sc);
                if (t >= 0) {
#pragma unroll
                    for (int ot = 0; ot < 8; ++ot) {
                        uint32_t word = 0u;
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            int8_t cq = 0;
                            if (s64 > 0.0) {
                                double q = rint(rr[ot][i] / s64);
                                q = q > 127.0 ? 127.0 : (q < -127.0 ? -127.0 : q);
                                cq = static_cast<int8_t>(q);
                            }
                            word |= (uint32_t)(uint8_t)cq << (8 * i);
                        }
                        *reinterpret_cast<uint32_t*>(static_cast<int8_t*>(p.res_val) + o + ot * 16) = word;
                    }
                    if (g4 == 0) p.res_scale[lh * p.n_res + s] = sc;
                }
            } else if (t >= 0) {
#pragma unroll
                for (int ot = 0; ot < 8; ++ot) {
                    if (RDT == DT_F32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(p.res_val) + o + ot * 16) =
                            f32x4{(float)rr[ot][0], (float)rr[ot][1], (float)rr[ot][2], (float)rr[ot][3]};
                    } else {
                        const uint32_t w0 = (uint32_t)f64_to_bf16_bits(rr[ot][0]) | ((uint32_t)f64_to_bf16_bits(rr[ot][1]) << 16);
                        const uint32_t w1v = (uint32_t)f64_to_bf16_bits(rr[ot][2]) | ((uint32_t)f64_to_bf16_bits(rr[ot][3]) << 16);
                        *reinterpret_cast<u32x2*>(static_cast<uint16_t*>(p.res_val) + o + ot * 16) = u32x2{w0, w1v};
                    }
                }
            }
        }
    }
}

int prefill_groups(const PrefillParams& p, int mode) {
    return mode == 0 ? (p.n_blocks + kPw - 1) / kPw : (p.n_res + kPw * kBlock - 1) / (kPw * kBlock);
}

hipError_t launch_prefill(const PrefillParams& p, int mode, hipStream_t s) {
    const int n_grp = p.n_groups;
    if (n_grp <= 0) return hipSuccess;
    const int pad = mode == 0 ? (n_grp + kXcds - 1) / kXcds * kXcds : n_grp;
    const dim3 grid((unsigned)((int64_t)p.n_slices * p.n_kv * pad));
    if (mode == 0) {
        hipLaunchKernelGGL((prefill_mfma_kernel<0, DT_F32>), grid, dim3(kPThreads), 0, s, p, pad);
    } else if (p.res_dtype == DT_F32) {
        hipLaunchKernelGGL((prefill_mfma_kernel<1, DT_F32>), grid, dim3(kPThreads), 0, s, p, pad);
    } else if (p.res_dtype == DT_BF16) {
        hipLaunchKernelGGL((prefill_mfma_kernel<1, DT_BF16>), grid, dim3(kPThreads), 0, s, p, pad);
    } else if (p.res_dtype == DT_I8) {
        hipLaunchKernelGGL((prefill_mfma_kernel<1, DT_I8>), grid, dim3(kPThreads), 0, s, p, pad);
    } else {
        hipLaunchKernelGGL((prefill_mfma_kernel<1, DT_I2>), grid, dim3(kPThreads), 0, s, p, pad);
    }
    return hipGetLastError();
}

}  // namespace lowram
