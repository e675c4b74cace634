// Cross-layer key factors for the prefill side.
//
// project site, Figure 3 (K ~ A . B: a factor shared by a group of adjacent
// layers and a smaller factor per layer) and the explainer's keys paragraph
// (xKV: one low-rank basis for adjacent layers, because key energy sits in few
// directions). The group's keys C = [K_1 | ... | K_G] (T x n, n = G D) are
// reduced to an orthonormal rank-r basis X (n x r) of their row space by
// randomized subspace iteration on the Gram matrix (Halko, Martinsson and
// Tropp, "Finding structure with randomness", SIAM Review 2011, Algorithm
// 4.4): M = C^T C, X_0 = Omega, X_i = orth(M X_{i-1}); then A = C X and
// B_l = (rows l D .. l D + D - 1 of X)^T, so K_l ~ A B_l.
//
//   xkv_gram_kernel        bf16 MFMA: partial 256 x 256 Gram tiles per token chunk
//   xkv_gram_reduce_kernel fp64 sum of the chunk partials into symmetric M
//   xkv_gemm_f64_kernel    fp64 products of the iteration (M X, Y^T Y)
//   xkv_chol_panel_kernel  Cholesky of the r x r Gram, one 64-column panel (one workgroup)
//   xkv_chol_update_kernel the trailing update after a panel (many workgroups)
//   xkv_trsm_kernel        X = Y L^-T, rows in parallel (CholeskyQR)
//   xkv_emit_kernel        bf16 B_l and the transposed basis
//   xkv_a_kernel           bf16 MFMA: A = C X
#include <hip/hip_runtime.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_util.hpp"

namespace lowram {

constexpr int kXT = 256;                 // tile edge of the MFMA kernels
constexpr int kXK = 64;                  // contraction step
constexpr int kXThreads = 512;           // 8 waves
constexpr int kXRowB = kXK * 2;          // LDS row: 64 bf16 along the contraction
constexpr int kXStage = kXT * kXRowB;    // one operand of one step: 32 KB
constexpr int kXMaxRank = 1024;

// LDS rows of 128 bytes hold eight 16-byte pieces; piece p of row r sits in
// slot p ^ (r & 7), so the MFMA reads (16 rows, one piece) hit distinct banks.
__device__ __forceinline__ uint32_t xslot(int row, int piece) {
    return (uint32_t)(row * kXRowB + ((piece ^ (row & 7)) << 4));
}

// One 64-wide contraction step of the wave's 64 x 128 block of a 256 x 256
// tile: operand rows [256][64 k] in swizzled LDS. acc[mt][nt] holds
// D[m][n] = sum_k op0[wi + 16 mt + m][k] op1[wj + 16 nt + n][k].
__device__ __forceinline__ void xkv_mma_step(const unsigned char* op0, const unsigned char* op1,
                                             f32x4 (&acc)[4][8], int wi, int wj, int lane) {
    const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
        bf16x8 af[4], bf[8];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) af[mt] = lds16(op0, xslot(wi + mt * 16 + l16, ks * 4 + g4));
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) bf[nt] = lds16(op1, xslot(wj + nt * 16 + l16, ks * 4 + g4));
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
            for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = mfma(af[mt], bf[nt], acc[mt][nt]);
    }
}

// Upper-triangle tile index -> (I, J), I <= J, row by row.
__device__ __forceinline__ void xkv_tile(int k, int nt, int& ti, int& tj) {
    int i = 0;
    while (k >= nt - i) {
        k -= nt - i;
        ++i;
    }
    ti = i;
    tj = i + k;
}

// k-th upper tile (I <= J) when the tiles are walked 4 x 4 blocks at a time
// (block rows in order, block columns from the diagonal on, row-major inside).
__device__ __forceinline__ void xkv_tile_blocked(int k, int nt, int& ti, int& tj) {
    const int nb = (nt + 3) / 4;
    for (int bi = 0; bi < nb; ++bi)
        for (int bj = bi; bj < nb; ++bj)
            for (int i = 4 * bi; i < min(nt, 4 * bi + 4); ++i)
                for (int j = max(i, 4 * bj); j < min(nt, 4 * bj + 4); ++j) {
                    if (k == 0) {
                        ti = i;
                        tj = j;
                        return;
                    }
                    --k;
                }
    ti = tj = 0;
}

// ---------------------------------------------------------------- Gram
// Block (b, problem): token chunk b / n_upper, tile b % n_upper (chunk-major,
// so the workgroups resident together share one chunk of C). The stored
// partial is the transposed tile: P[a][b] = sum_t C[t][256 I + b] C[t][256 J + a]
// = M[256 J + a][256 I + b].
//
// Four waves, one per SIMD, each owning a 128 x 128 quarter of the tile (256
// accumulator registers). The keys come into LDS untransposed, by direct
// copies four 32-token steps ahead in a ring of five stages (the whole 160 KB
// of LDS): per stage and operand 32 token rows x 256 columns (512-byte rows of
// 32 pieces of 16 bytes, piece p of row t in slot p ^ gsw(t)). The MFMA fragments are read
// with the transposing LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lanes 4r .. 4r+3 name row r's 16 consecutive columns and lane j gets
// column j of those 4 rows, i.e. 4 consecutive tokens of one column; two such
// reads make the 8 tokens of a fragment.
constexpr int kGramThreads = 256;
constexpr int kGK = 32;                          // tokens per step
constexpr int kGRowB = kXT * 2;                  // 512-byte rows
constexpr int kGOp = kGK * kGRowB;               // 16 KB per operand per stage
constexpr int kGStage = 2 * kGOp;                // both operands

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;

// Row t's slot swizzle: twice a 4-bit value from bits 0-1 and 3-4 of t, so the
// 16 rows (8 g + v, g, v < 4) that one transposing read touches hit 16
// distinct 32-byte column pairs, two per bank set.
__device__ __forceinline__ int gsw(int t) { return 2 * ((t & 3) | (((t >> 3) & 3) << 2)); }

__device__ __forceinline__ bf16x8 tr_frag(const unsigned char* op, uint32_t off) {
    const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(op + off));
    const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(op + off + 4 * kGRowB));
    // Concatenated as they are: any repacking would be vector instructions
    // that wait on both reads.
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8, v);
}

// 64 MFMAs of one 32-token step of the wave's 128 x 128 block.
__device__ __forceinline__ void gram_step(const unsigned char* stage, f32x4 (&acc)[8][8], int wi, int wj,
                                          uint32_t lane_off, int lane_sw) {
    const unsigned char* op0 = stage;
    const unsigned char* op1 = stage + kGOp;
    auto off = [&](int m0) { return lane_off + ((uint32_t)(((m0 >> 3) ^ lane_sw)) << 4); };
    bf16x8 af[8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) af[mt] = tr_frag(op0, off(wi + mt * 16));
#pragma unroll
    for (int nh = 0; nh < 2; ++nh) {
        bf16x8 bf[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bf[nt] = tr_frag(op1, off(wj + (nh * 4 + nt) * 16));
#pragma unroll
        for (int mt = 0; mt < 8; ++mt)
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) acc[mt][nh * 4 + nt] = mfma(af[mt], bf[nt], acc[mt][nh * 4 + nt]);
    }
}

__global__ __launch_bounds__(kGramThreads, 1) void xkv_gram_kernel(XkvParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char st0[kGStage];
    __shared__ __attribute__((aligned(16))) unsigned char st1[kGStage];
    __shared__ __attribute__((aligned(16))) unsigned char st2[kGStage];
    __shared__ __attribute__((aligned(16))) unsigned char st3[kGStage];
    __shared__ __attribute__((aligned(16))) unsigned char st4[kGStage];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    // Blocks go round-robin over the 8 XCDs; XCD x takes the contiguous run
    // of positions x * per .. x * per + per - 1, in an order that walks the
    // upper tiles 4 x 4 blocks at a time, so the workgroups resident on one
    // XCD share few column slices in its L2.
    const int total = p.n_chunks * p.n_upper, per = (total + 7) / 8;
    const int pos = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (pos >= total) return;
    const int chunk = pos / p.n_upper;
    int ti, tj;
    xkv_tile_blocked(pos - chunk * p.n_upper, p.nt, ti, tj);
    const int tile = ti * p.nt - ti * (ti - 1) / 2 + (tj - ti);     // row-major upper index
    const int t_begin = chunk * p.chunk_len;
    const int t_end = min(p.ctx_len, t_begin + p.chunk_len);
    const int n_steps = (t_end - t_begin + kGK - 1) / kGK;
    const int64_t prob = blockIdx.y;

    // Operand slices as buffers over this chunk's tokens (zeros past t_end).
    auto slice = [&](int tcol) {
        const int col0 = tcol * kXT, layer = col0 / p.width;
        const __bf16* base = p.keys + (prob * p.n_layers + layer) * p.ctx_len * (int64_t)p.width +
                             (int64_t)t_begin * p.width + (col0 - layer * p.width);
        return buffer_rsrc(base, (uint32_t)((int64_t)(t_end - t_begin) * p.width * 2));
    };
    const __amdgpu_buffer_rsrc_t r0 = slice(ti), r1 = slice(tj);
    // Copies: wave w fills rows 8 w .. 8 w + 7 of both operands, 2 rows per
    // instruction; lane i lands in row 8 w + 2 q + i / 32, slot i % 32, and
    // fetches the piece that belongs there.
    const uint32_t row_b = (uint32_t)(p.width * 2);
    uint32_t voff[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int row = w * 8 + q * 2 + (lane >> 5);
        const int piece = (lane & 31) ^ gsw(row);
        voff[q] = (uint32_t)row * row_b + (uint32_t)piece * 16;
    }
    auto dma = [&](int s, unsigned char* stage) {
        const uint32_t soff = (uint32_t)s * kGK * row_b;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            dma16(r0, stage + (w * 8 + q * 2) * kGRowB, voff[q], soff);
            dma16(r1, stage + kGOp + (w * 8 + q * 2) * kGRowB, voff[q], soff);
        }
    };
    // Transposing-read address of this lane (fragment rows m0 added per read).
    const int g = lane >> 4, i16 = lane & 15;
    const int trow = 8 * g + (i16 >> 2);
    const int lane_sw = gsw(trow) | ((i16 & 3) >> 1);
    const uint32_t lane_off = (uint32_t)(trow * kGRowB + ((i16 & 1) << 3));

    f32x4 acc[8][8];
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wi = (w >> 1) * 128, wj = (w & 1) * 128;

    dma(0, st0);
    if (n_steps > 1) dma(1, st1);
    if (n_steps > 2) dma(2, st2);
    if (n_steps > 3) dma(3, st3);
    // Step s: wait for this wave's copies of s (those of s+1 .. s+3 may stay
    // in flight, 8 per step), meet, start s+4 into the stage s-1 used, multiply.
    auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
        if (s + 3 < n_steps) wait_vmcnt<24>();
        else if (s + 2 < n_steps) wait_vmcnt<16>();
        else if (s + 1 < n_steps) wait_vmcnt<8>();
        else wait_vmcnt<0>();
        barrier_lds();
        if (s + 4 < n_steps) dma(s + 4, nxt);
        gram_step(cur, acc, wi, wj, lane_off, lane_sw);
    };
    for (int s = 0; s < n_steps; s += 5) {
        step(s, st0, st4);
        if (s + 1 < n_steps) step(s + 1, st1, st0);
        if (s + 2 < n_steps) step(s + 2, st2, st1);
        if (s + 3 < n_steps) step(s + 3, st3, st2);
        if (s + 4 < n_steps) step(s + 4, st4, st3);
    }
    float* out = p.partials + ((prob * p.n_chunks + chunk) * p.n_upper + tile) * (kXT * kXT);
    const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt)
            *reinterpret_cast<f32x4*>(out + (wj + nt * 16 + l16) * kXT + wi + mt * 16 + g4 * 4) = acc[mt][nt];
}

// M[256 J + a][256 I + b] = sum over chunks of P (binary64, chunk order),
// mirrored off the diagonal. Grid (16 groups of 16 rows a, n_upper tiles,
// problems), 256 threads (b).
constexpr int kRedRows = 16;                    // tile rows per reduction block

__global__ __launch_bounds__(256) void xkv_gram_reduce_kernel(XkvParams p) {
    // Block: rows a0 .. a0+15 of one upper tile, thread b its column. The
    // sums go to M directly (coalesced along b) and, for an off-diagonal tile,
    // to the mirrored block through LDS, so that each thread then writes 16
    // consecutive doubles of one mirrored row.
    __shared__ double sub[kRedRows][kXT + 1];
    const int tile = blockIdx.y, a0 = blockIdx.x * kRedRows, b = threadIdx.x;
    const int64_t prob = blockIdx.z;
    int ti, tj;
    xkv_tile(tile, p.nt, ti, tj);
    const float* src = p.partials + (prob * p.n_chunks * p.n_upper + tile) * (kXT * kXT) + a0 * kXT + b;
    double* const m = p.m + prob * p.n * (int64_t)p.n;
    const int64_t chunk_stride = (int64_t)p.n_upper * (kXT * kXT);
#pragma unroll 4
    for (int r = 0; r < kRedRows; ++r) {
        double v = 0.0;
        for (int c = 0; c < p.n_chunks; ++c) v += (double)src[c * chunk_stride + r * kXT];
        m[((int64_t)tj * kXT + a0 + r) * p.n + (int64_t)ti * kXT + b] = v;
        sub[r][b] = v;
    }
    if (ti == tj) return;                          // the whole block takes this branch
    __syncthreads();
    double* const dst = m + ((int64_t)ti * kXT + b) * p.n + (int64_t)tj * kXT + a0;
#pragma unroll
    for (int r = 0; r < kRedRows; ++r) dst[r] = sub[r][b];
}

// ------------------------------------------------------- fp64 products
// Per problem q = z / splits and split z % splits: C_q (+ split * c_split)
// = op(A_q) op(B_q) over k in [split kc, min(k, split kc + kc)), with
// X_q = X + q sX, op(A)(i, kk) = TA ? A[kk lda + i] : A[i lda + kk] and
// op(B)(kk, j) = TB ? B[j ldb + kk] : B[kk ldb + j].
//
// fp64 MFMA (v_mfma_f64_16x16x4_f64): 128 x 128 tiles, 16 deep, four waves
// of 64 x 64 (4 x 4 blocks of 16 x 16). LDS holds op(A) as [k][i] and op(B)
// as [k][j], rows padded to 144 doubles so that the operand reads (16
// consecutive i or j, four k rows per wave) and the staging writes hit
// distinct banks; two stages, the next tile's loads held in registers while
// the current one is multiplied.
struct GemmArgs {
    int m, n, k, kc, splits;
    const double* A; int64_t lda, sA;
    const double* B; int64_t ldb, sB;
    double* C; int64_t ldc, sC, c_split;
};
typedef double f64x4 __attribute__((ext_vector_type(4)));
constexpr int kGm = 128, kGk = 16, kGld = 144;

template <bool T>
__device__ __forceinline__ void gemm_load(const double* X, int64_t ld, int rows, int k0, int ke, int r0, int tid,
                                          double (&v)[8]) {
    // The 128 x 16 tile of op(X) (rows r0.., k k0..): T means X is stored
    // [k][row] (rows contiguous), else [row][k]. Thread tid fetches four
    // 2-element pieces.
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;
        int row, kk;
        if (T) { row = (e & 63) * 2; kk = e >> 6; }        // 2 consecutive rows at one k
        else { row = e & 127; kk = (e >> 7) * 2; }         // 2 consecutive k at one row
        const int gr = r0 + row, gk = k0 + kk;
        if (T) {
            v[2 * u] = (gr < rows && gk < ke) ? X[(int64_t)gk * ld + gr] : 0.0;
            v[2 * u + 1] = (gr + 1 < rows && gk < ke) ? X[(int64_t)gk * ld + gr + 1] : 0.0;
        } else {
            v[2 * u] = (gr < rows && gk < ke) ? X[(int64_t)gr * ld + gk] : 0.0;
            v[2 * u + 1] = (gr < rows && gk + 1 < ke) ? X[(int64_t)gr * ld + gk + 1] : 0.0;
        }
    }
}

template <bool T>
__device__ __forceinline__ void gemm_store(double* s, int tid, const double (&v)[8]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
        const int e = tid + 256 * u;
        if (T) {
            const int row = (e & 63) * 2, kk = e >> 6;
            s[kk * kGld + row] = v[2 * u];
            s[kk * kGld + row + 1] = v[2 * u + 1];
        } else {
            const int row = e & 127, kk = (e >> 7) * 2;
            s[kk * kGld + row] = v[2 * u];
            s[(kk + 1) * kGld + row] = v[2 * u + 1];
        }
    }
}

template <bool TA, bool TB>
__global__ __launch_bounds__(256, 2) void xkv_gemm_f64_kernel(GemmArgs g) {
    __shared__ double as[2][kGk * kGld], bs[2][kGk * kGld];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int i0 = blockIdx.y * kGm, j0 = blockIdx.x * kGm;
    const int q = blockIdx.z / g.splits, split = blockIdx.z - q * g.splits;
    const double* const A = g.A + q * g.sA;
    const double* const B = g.B + q * g.sB;
    const int kb = split * g.kc, ke = min(g.k, kb + g.kc);
    const int wm = (w >> 1) * 64, wn = (w & 1) * 64;
    const int l16 = lane & 15, kl = lane >> 4;
    f64x4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = f64x4{0.0, 0.0, 0.0, 0.0};
    double va[8], vb[8];
    // op(A)(i, k): stored [k][i] when TA; op(B)(k, j): stored [k][j] unless TB.
    gemm_load<TA>(A, g.lda, g.m, kb, ke, i0, tid, va);
    gemm_load<!TB>(B, g.ldb, g.n, kb, ke, j0, tid, vb);
    gemm_store<TA>(as[0], tid, va);
    gemm_store<!TB>(bs[0], tid, vb);
    __syncthreads();
    int buf = 0;
    for (int k0 = kb; k0 < ke; k0 += kGk) {
        const bool more = k0 + kGk < ke;
        if (more) {
            gemm_load<TA>(A, g.lda, g.m, k0 + kGk, ke, i0, tid, va);
            gemm_load<!TB>(B, g.ldb, g.n, k0 + kGk, ke, j0, tid, vb);
        }
        const double* sa = as[buf];
        const double* sb = bs[buf];
#pragma unroll
        for (int ks = 0; ks < kGk / 4; ++ks) {
            double fa[4], fb[4];
#pragma unroll
            for (int a = 0; a < 4; ++a) fa[a] = sa[(ks * 4 + kl) * kGld + wm + a * 16 + l16];
#pragma unroll
            for (int b = 0; b < 4; ++b) fb[b] = sb[(ks * 4 + kl) * kGld + wn + b * 16 + l16];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) acc[a][b] = __builtin_amdgcn_mfma_f64_16x16x4f64(fa[a], fb[b], acc[a][b], 0, 0, 0);
        }
        if (more) {
            gemm_store<TA>(as[buf ^ 1], tid, va);
            gemm_store<!TB>(bs[buf ^ 1], tid, vb);
        }
        __syncthreads();
        buf ^= 1;
    }
    // D block (a, b) of the fp64 MFMA: value v of a lane is row lane / 16 + 4 v,
    // column lane % 16 (rows interleaved, unlike the fp32 variants).
    double* out = g.C + q * g.sC + split * g.c_split;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int j = j0 + wn + b * 16 + l16;
            if (j >= g.n) continue;
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = i0 + wm + a * 16 + kl + 4 * v;
                if (i < g.m) out[(int64_t)i * g.ldc + j] = acc[a][b][v];
            }
        }
}

// out_q[i] = sum over s of parts_q[s count + i], in split order (grid y: problem q).
__global__ __launch_bounds__(256) void xkv_sum_splits_kernel(const double* parts, double* out, int64_t count, int splits) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= count) return;
    const int64_t q = blockIdx.y;
    double v = 0.0;
    for (int s = 0; s < splits; ++s) v += parts[(q * splits + s) * count + i];
    out[q * count + i] = v;
}

// ---------------------------------------------------------- CholeskyQR
constexpr int kCholPw = 16;

// In-place lower Cholesky factor of the r x r Gram g (row-major; the strict
// upper triangle is left as it was), blocked by 64-column panels: for panel
// j0 one workgroup per problem factors columns j0 .. j0+63 (16-column steps
// in LDS, each step's update kept inside the panel), then
// xkv_chol_update_kernel subtracts L21 L21^T from the trailing lower
// triangle on many workgroups. A pivot at or below r * 2^-52 * max diag (of
// the Gram as given) marks the column dead: its L column is zero and the
// solve gives that basis column zero (the block is rank deficient there).
constexpr int kCholNb = 64;                 // columns per panel; the rank is a multiple of it

__global__ __launch_bounds__(1024) void xkv_chol_panel_kernel(double* g, int r, int32_t* dead, double* taus, int j0) {
    __shared__ double pan[kXMaxRank * kCholPw];
    __shared__ double red[16], pivs[kCholPw], invs[kCholPw];
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    g += (int64_t)blockIdx.x * r * r;
    dead += (int64_t)blockIdx.x * r;
    double tau;
    if (j0 == 0) {                          // the threshold comes from the diagonal before any update
        double dm = 0.0;
        for (int i = tid; i < r; i += 1024) dm = fmax(dm, g[(int64_t)i * r + i]);
        for (int off = 32; off > 0; off >>= 1) dm = fmax(dm, __shfl_xor(dm, off, kWave));
        if (lane == 0) red[w] = dm;
        __syncthreads();
        dm = red[0];
        for (int i = 1; i < 16; ++i) dm = fmax(dm, red[i]);
        tau = (double)r * 0x1p-52 * dm;
        if (tid == 0) taus[blockIdx.x] = tau;
    } else {
        tau = taus[blockIdx.x];
    }
    const int jend = j0 + kCholNb;          // r is a multiple of kCholNb

    for (int c0 = j0; c0 < jend; c0 += kCholPw) {
        const int rows = r - c0;
        // Eight loads per thread in flight before any LDS store (a load and
        // its store per iteration made each iteration a memory round trip);
        // entries past the panel read its last one and are not stored.
        const int n_pan = rows * kCholPw;
        for (int e0 = tid; e0 < n_pan; e0 += 1024 * 8) {
            double v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = min(e0 + 1024 * k, n_pan - 1);
                v[k] = g[(int64_t)(c0 + e / kCholPw) * r + c0 + e % kCholPw];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k)
                if (e0 + 1024 * k < n_pan) pan[e0 + 1024 * k] = v[k];
        }
        __syncthreads();
        // Column c stays unscaled until the end of the 16 steps: every thread
        // forms the two scaled factors of its update itself (the same rounded
        // products a scaled column would hold), so a step needs one barrier.
        for (int c = 0; c < kCholPw; ++c) {
            const double d = pan[c * kCholPw + c];
            const bool dd = !(d > tau);
            const double piv = dd ? 0.0 : sqrt(d);
            const double inv = dd ? 0.0 : 1.0 / piv;
            if (tid == 0) {
                dead[c0 + c] = dd ? 1 : 0;
                pivs[c] = piv;
                invs[c] = inv;
            }
            const int nc = kCholPw - 1 - c;
            for (int e = tid; e < (rows - c - 1) * nc; e += 1024) {
                const int i = c + 1 + e / nc, cc = c + 1 + e % nc;
                if (cc <= i) pan[i * kCholPw + cc] -= (pan[i * kCholPw + c] * inv) * (pan[cc * kCholPw + c] * inv);
            }
            __syncthreads();
        }
        for (int e = tid; e < rows * kCholPw; e += 1024) {
            const int i = e / kCholPw, c = e % kCholPw;
            if (c <= i) {
                const double v = i == c ? pivs[c] : pan[e] * invs[c];
                pan[e] = v;
                g[(int64_t)(c0 + i) * r + c0 + c] = v;
            }
        }
        __syncthreads();
        // The rest of this panel: columns c0+16 .. jend-1, every row below,
        // in 4 x 4 blocks (block column bk, block row bi >= bk).
        const int nbi = (rows - kCholPw) / 4, nbk = (jend - c0 - kCholPw) / 4;
        for (int e = tid; e < nbi * nbk; e += 1024) {
            const int bi = e / nbk, bk = e % nbk;
            if (bk > bi) continue;
            const int i0 = kCholPw + bi * 4, k0 = kCholPw + bk * 4;
            // The block's 16 entries of G (all inside the matrix, the upper
            // ones too) are loaded before the products and written back under
            // the triangle test: a load under that test made each entry a
            // memory round trip of its own.
            double gv[4][4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) gv[a][b] = g[(int64_t)(c0 + i0 + a) * r + c0 + k0 + b];
            double sacc[4][4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b) sacc[a][b] = 0.0;
#pragma unroll 4
            for (int c = 0; c < kCholPw; ++c) {
                double li[4], lk[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    li[q] = pan[(i0 + q) * kCholPw + c];
                    lk[q] = pan[(k0 + q) * kCholPw + c];
                }
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int b = 0; b < 4; ++b) sacc[a][b] = fma(li[a], lk[b], sacc[a][b]);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    if (k0 + b <= i0 + a) g[(int64_t)(c0 + i0 + a) * r + c0 + k0 + b] = gv[a][b] - sacc[a][b];
        }
        __syncthreads();
    }
}

// Trailing update after panel j0: G[i][k] -= sum_c L[i][c] L[k][c] over the
// panel's columns c, for i >= k >= j0 + 64. One workgroup per 64 x 64 tile
// of the lower block triangle (grid x: tile, grid y: problem); each thread a
// 4 x 4 block, the tile's two row sets of L staged in LDS.
__global__ __launch_bounds__(256) void xkv_chol_update_kernel(double* g, int r, int j0) {
    __shared__ double li[kCholNb][kCholNb + 1], lk[kCholNb][kCholNb + 1];
    const int tid = threadIdx.x;
    g += (int64_t)blockIdx.y * r * r;
    const int base = j0 + kCholNb;
    // tile index -> (ti, tk), tk <= ti
    const int e = blockIdx.x;
    int ti = (int)((sqrt(8.0 * (double)e + 1.0) - 1.0) * 0.5);
    while (ti * (ti + 1) / 2 > e) --ti;
    while ((ti + 1) * (ti + 2) / 2 <= e) ++ti;
    const int tk = e - ti * (ti + 1) / 2;
    const int r0 = base + ti * kCholNb, k0 = base + tk * kCholNb;      // both < r: r - base is a multiple of 64
    // All 32 loads of a thread in flight before its LDS stores.
    static_assert(kCholNb * kCholNb % 256 == 0, "whole tiles per thread");
    double vi[kCholNb * kCholNb / 256], vk[kCholNb * kCholNb / 256];
#pragma unroll
    for (int q = 0; q < kCholNb * kCholNb / 256; ++q) {
        const int x = tid + 256 * q, row = x / kCholNb, c = x % kCholNb;
        vi[q] = g[(int64_t)(r0 + row) * r + j0 + c];
        vk[q] = g[(int64_t)(k0 + row) * r + j0 + c];
    }
#pragma unroll
    for (int q = 0; q < kCholNb * kCholNb / 256; ++q) {
        const int x = tid + 256 * q, row = x / kCholNb, c = x % kCholNb;
        li[row][c] = vi[q];
        lk[row][c] = vk[q];
    }
    __syncthreads();
    const int a0 = (tid >> 4) * 4, b0 = (tid & 15) * 4;
    // This thread's 16 entries of G, loaded before the products (all inside
    // the matrix; the triangle test applies to the write-back only).
    double gv[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) gv[a][b] = g[(int64_t)(r0 + a0 + a) * r + k0 + b0 + b];
    double sacc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) sacc[a][b] = 0.0;
#pragma unroll 4
    for (int c = 0; c < kCholNb; ++c) {
        double x[4], y[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            x[q] = li[a0 + q][c];
            y[q] = lk[b0 + q][c];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int b = 0; b < 4; ++b) sacc[a][b] = fma(x[a], y[b], sacc[a][b]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const int i = r0 + a0 + a, k = k0 + b0 + b;
            if (k <= i) g[(int64_t)i * r + k] = gv[a][b] - sacc[a][b];
        }
}

// Blocked Cholesky of n_prob r x r Grams (r a multiple of 64); taus holds
// n_prob doubles of scratch.
static void launch_chol(double* g, int r, int32_t* dead, double* taus, int n_prob, hipStream_t s) {
    for (int j0 = 0; j0 < r; j0 += kCholNb) {
        hipLaunchKernelGGL(xkv_chol_panel_kernel, dim3((unsigned)n_prob), dim3(1024), 0, s, g, r, dead, taus, j0);
        const int nt = (r - j0 - kCholNb) / kCholNb;
        if (nt > 0)
            hipLaunchKernelGGL(xkv_chol_update_kernel, dim3((unsigned)(nt * (nt + 1) / 2), (unsigned)n_prob), dim3(256), 0,
                               s, g, r, j0);
    }
}

// X = Y L^-T for 16 rows per workgroup: x_j = (y_j - sum_{k<j} L[j][k] x_k) / L[j][j],
// x_j = 0 for a dead column. Lanes 16 q .. 16 q + 15 of a wave share one row.
// Y = I (r rows) when y is null, which gives L^-T itself. Grid y: problem.
constexpr int kTrRows = 16;
__global__ __launch_bounds__(256) void xkv_trsm_kernel(const double* y, double* x, const double* l, const int32_t* dead,
                                                       int nrows, int r) {
    __shared__ double xs[kTrRows][kXMaxRank];
    const int tid = threadIdx.x, lane = tid & 63, row = tid >> 4, c = tid & 15;
    const int r0 = blockIdx.x * kTrRows;
    const int64_t q = blockIdx.y;
    l += q * r * r;
    dead += q * r;
    x += q * nrows * r;
    if (y) y += q * nrows * r;
    const int n_x = kTrRows * r;
    if (y) {
        // Eight loads per thread in flight before its LDS stores; rows past
        // the end read the last row and store zero.
        for (int e0 = tid; e0 < n_x; e0 += 256 * 8) {
            double v[8];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = min(e0 + 256 * k, n_x - 1), i = e / r, j = e % r;
                v[k] = y[(int64_t)min(r0 + i, nrows - 1) * r + j];
            }
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int e = e0 + 256 * k;
                if (e < n_x) xs[e / r][e % r] = r0 + e / r >= nrows ? 0.0 : v[k];
            }
        }
    } else {
        for (int e = tid; e < n_x; e += 256) {
            const int i = e / r, j = e % r;
            xs[i][j] = r0 + i < nrows && r0 + i == j ? 1.0 : 0.0;
        }
    }
    __syncthreads();
    for (int jb = 0; jb < r; jb += 16) {
        const int j = jb + c;
        const double* lj = l + (int64_t)j * r;
        double s0 = 0.0, s1 = 0.0;
        for (int k = 0; k < jb; k += 2) {
            s0 = fma(xs[row][k], lj[k], s0);
            s1 = fma(xs[row][k + 1], lj[k + 1], s1);
        }
        double v = xs[row][j] - (s0 + s1);
        const double ljj = lj[j];
        const bool dj = dead[j] != 0;
        // L[j][jb .. jb+15] in registers before the sweep, so no step of it
        // waits for memory.
        double lb[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const double2 t = *reinterpret_cast<const double2*>(lj + jb + 2 * i);
            lb[2 * i] = t.x;
            lb[2 * i + 1] = t.y;
        }
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) {
            double xv = (dj || !(ljj != 0.0)) ? 0.0 : v / ljj;
            xv = __shfl(xv, (lane & ~15) | cc, kWave);
            if (c > cc) v = fma(-lb[cc], xv, v);
            if (c == cc) xs[row][j] = xv;
        }
    }
    __syncthreads();
    for (int e = tid; e < kTrRows * r; e += 256) {
        const int i = e / r, j = e % r;
        if (r0 + i < nrows) x[(int64_t)(r0 + i) * r + j] = xs[i][j];
    }
}

// ------------------------------------------------------------- outputs
// b_l = bf16(X) in X's own [n, r] layout, xt = bf16(X)^T [r, n], basis = X
// (grid z: problem).
__global__ __launch_bounds__(256) void xkv_emit_kernel(XkvParams p, const double* xb) {
    __shared__ uint16_t tl[64][64 + 2];
    const int i0 = blockIdx.y * 64, c0 = blockIdx.x * 64;
    const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
    const int64_t off = (int64_t)blockIdx.z * p.n * p.rank;
    for (int q = ty; q < 64; q += 4) {
        const int64_t e = off + (int64_t)(i0 + q) * p.rank + c0 + tx;
        const double v = xb[e];
        const uint16_t h = f64_to_bf16_bits(v);
        reinterpret_cast<uint16_t*>(p.b_l)[e] = h;
        if (p.basis) p.basis[e] = v;
        tl[q][tx] = h;
    }
    __syncthreads();
    for (int q = ty; q < 64; q += 4)
        reinterpret_cast<uint16_t*>(p.xt)[off + (int64_t)(c0 + q) * p.n + i0 + tx] = tl[tx][q];
}

// A = C X as A^T tiles: operand 0 = rows c of xt (256 per tile, zeros past
// r), operand 1 = token rows of C (zeros past T), contraction over n in
// steps of 64 inside one layer. Both come in by direct copies into two static
// stage buffers. Lane (l16, g4) holds A[t][c .. c+3] for 4 consecutive c.
__global__ __launch_bounds__(kXThreads, 1) void xkv_a_kernel(XkvParams p) {
    __shared__ __attribute__((aligned(16))) unsigned char st0[2 * kXStage];
    __shared__ __attribute__((aligned(16))) unsigned char st1[2 * kXStage];
    const int tid = threadIdx.x, lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n_ct = (p.rank + kXT - 1) / kXT;
    // Blocks go round-robin over the 8 XCDs. XCD x takes token tiles x, x + 8,
    // x + 16, ..., each with all its column tiles in consecutive positions, so
    // the workgroups that read one token tile's keys share them in one L2.
    // The grid is padded to a multiple of 8 token tiles; padding blocks exit.
    const int n_tt = (p.ctx_len + kXT - 1) / kXT;
    const int pos = blockIdx.x >> 3;
    const int ct = pos % n_ct, tt = (pos / n_ct) * 8 + (blockIdx.x & 7);
    if (tt >= n_tt) return;
    const int c0 = ct * kXT, t0 = tt * kXT;
    const int n_steps = p.n / kXK;
    const int64_t prob = blockIdx.y;
    const __bf16* const keys = p.keys + prob * p.n_layers * p.ctx_len * (int64_t)p.width;
    const __bf16* const xt = p.xt + prob * p.rank * (int64_t)p.n;
    __bf16* const a_out = p.a + prob * p.ctx_len * (int64_t)p.rank;

    // Waves 0-3 copy operand 0, waves 4-7 operand 1; each wave 64 rows, eight
    // 1 KB copies (8 rows x 8 pieces, lane i -> row i / 8, slot i % 8).
    const int op = w >> 2;
    const int dma_row = lane >> 3;
    const uint32_t dma_piece = (uint32_t)(((lane & 7) ^ dma_row) * 16);
    const int rbase = (w & 3) * 64;
    const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(xt, (uint32_t)((int64_t)p.rank * p.n * 2));
    auto dma = [&](int s, unsigned char* buf) {
        const int k0 = s * kXK;
        if (op == 0) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = c0 + rbase + q * 8 + dma_row;
                dma16(rx, buf + (rbase + q * 8) * kXRowB, (uint32_t)(((int64_t)row * p.n + k0) * 2) + dma_piece, 0u);
            }
        } else {
            const int layer = k0 / p.width;
            const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(keys + (int64_t)layer * p.ctx_len * p.width,
                                                          (uint32_t)((int64_t)p.ctx_len * p.width * 2));
            const int kcol = k0 - layer * p.width;
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int row = t0 + rbase + q * 8 + dma_row;
                dma16(rc, buf + kXStage + (rbase + q * 8) * kXRowB,
                      (uint32_t)(((int64_t)row * p.width + kcol) * 2) + dma_piece, 0u);
            }
        }
    };

    f32x4 acc[4][8];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 8; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int wi = (w >> 1) * 64, wj = (w & 1) * 128;
    dma(0, st0);
    auto step = [&](int s, const unsigned char* cur, unsigned char* nxt) {
        wait_vmcnt<0>();
        barrier_lds();      // every wave's copies of step s landed; step s-1's reads are done
        if (s + 1 < n_steps) dma(s + 1, nxt);
        xkv_mma_step(cur, cur + kXStage, acc, wi, wj, lane);
    };
    for (int s = 0; s < n_steps; s += 2) {
        step(s, st0, st1);
        if (s + 1 < n_steps) step(s + 1, st1, st0);
    }
    wait_vmcnt<0>();
    const int l16 = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int nt = 0; nt < 8; ++nt) {
        const int t = t0 + wj + nt * 16 + l16;
        if (t >= p.ctx_len) continue;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int c = c0 + wi + mt * 16 + g4 * 4;
            if (c >= p.rank) continue;
            const f32x4 v = acc[mt][nt];
            const uint32_t w0 = (uint32_t)f32_to_bf16_bits(v[0]) | ((uint32_t)f32_to_bf16_bits(v[1]) << 16);
            const uint32_t w1 = (uint32_t)f32_to_bf16_bits(v[2]) | ((uint32_t)f32_to_bf16_bits(v[3]) << 16);
            *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a_out) + (int64_t)t * p.rank + c) = u32x2{w0, w1};
        }
    }
}

// -------------------------------------------------------------- launchers
size_t xkv_partials_floats(const XkvParams& p) { return (size_t)p.n_chunks * p.n_upper * kXT * kXT; }

hipError_t launch_xkv_gram(const XkvParams& p, hipStream_t s) {
    const unsigned per = (unsigned)((p.n_chunks * p.n_upper + 7) / 8);
    hipLaunchKernelGGL(xkv_gram_kernel, dim3(8 * per, (unsigned)p.n_batch), dim3(kGramThreads), 0, s, p);
    return hipGetLastError();
}

// out = in (rows x r) times the r x r matrix w, per problem (in's problem
// stride 0 for the shared starting block).
// `symmetric` says in == in^T (the Gram matrix), which is then read in its
// transposed, coalesced form.
static void gemm_nn(const XkvParams& p, int rows, int k, const double* in, int64_t s_in, int64_t ld_in,
                    const double* w, int64_t s_w, double* out, bool symmetric, hipStream_t s) {
    GemmArgs g{};
    g.m = rows; g.n = p.rank; g.k = k; g.kc = k; g.splits = 1;
    g.A = in; g.lda = ld_in; g.sA = s_in;
    g.B = w; g.ldb = p.rank; g.sB = s_w;
    g.C = out; g.ldc = p.rank; g.sC = (int64_t)rows * p.rank; g.c_split = 0;
    const dim3 grid((unsigned)((p.rank + kGm - 1) / kGm), (unsigned)((rows + kGm - 1) / kGm), (unsigned)p.n_batch);
    if (symmetric)
        hipLaunchKernelGGL((xkv_gemm_f64_kernel<true, false>), grid, dim3(256), 0, s, g);
    else
        hipLaunchKernelGGL((xkv_gemm_f64_kernel<false, false>), grid, dim3(256), 0, s, g);
}

// g = y^T y (r x r per problem), the n-long contraction split k_splits ways.
static void gram_tn(const XkvParams& p, const double* y, hipStream_t s) {
    const int r = p.rank;
    const int64_t nr = (int64_t)p.n * r, rr = (int64_t)r * r;
    GemmArgs g{};
    g.m = r; g.n = r; g.k = p.n; g.kc = (p.n + p.k_splits - 1) / p.k_splits; g.splits = p.k_splits;
    g.A = y; g.lda = r; g.sA = nr;
    g.B = y; g.ldb = r; g.sB = nr;
    g.C = p.g_parts; g.ldc = r; g.sC = rr * p.k_splits; g.c_split = rr;
    const dim3 grid((unsigned)((r + kGm - 1) / kGm), (unsigned)((r + kGm - 1) / kGm), (unsigned)(p.n_batch * p.k_splits));
    hipLaunchKernelGGL((xkv_gemm_f64_kernel<true, false>), grid, dim3(256), 0, s, g);
    hipLaunchKernelGGL(xkv_sum_splits_kernel, dim3((unsigned)((rr + 255) / 256), (unsigned)p.n_batch), dim3(256), 0, s,
                       p.g_parts, p.g, rr, p.k_splits);
}

// out = orth(in) by one CholeskyQR pass: G = in^T in = L L^T, out = in L^-T
// (L^-T from a triangular solve on the identity, then one product).
static void cholqr(const XkvParams& p, const double* in, double* out, hipStream_t s) {
    const int r = p.rank;
    gram_tn(p, in, s);
    launch_chol(p.g, r, p.dead, p.g_parts, p.n_batch, s);     // g_parts is free until the next Gram
    hipLaunchKernelGGL(xkv_trsm_kernel, dim3((unsigned)((r + kTrRows - 1) / kTrRows), (unsigned)p.n_batch), dim3(256), 0,
                       s, (const double*)nullptr, p.rinv, p.g, p.dead, r, r);
    gemm_nn(p, p.n, r, in, (int64_t)p.n * r, r, p.rinv, (int64_t)r * r, out, false, s);
}

// Iterations, then the outputs. X_i = orth(M X_{i-1}); the intermediate
// steps take one CholeskyQR pass (only their span feeds the next product),
// the last one two (the second restores orthogonality to rounding level).
hipError_t launch_xkv_factor(const XkvParams& p, hipStream_t s) {
    hipLaunchKernelGGL(xkv_gram_reduce_kernel, dim3(kXT / kRedRows, (unsigned)p.n_upper, (unsigned)p.n_batch), dim3(256), 0, s, p);
    const int64_t nr = (int64_t)p.n * p.rank;
    double* buf[2] = {p.x, p.y};
    const double* in = p.omega;
    int64_t s_in = 0;
    int cur = -1;
    for (int it = 0; it < p.n_iter; ++it) {
        const int prod = cur == 0 ? 1 : 0;
        gemm_nn(p, p.n, p.n, p.m, (int64_t)p.n * p.n, p.n, in, s_in, buf[prod], true, s);   // M X
        cur = prod;
        const int passes = it + 1 == p.n_iter ? 2 : 1;
        for (int ps = 0; ps < passes; ++ps) {
            cholqr(p, buf[cur], buf[1 - cur], s);
            cur = 1 - cur;
        }
        in = buf[cur];
        s_in = nr;
    }
    hipLaunchKernelGGL(xkv_emit_kernel, dim3((unsigned)(p.rank / 64), (unsigned)(p.n / 64), (unsigned)p.n_batch),
                       dim3(256), 0, s, p, (const double*)buf[cur]);
    const int n_ct = (p.rank + kXT - 1) / kXT, n_tt = (p.ctx_len + kXT - 1) / kXT;
    hipLaunchKernelGGL(xkv_a_kernel, dim3((unsigned)(n_ct * ((n_tt + 7) / 8) * 8), (unsigned)p.n_batch), dim3(kXThreads), 0, s, p);
    return hipGetLastError();
}

// ------------------------------------------------- pseudoinverse start
// explainer, Slim Attention paragraph: the predictor's linear map starts at
// the best linear guess the projections allow, W_lin = pinv(W_K) W_V (row
// vectors: k = x W_K, v = x W_V). For W_K of full column rank,
// pinv(W_K) = (W_K^T W_K)^-1 W_K^T, so with G = W_K^T W_K = L L^T and
// B = W_K^T W_V: W_lin = L^-T (L^-T)^T B, in binary64 on the same products,
// Cholesky and triangular solve as the factorisation above.
__global__ __launch_bounds__(256) void xkv_cvt_kernel(const __bf16* src, double* dst, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) dst[i] = (double)bf16_bits_to_f32(reinterpret_cast<const uint16_t*>(src)[i]);
}

// w_lin[q][o][i] = W_lin[i][o] (output-major), bf16 by one rounding, and binary64.
__global__ __launch_bounds__(256) void pinv_out_kernel(PinvParams p) {
    const int q = blockIdx.y;
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= p.d * p.d) return;
    const int o = e / p.d, i = e - o * p.d;
    const double v = p.x[((int64_t)q * p.d + i) * p.d + o];
    reinterpret_cast<uint16_t*>(p.w_lin)[(int64_t)q * p.d * p.d + e] = f64_to_bf16_bits(v);
    if (p.w_lin64) p.w_lin64[(int64_t)q * p.d * p.d + e] = v;
}

hipError_t launch_pinv(const PinvParams& p, hipStream_t s) {
    const int d = p.d, P = p.n_maps;
    const int64_t hd = (int64_t)p.hidden * d, dd = (int64_t)d * d;
    const int64_t nel = hd * P;
    hipLaunchKernelGGL(xkv_cvt_kernel, dim3((unsigned)((nel + 255) / 256)), dim3(256), 0, s, p.w_k, p.wk64, nel);
    hipLaunchKernelGGL(xkv_cvt_kernel, dim3((unsigned)((nel + 255) / 256)), dim3(256), 0, s, p.w_v, p.wv64, nel);
    auto gram = [&](const double* b, double* out) {     // out = W_K^T b over the hidden axis, split
        GemmArgs g{};
        g.m = d; g.n = d; g.k = p.hidden; g.kc = (p.hidden + p.splits - 1) / p.splits; g.splits = p.splits;
        g.A = p.wk64; g.lda = d; g.sA = hd;
        g.B = b; g.ldb = d; g.sB = hd;
        g.C = p.g_parts; g.ldc = d; g.sC = dd * p.splits; g.c_split = dd;
        const dim3 grid((unsigned)((d + kGm - 1) / kGm), (unsigned)((d + kGm - 1) / kGm), (unsigned)(P * p.splits));
        hipLaunchKernelGGL((xkv_gemm_f64_kernel<true, false>), grid, dim3(256), 0, s, g);
        hipLaunchKernelGGL(xkv_sum_splits_kernel, dim3((unsigned)((dd + 255) / 256), (unsigned)P), dim3(256), 0, s,
                           p.g_parts, out, dd, p.splits);
    };
    gram(p.wk64, p.g);
    gram(p.wv64, p.bm);
    launch_chol(p.g, d, p.dead, p.g_parts, P, s);             // g_parts is free: both Grams are summed
    hipLaunchKernelGGL(xkv_trsm_kernel, dim3((unsigned)((d + kTrRows - 1) / kTrRows), (unsigned)P), dim3(256), 0, s,
                       (const double*)nullptr, p.rinv, p.g, p.dead, d, d);
    auto small = [&](bool ta, const double* a, const double* b, double* out) {
        GemmArgs g{};
        g.m = d; g.n = d; g.k = d; g.kc = d; g.splits = 1;
        g.A = a; g.lda = d; g.sA = dd;
        g.B = b; g.ldb = d; g.sB = dd;
        g.C = out; g.ldc = d; g.sC = dd; g.c_split = 0;
        const dim3 grid((unsigned)((d + kGm - 1) / kGm), (unsigned)((d + kGm - 1) / kGm), (unsigned)P);
        if (ta) hipLaunchKernelGGL((xkv_gemm_f64_kernel<true, false>), grid, dim3(256), 0, s, g);
        else hipLaunchKernelGGL((xkv_gemm_f64_kernel<false, false>), grid, dim3(256), 0, s, g);
    };
    small(true, p.rinv, p.bm, p.t1);      // (L^-T)^T B
    small(false, p.rinv, p.t1, p.x);      // L^-T ((L^-T)^T B)
    hipLaunchKernelGGL(pinv_out_kernel, dim3((unsigned)((dd + 255) / 256), (unsigned)P), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace lowram
