// Fused bf16 MFMA decode kernel for gfx950 (wave64, v_mfma_f32_16x16x32_bf16).
//
// Work split: one wave per attended 64-token block, four blocks of one KV head
// per workgroup, so the head's B_l chunks and predictor weights are staged in
// LDS once and shared by the four waves. Workgroup ids are remapped so that
// the KV heads of one block group land on the same XCD (its L2 then serves the
// eight reads of the same A rows).
//
// Per wave, all on MFMA with fp32 accumulation:
//   1. K^T[n][t] = B_l[:, head]^T . A_blk^T  over the rank, 64 rank columns
//      per chunk. Each chunk of B_l (shared) and of the wave's own A rows
//      (bf16 factor) is copied global -> LDS by direct loads one chunk ahead,
//      into unpadded rows with an XOR swizzle; no registers hold data in
//      flight, so the next chunk's loads are issued before this chunk's
//      MFMAs. int8 A rows take the same copies into two alternating
//      buffers, are widened to bf16 (exact) after the LDS read, and their
//      per-row scale multiplies the accumulator column.
//   2. The accumulators, rounded to bf16, are used in place as the A operand
//      of the next products (the k-slot order of an MFMA is free as long as
//      both operands agree, which removes any transpose):
//      S^T = K . Q^T  (query heads of this KV head padded to 16 columns),
//      Z   = K . [W1 | W_lin]^T  in chunks of 64 features.
//   3. Softmax weights against the workgroup-wide max; gelu(Z_W1 + b1) in
//      fp32; O = P . [gelu | K W_lin]  (P in registers as the A operand). The
//      W1 chunks and the W_lin chunks run as separate passes, so each tile's
//      MFMAs interleave with the previous tile's GELU; weight chunks are
//      loaded two chunks ahead.
//   4. Residual rows of the block add P[t] * R to the K W_lin part (bf16 rows
//      on MFMA 16x16x16, int8 and 2-bit rows on MFMA 16x16x32 with the row
//      scale in the weight, all through transposing LDS reads; fp32 rows per
//      row).
//   5. The four waves' O are summed in fixed order into one partial record
//      (m, l, O_G[h], O_V[d]); the combine kernel applies W2 and b2 after the
//      split merge: sum_t p_t (g_t W2 + b2) = (sum_t p_t g_t) W2 + l b2.
#include <math.h>

#include <type_traits>

#include "kernels.hpp"
#include "mfma_util.hpp"

namespace lowram {

namespace {

constexpr int kWaves = 4;                 // blocks per workgroup
constexpr int kThreads = kWaves * kWave;
constexpr int kKc = 64;                   // rank columns per staged B_l chunk
constexpr int kFc = 64;                   // features per staged weight chunk
constexpr int kRowBytes = kKc * 2;        // one bf16 row of a rank chunk: 128 bytes, eight 16-byte pieces
constexpr int kStage = kFc * kHeadDim;    // elements per stage buffer: a weight chunk (= a B_l chunk)
constexpr int kQRow = kHeadDim + 8;
constexpr int kMaxG = 8;
constexpr int kMaxHidden = 1024;             // the largest hidden width the library takes
constexpr int kXcd = 8;                   // XCDs on MI355X; workgroups go round-robin over them
constexpr int kABytes = kBlock * kRowBytes;   // one wave's A rows of a rank chunk: 8 KB
static_assert(128 * kRowBytes == kStage * 2, "a stage buffer holds one B_l chunk or one weight chunk");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_t;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2* lds_i32x2_t;

// Two 4-element halves (n .. n+3 and n+16 .. n+19) of a bf16 LDS row.
__device__ __forceinline__ bf16x8 lds_pair(const __bf16* row, int n) {
    const u32x2 lo = *reinterpret_cast<const u32x2*>(row + n);
    const u32x2 hi = *reinterpret_cast<const u32x2*>(row + n + 16);
    u32x4 v;
    v[0] = lo[0]; v[1] = lo[1]; v[2] = hi[0]; v[3] = hi[1];
    return as_bf16x8(v);
}

// 8 int8 codes -> 8 bf16 (exact: |q| <= 127 needs 7 bits).
__device__ __forceinline__ bf16x8 i8x8_to_bf16(u32x2 v) {
    bf16x8 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int q = static_cast<int8_t>((v[i >> 2] >> (8 * (i & 3))) & 0xffu);
        r[i] = (__bf16)static_cast<float>(q);
    }
    return r;
}


// Rank-chunk tiles in LDS are unpadded 128-byte rows of eight 16-byte
// pieces; piece p of row r sits in slot p ^ (r & 7). A wave's 16-byte reads
// of one logical piece from 16 consecutive rows are then free of bank
// conflicts on gfx950 (measured: as fast as contiguous reads, where padded
// 144-byte rows take 1.7x as long).
__device__ __forceinline__ int swz(int r) { return r & 7; }

}  // namespace

template <int ADT, int RDT>
__global__ __launch_bounds__(kThreads, 2) void decode_mfma_kernel(DecodeParams p, int n_split_pad) {
    // ---- workgroup -> (b, KV head, split), heads of one split on one XCD
    const int per_b = n_split_pad * p.n_kv;
    const int b = blockIdx.x / per_b;
    const int rem = blockIdx.x % per_b;
    const int xcd = rem % kXcd, slot = rem / kXcd;
    const int h = slot % p.n_kv;
    const int split = (slot / p.n_kv) * kXcd + xcd;
    if (split >= p.n_split) return;
    const int n_att = attended_count(p, b);
    if (split * kWaves >= n_att) return;         // beyond this sequence's attended blocks

    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave index, provably uniform
    const int l16 = lane & 15, g4 = lane >> 4;
    const int G = p.group, H = p.hidden, R = p.rank;

    // LDS: two stage buffers (B_l rank chunks in the main loop, weight chunks
    // after it), one region that holds each wave's A rows in the main loop
    // and the epilogue's small arrays after it, and each wave's 4 KB of
    // residual rows. Separate objects, so the compiler's waits for
    // direct-to-LDS loads can stay per buffer. 80 KB: two workgroups per CU.
    __shared__ __attribute__((aligned(16))) __bf16 stg0[kStage], stg1[kStage];
    __shared__ __attribute__((aligned(16))) unsigned char sa[kWaves * kABytes];
    __shared__ __attribute__((aligned(16))) unsigned char sres[kWaves * 4096];
    __bf16* const qs = reinterpret_cast<__bf16*>(sa);                                  // [16][kQRow]
    float (*const pl)[kMaxG][kBlock + 1] = reinterpret_cast<float (*)[kMaxG][kBlock + 1]>(sa + 4352);   // softmax weights, rows padded
    // per-wave O of a feature chunk, two buffers; they reuse the space of qs
    // and pl, which are dead by the feature loop
    float (*const oslot0)[kMaxG][kFc] = reinterpret_cast<float (*)[kMaxG][kFc]>(sa);
    float (*const oslot1)[kMaxG][kFc] = reinterpret_cast<float (*)[kMaxG][kFc]>(sa + 8192);
    float* const b1s = reinterpret_cast<float*>(sa + 20736);                           // [kMaxHidden] hidden bias
    float (*const mw)[kMaxG] = reinterpret_cast<float (*)[kMaxG]>(sa + 24832);         // per-wave score max
    float (*const lw)[kMaxG] = reinterpret_cast<float (*)[kMaxG]>(sa + 24960);         // per-wave weight sum
    int* const cnt_tok = reinterpret_cast<int*>(sa + 25088);
    int* const cnt_res = reinterpret_cast<int*>(sa + 25104);
    static_assert(25120 <= kWaves * kABytes && 20736 + 4 * kMaxHidden <= 24832 && 16 * kQRow * 2 <= 4352 && 2 * 8192 <= 20736 &&
                      4352 + kWaves * kMaxG * (kBlock + 1) * 4 <= 20736,
                  "epilogue arrays overflow sa");

    const int bi = split * kWaves + w;                 // this wave's attended-block index
    const int blk_or_none = bi < n_att ? attended_block(p, b, bi) : -1;
    const bool active = blk_or_none >= 0;
    const int blk = active ? blk_or_none : 0;
    const int t0 = blk * kBlock;
    const int nt = active ? min(kBlock, p.ctx_len - t0) : 0;

    // Residual slots lo .. hi-1 of this wave's block (wave-uniform).
    const int64_t res_row = ((int64_t)b * p.n_kv + h) * p.n_res;
    int lo = 0, hi = 0;
    if (active) {
        const int64_t pr = ((int64_t)b * p.n_kv + h) * (p.n_blocks + 1) + blk;
        lo = max(0, min(p.res_ptr[pr], p.n_res));
        hi = max(lo, min(p.res_ptr[pr + 1], p.n_res));
    }
    lo = __builtin_amdgcn_readfirstlane(lo);
    hi = __builtin_amdgcn_readfirstlane(hi);
    // The block's residual rows are consecutive rows of res_val. Each wave
    // copies up to kResRows of them at a time into its 4 KB of sres; the first
    // batch starts here, so it lands while the keys are rebuilt.
    constexpr int kResRowB = RDT == DT_I2 ? kHeadDim / 4 : kHeadDim * (RDT == DT_F32 ? 4 : (RDT == DT_BF16 ? 2 : 1));
    // 8 (f32), 16 (bf16), 32 (int8), 64 (2-bit: one row per lane holds the tokens)
    constexpr int kResRows = 4096 / kResRowB < kWave ? 4096 / kResRowB : kWave;
    constexpr int kResPieces = kResRows * kResRowB / 1024;
    unsigned char* const rs_w = sres + w * 4096;
    auto dma_res = [&](int q0) {
        const int n = min(kResRows, hi - q0);
        const __amdgpu_buffer_rsrc_t rr = buffer_rsrc(
            static_cast<const unsigned char*>(p.res_val) + (res_row + q0) * (int64_t)kResRowB, (uint32_t)(n * kResRowB));
#pragma unroll
        for (int q = 0; q < kResPieces; ++q) {
            uint32_t src = (uint32_t)(q * 1024 + lane * 16);
            if constexpr (RDT == DT_BF16) {
                // 256-byte rows; 32-byte piece pair c of row r sits at pair
                // c ^ (r & 7), so the transposing reads below are free of bank
                // conflicts: lane i fills row 4q + i/16, slot i%16.
                const int r = 4 * q + (lane >> 4), slot = lane & 15;
                src = (uint32_t)(r * 256 + (((((slot >> 1) ^ (r & 7)) << 1) | (slot & 1)) * 16));
            } else if constexpr (RDT == DT_I8) {
                // 128-byte rows; 16-byte piece c of row r sits in slot
                // c ^ (r & 7): lane i fills row 8q + i/8, slot i%8.
                const int r = 8 * q + (lane >> 3), slot = lane & 7;
                src = (uint32_t)(r * 128 + ((slot ^ (r & 7)) * 16));
            } else if constexpr (RDT == DT_I2) {
                // 32-byte rows; 16-byte half c of row r sits in slot
                // c ^ ((r >> 3) & 1): lane i fills row 32q + i/2, slot i%2.
                const int r = 32 * q + (lane >> 1), slot = lane & 1;
                src = (uint32_t)(r * 32 + ((slot ^ ((r >> 3) & 1)) * 16));
            }
            dma16<kNonTemporal>(rr, rs_w + q * 1024, src, 0u);
        }
    };
    // Token and int8 scale of residual row q0 + lane.
    // Lanes past the batch read its last row: every use of tok and scl checks
    // the row against the batch size. The loads carry no lane test and their
    // values stay as stored (the caller takes t0 off where it uses them):
    // a lane test, or arithmetic right after the load, made the compiler wait
    // for it, and for every copy issued before it, on the spot.
    auto res_meta = [&](int q0, int& tok, float& scl) {
        const int n = min(kResRows, hi - q0);            // >= 1: q0 < hi
        const int64_t r = res_row + q0 + min(lane, n - 1);
        tok = p.res_idx[r];
        scl = res_scaled(RDT) ? p.res_scale[r] : 1.f;
    };
    int tok0 = -1;
    float scl0 = 1.f;
    if (lo < hi) {
        dma_res(lo);
        res_meta(lo, tok0, scl0);
    }

    // Epilogue operands that do not depend on the keys, loaded now so that
    // they arrive with the first chunk's copies instead of costing a round
    // trip after the key loop: this thread's 8 query elements (rows >= G
    // read row G - 1 and are zeroed where staged), its hidden-bias values
    // (without b1 the query is read instead and dropped), and for int8 A the
    // row scales of its token columns (columns past the block read the
    // block's first row; those keys are zero).
    const int qj = tid >> 4, qc = (tid & 15) * 8;
    const u32x4 qv_raw = *reinterpret_cast<const u32x4*>(static_cast<const __bf16*>(p.q) +
                                                        ((int64_t)b * p.n_q + h * G + min(qj, G - 1)) * kHeadDim + qc);
    const bool has_b1 = p.b1 != nullptr;
    const uint16_t* const b1src = has_b1 ? static_cast<const uint16_t*>(p.b1) + ((int64_t)b * p.n_kv + h) * H
                                         : static_cast<const uint16_t*>(p.q);
    uint16_t b1_raw[kMaxHidden / kThreads];
#pragma unroll
    for (int k = 0; k < kMaxHidden / kThreads; ++k) b1_raw[k] = b1src[has_b1 ? min(tid + kThreads * k, H - 1) : 0];
    float ascl[4] = {1.f, 1.f, 1.f, 1.f};
    if constexpr (ADT == DT_I8) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int tl = tt * 16 + l16;
            const float sv = p.a_scale[(int64_t)b * p.ctx_len + t0 + (tl < nt ? tl : 0)];
            ascl[tt] = tl < nt ? sv : 1.f;
        }
    }

    // ---- 1. K^T = B_l(head)^T . A_blk^T
    constexpr int EA = ADT == DT_BF16 ? 2 : 1;   // bytes per A element
    const int64_t a_row0 = (int64_t)b * p.ctx_len + t0;
    const __amdgpu_buffer_rsrc_t ra =
        buffer_rsrc(static_cast<const char*>(p.a) + a_row0 * R * EA, (uint32_t)(nt * R * EA));
    const __amdgpu_buffer_rsrc_t rb =
        buffer_rsrc(static_cast<const __bf16*>(p.b_l) + ((int64_t)b * p.n_kv + h) * kHeadDim * (int64_t)R,
             (uint32_t)(kHeadDim * R * 2));
    const int n_chunks = R / kKc;

    // Direct loads of a rank chunk: instruction q of a wave fills 8 rows
    // (1 KB); lane i takes row 8q + i/8 and the piece that the swizzle puts
    // in slot i%8 (rows start at multiples of 8, so swz = i/8).
    const int dma_row = lane >> 3;
    const uint32_t dma_piece = (uint32_t)(((lane & 7) ^ dma_row) * 16);
    uint32_t bl_off[4];         // B_l: this wave fills rows 32w .. 32w+31 of the head's 128
#pragma unroll
    for (int q = 0; q < 4; ++q) bl_off[q] = (uint32_t)((w * 32 + q * 8 + dma_row) * R * 2) + dma_piece;
    // Copies past the last chunk go to a resource of size zero: they read
    // zeros and touch no memory, so every chunk issues the same copies.
    const __amdgpu_buffer_rsrc_t rnone = buffer_rsrc(p.b_l, 0u);
    auto dma_bl = [&](int c, __bf16* buf) {
        const __amdgpu_buffer_rsrc_t rbs = c < n_chunks ? rb : rnone;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            dma16(rbs, reinterpret_cast<unsigned char*>(buf) + (w * 32 + q * 8) * kRowBytes, bl_off[q], (uint32_t)(c * kRowBytes));
    };
    unsigned char* const sa_w = sa + w * kABytes;     // this wave's A rows (bf16 factor)
    auto dma_a = [&](int c) {
        const __amdgpu_buffer_rsrc_t ras = c < n_chunks ? ra : rnone;
#pragma unroll
        for (int q = 0; q < 8; ++q)
            dma16(ras, sa_w + q * 8 * kRowBytes, (uint32_t)((q * 8 + dma_row) * R * 2) + dma_piece, (uint32_t)(c * kRowBytes));
    };

    // MFMA operand reads: lane (l16, g4) takes row l16 of a 16-row tile at
    // logical piece 4 kk + g4, i.e. slot (4 kk + g4) ^ swz(l16).
    const int xs = g4 ^ swz(l16);
    const uint32_t rd_off[2] = {(uint32_t)(l16 * kRowBytes + xs * 16), (uint32_t)(l16 * kRowBytes + (xs ^ 4) * 16)};


    f32x4 acc[8][4];
#pragma unroll
    for (int nt_ = 0; nt_ < 8; ++nt_)
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) acc[nt_][tt] = f32x4{0.f, 0.f, 0.f, 0.f};

    // 64 MFMAs of one rank chunk: B_l tiles from `sb`, the 4 token tiles in
    // a8. Step s covers kk = s / 8, B_l tile s % 8; its fragment is read two
    // steps ahead.
    auto mma_chunk = [&](const __bf16* sb, const bf16x8 (&a8)[2][4]) {
        auto rd = [&](int st) { return lds16(sb, rd_off[st >> 3] + (st & 7) * 16 * kRowBytes); };
        bf16x8 bq[3];
        bq[0] = rd(0);
        bq[1] = rd(1);
#pragma unroll
        for (int st = 0; st < 16; ++st) {
            if (st + 2 < 16) bq[(st + 2) % 3] = rd(st + 2);
            const int kk = st >> 3, nt_ = st & 7;
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) acc[nt_][tt] = mfma(bq[st % 3], a8[kk][tt], acc[nt_][tt]);
        }
        // Keep that order through scheduling: two reads, then (read, 4 MFMAs)
        // fourteen times, then the last 8 MFMAs.
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
#pragma unroll
        for (int st = 0; st < 14; ++st) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
    };

    // MFMA steps s0 .. s1-1 of one rank chunk (B_l tile st % 8, k-step st / 8),
    // each B_l fragment read two steps ahead; the first two are read by the caller.
    auto mma_part = [&](const __bf16* sb, const bf16x8 (&a8)[2][4], bf16x8 (&bq)[3], auto s0c, auto s1c) {
        constexpr int s0 = decltype(s0c)::value, s1 = decltype(s1c)::value;
        auto rd = [&](int st) { return lds16(sb, rd_off[st >> 3] + (st & 7) * 16 * kRowBytes); };
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

    if constexpr (ADT == DT_BF16) {
        // Per chunk c: read this wave's A fragments of c (copied during the
        // previous chunk), start the B_l copy of chunk c+1 into the other stage
        // buffer, run four MFMA steps, then (the A reads are done by then)
        // start the A copy of chunk c+1 into the consumed region and run the
        // other twelve steps; wait for the B_l copy only (the A copy stays in
        // flight) and meet at the barrier.
        dma_bl(0, stg0);
        dma_a(0);
        wait_vmcnt<8>();
        barrier_lds();
        auto chunk = [&](int c, const __bf16* cur, __bf16* nxt) {
            bf16x8 a8[2][4];
            wait_vmcnt<0>();   // this wave's copy of the chunk's A rows (the only copy in flight)
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) a8[kk][tt] = lds16(sa_w, rd_off[kk] + tt * 16 * kRowBytes);
            dma_bl(c + 1, nxt);
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 bq[3];
            bq[0] = lds16(cur, rd_off[0]);
            bq[1] = lds16(cur, rd_off[0] + 16 * kRowBytes);
            mma_part(cur, a8, bq, std::integral_constant<int, 0>{}, std::integral_constant<int, 4>{});
            __builtin_amdgcn_sched_barrier(0);
            wait_lgkmcnt<2>();   // LDS reads complete in order: with two B_l reads issued since, the A reads are done
            dma_a(c + 1);
            __builtin_amdgcn_sched_barrier(0);
            mma_part(cur, a8, bq, std::integral_constant<int, 4>{}, std::integral_constant<int, 16>{});
            wait_vmcnt<8>();
            barrier_lds();
        };
        for (int c = 0; c < n_chunks; c += 2) {     // static buffers: even chunks in stg0
            chunk(c, stg0, stg1);
            if (c + 1 < n_chunks) chunk(c + 1, stg1, stg0);
        }
    } else {
        // int8 factor: this wave's 64-byte A rows of a rank chunk are copied
        // global -> LDS like the bf16 rows, into two 4 KB buffers that
        // alternate by chunk, so the copy of chunk c+1 starts with the chunk's
        // B_l copy. 16-byte piece c of row r sits in slot c ^ ((r >> 2) & 3),
        // which keeps the 8-byte fragment reads of 16 consecutive rows free of
        // bank conflicts. The codes are widened exactly to bf16 after the read.
        constexpr int kA8Bytes = kBlock * kKc;
        static_assert(2 * kA8Bytes <= kABytes, "two int8 A buffers per wave");
        uint32_t a8_src[4];     // instruction q fills rows 16q .. 16q+15: lane i takes row 16q + i/4, slot i%4
#pragma unroll
        for (int q = 0; q < 4; ++q)
            a8_src[q] = (uint32_t)((16 * q + (lane >> 2)) * R + (((lane & 3) ^ g4) * 16));
        auto dma_a8 = [&](int c) {
            const __amdgpu_buffer_rsrc_t ras = c < n_chunks ? ra : rnone;
            unsigned char* const dst = sa_w + (c & 1) * kA8Bytes;
#pragma unroll
            for (int q = 0; q < 4; ++q) dma16(ras, dst + q * 1024, a8_src[q], (uint32_t)(c * kKc));
        };
        // Fragment (kk, tt): row 16 tt + l16, rank columns 32 kk + 8 g4 .. +7,
        // i.e. piece 2 kk + g4 / 2, half g4 % 2.
        uint32_t a8_rd[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
            a8_rd[kk] = (uint32_t)(l16 * kKc + (((2 * kk + (g4 >> 1)) ^ (l16 >> 2)) * 16) + 8 * (g4 & 1));
        dma_bl(0, stg0);
        dma_a8(0);
        wait_vmcnt<4>();       // the residual copy and B_l chunk 0 (issued first) have landed
        barrier_lds();
        auto chunk = [&](int c, const __bf16* cur, __bf16* nxt) {
            wait_vmcnt<0>();   // this wave's A rows of chunk c (the only copy in flight)
            const unsigned char* const ab = sa_w + (c & 1) * kA8Bytes;
            u32x2 raw[2][4];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt)
                    raw[kk][tt] = *reinterpret_cast<const u32x2*>(ab + a8_rd[kk] + tt * 16 * kKc);
            dma_bl(c + 1, nxt);
            dma_a8(c + 1);
            bf16x8 a8[2][4];
#pragma unroll
            for (int kk = 0; kk < 2; ++kk)
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) a8[kk][tt] = i8x8_to_bf16(raw[kk][tt]);
            mma_chunk(cur, a8);
            wait_vmcnt<4>();   // B_l of chunk c+1 (issued before the A copy) has landed
            barrier_lds();
        };
        for (int c = 0; c < n_chunks; c += 2) {
            chunk(c, stg0, stg1);
            if (c + 1 < n_chunks) chunk(c + 1, stg1, stg0);
        }
    }

    // Nothing is in flight here (the last chunk starts no copy, and the memory
    // counter is in order, so the residual copy started before the loop has
    // landed); saying so lets the compiler drop its conservative waits on the
    // A region and the stage buffers, which the epilogue reuses.
    wait_vmcnt<0>();

    const u32x4 qv = qj < G ? qv_raw : u32x4{0u, 0u, 0u, 0u};

    // Tokens past the block's end contribute nothing: their factor rows were
    // read through a resource that ends at the block, as zeros, so their K
    // columns are zero already. int8 A: the per-row scale multiplies its column.
    if constexpr (ADT == DT_I8) {
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
#pragma unroll
            for (int nt_ = 0; nt_ < 8; ++nt_)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc[nt_][tt][i] *= ascl[tt];
        }
    }

    // ---- stage the query rows of this head (rows >= G zero); sa is free now
    *reinterpret_cast<u32x4*>(qs + qj * kQRow + qc) = qv;
    barrier_lds();           // not __syncthreads: the residual copy stays in flight

    // K as the A operand: kf[tt][s] holds n = 32s + 4g + (0..3) and 32s + 16 + 4g + (0..3).
    bf16x8 kf[4][4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int s = 0; s < 4; ++s) kf[tt][s] = pack8(acc[2 * s][tt], acc[2 * s + 1][tt]);

    // ---- 2. scores S^T = K . Q^T ; lane holds S[j = l16][t = 16 tt + 4 g4 + i]
    f32x4 sc[4];
    {
        bf16x8 qf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[s] = lds_pair(qs + l16 * kQRow, 32 * s + 4 * g4);
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            sc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int s = 0; s < 4; ++s) sc[tt] = mfma(kf[tt][s], qf[s], sc[tt]);
        }
    }
    float mloc = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tl = tt * 16 + 4 * g4 + i;
            const float v = tl < nt ? sc[tt][i] * p.scale : -INFINITY;
            sc[tt][i] = v;
            mloc = fmaxf(mloc, v);
        }
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16, kWave));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32, kWave));
    if (lane < G) mw[w][lane] = mloc;
    barrier_lds();
    float M = -INFINITY;
    if (l16 < G)
        for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, mw[ww][l16]);
    float lsum = 0.f;
#pragma unroll
    for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float e = (l16 < G && M != -INFINITY && sc[tt][i] != -INFINITY) ? __expf(sc[tt][i] - M) : 0.f;
            sc[tt][i] = e;
            lsum += e;
            if (l16 < G) pl[w][l16][tt * 16 + 4 * g4 + i] = e;
        }
    lsum += __shfl_xor(lsum, 16, kWave);
    lsum += __shfl_xor(lsum, 32, kWave);
    if (lane < G) lw[w][lane] = lsum;
    // P as the A operand over tokens: pf[u] holds t = 32u + 4g + (0..3) and 32u + 16 + 4g + (0..3).
    bf16x8 pf[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) pf[u] = pack8(sc[2 * u], sc[2 * u + 1]);

    // ---- 3/4. feature chunks of W1: Z = K W1^T + b1, gelu, O_G = P gelu(Z)
    const int n_fchunks = H / kFc;
    const __bf16* w1 = static_cast<const __bf16*>(p.w1) + ((int64_t)b * p.n_kv + h) * H * (int64_t)kHeadDim;
    const __bf16* wl = static_cast<const __bf16*>(p.w_lin) + ((int64_t)b * p.n_kv + h) * kHeadDim * (int64_t)kHeadDim;
    float* rec0 = p.partials + (((int64_t)b * p.n_q + h * G) * p.n_split + split) * (int64_t)p.part_stride;
    const int64_t rec_step = (int64_t)p.n_split * p.part_stride;

    auto stage_w = [&](int fc, u32x4 (&reg)[4]) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + kThreads * q, row = e >> 4, col = (e & 15) * 8;
            const int f = fc * kFc + row;
            reg[q] = *reinterpret_cast<const u32x4*>(w1 + (int64_t)f * kHeadDim + col);
        }
    };
    // Weight chunks in LDS: 256-byte rows (one feature) of sixteen 16-byte
    // pieces. Piece 4s + g holds the elements the MFMA lane group g needs for
    // k-group s: 32s + 4g + (0..3) and 32s + 16 + 4g + (0..3), matching the
    // k-slots of kf. Piece P of row f sits in slot P ^ (f & 15), so a wave's
    // reads of one piece from 16 consecutive rows are conflict-free. A 16-byte
    // global chunk c (elements 8c .. 8c+7) fills the half (c / 2) & 1 of two
    // pieces.
    auto store_w = [&](int buf, const u32x4 (&reg)[4]) {
        unsigned char* base = reinterpret_cast<unsigned char*>(buf ? stg1 : stg0);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int e = tid + kThreads * q, row = e >> 4, c = e & 15;
            const int sg = c >> 2, j = c & 3, g0 = (j & 1) * 2, half = j >> 1;
            unsigned char* r0 = base + row * 256 + half * 8;
            *reinterpret_cast<u32x2*>(r0 + (((4 * sg + g0) ^ (row & 15)) * 16)) = u32x2{reg[q][0], reg[q][1]};
            *reinterpret_cast<u32x2*>(r0 + (((4 * sg + g0 + 1) ^ (row & 15)) * 16)) = u32x2{reg[q][2], reg[q][3]};
        }
    };

    // Residual rows of this block, weighted by P, for all d value features at
    // once: rv[ft][i] holds feature 16 ft + l16 of query head 4 g4 + i. The
    // rows come from the LDS copies; row r's token comes from lane r.
    f32x4 rv[8];
#pragma unroll
    for (int ft = 0; ft < 8; ++ft) rv[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
    int applied = 0;
    if constexpr (RDT == DT_BF16) {
        // sum_r P[j][t_r] R[r][f] on MFMA 16x16x16 (bf16 operands, fp32 sums),
        // 16 rows a batch. A operand: lane (l16, g4) holds the weights of query
        // head l16 for rows 4 g4 .. 4 g4 + 3 (token of row r from lane r); B
        // operand: the transposing LDS read gives lane (l16, g4) feature
        // 16 ft + l16 of those four rows. The result lands as rv[ft][i] =
        // feature 16 ft + l16 of query head 4 g4 + i. Rows past n are the
        // zeros the copy left and get weight zero, as do rows outside the block.
        static_assert(kResRows == 16, "one MFMA k-step per batch of bf16 rows");
        for (int q0 = lo; q0 < hi; q0 += kResRows) {
            if (q0 != lo) {
                wait_lgkmcnt0();               // this wave's reads of the previous rows are done
                dma_res(q0);
            }
            const int n = min(kResRows, hi - q0);
            int tok = tok0;
            float scl_unused = 1.f;
            if (q0 != lo) res_meta(q0, tok, scl_unused);
            tok -= t0;
            applied += __popcll(__ballot(lane < n && tok >= 0 && tok < nt));
            s16x4 pa;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = 4 * g4 + i;
                const int t = __shfl(tok, r, kWave);
                const bool ok = r < n && t >= 0 && t < nt && l16 < G;
                pa[i] = __builtin_bit_cast(short, (__bf16)(ok ? pl[w][l16][t] : 0.f));
            }
            wait_vmcnt<0>();
            const int rr = 4 * g4 + (l16 >> 2);
#pragma unroll
            for (int ft = 0; ft < 8; ++ft) {
                const uint32_t off = (uint32_t)(rr * 256 + ((((ft ^ (rr & 7)) << 1) | ((l16 & 3) >> 1)) * 16) + 8 * (l16 & 1));
                const s16x4 pb = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t)(rs_w + off));
                rv[ft] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, pb, rv[ft], 0, 0, 0);
            }
        }
    } else if constexpr (RDT == DT_I8) {
        // The same product for int8 rows on MFMA 16x16x32, 32 rows a batch,
        // the row scale folded into the weight: A operand lane (l16, g4)
        // holds P[l16][t_r] * s_r for rows r = 8 g4 .. 8 g4 + 7; the
        // transposing byte read gives lane (l16, g4) feature 16 ft + l16 of
        // those eight rows, widened exactly to bf16.
        static_assert(kResRows == 32, "one MFMA k-step per batch of int8 rows");
        for (int q0 = lo; q0 < hi; q0 += kResRows) {
            if (q0 != lo) {
                wait_lgkmcnt0();               // this wave's reads of the previous rows are done
                dma_res(q0);
            }
            const int n = min(kResRows, hi - q0);
            int tok = tok0;
            float scl = scl0;
            if (q0 != lo) res_meta(q0, tok, scl);
            tok -= t0;
            applied += __popcll(__ballot(lane < n && tok >= 0 && tok < nt));
            bf16x8 pa;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int r = 8 * g4 + i;
                const int t = __shfl(tok, r, kWave);
                const float sr = __shfl(scl, r, kWave);
                const bool ok = r < n && t >= 0 && t < nt && l16 < G;
                pa[i] = (__bf16)(ok ? pl[w][l16][t] * sr : 0.f);
            }
            wait_vmcnt<0>();
            const int rr = 8 * g4 + (l16 >> 1);
#pragma unroll
            for (int ft = 0; ft < 8; ++ft) {
                const uint32_t off = (uint32_t)(rr * 128 + ((ft ^ (rr & 7)) * 16) + 8 * (l16 & 1));
                const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t)(rs_w + off));
                rv[ft] = mfma(pa, i8x8_to_bf16(u32x2{(unsigned)raw[0], (unsigned)raw[1]}), rv[ft]);
            }
        }
    } else if constexpr (RDT == DT_I2) {
        // 2-bit rows on MFMA 16x16x32: 64 rows a batch, 32 a k-step. The
        // byte-transposing read gives lane (l16, g4) byte column 16 bt + l16
        // of rows 8 g4 .. 8 g4 + 7; that byte holds the codes of features
        // 4 (16 bt + l16) + c, c = 0..3, in bits 2c. One byte permute per two
        // codes q makes the bf16 bit patterns 0x4300 | q, i.e. the values
        // 128 + q exactly. The level is q - 1.5, so the weighted sum is
        // sum_r w_r (128 + q_r) + sum_r w_r (-128) + sum_r w_r (-1.5), the two
        // constant terms taken on the same MFMA (-128 and -1.5 are exact in
        // bf16) and added once at the end. The weight w_r = P[j][t_r] s_r as
        // for int8. Output tile 4 bt + c holds feature 4 (16 bt + l16) + c.
        static_assert(kResRows == 64, "two MFMA k-steps per batch of 2-bit rows");
        bf16x8 cm128, cm15;
#pragma unroll
        for (int i = 0; i < 8; ++i) { cm128[i] = (__bf16)(-128.f); cm15[i] = (__bf16)(-1.5f); }
        f32x4 corr = {0.f, 0.f, 0.f, 0.f};
        for (int q0 = lo; q0 < hi; q0 += kResRows) {
            if (q0 != lo) {
                wait_lgkmcnt0();               // this wave's reads of the previous rows are done
                dma_res(q0);
            }
            const int n = min(kResRows, hi - q0);
            int tok = tok0;
            float scl = scl0;
            if (q0 != lo) res_meta(q0, tok, scl);
            tok -= t0;
            applied += __popcll(__ballot(lane < n && tok >= 0 && tok < nt));
            wait_vmcnt<0>();
            for (int ks = 0; ks * 32 < n; ++ks) {
                bf16x8 pa;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int r = 32 * ks + 8 * g4 + i;
                    const int t = __shfl(tok, r, kWave);
                    const float sr = __shfl(scl, r, kWave);
                    const bool ok = r < n && t >= 0 && t < nt && l16 < G;
                    pa[i] = (__bf16)(ok ? pl[w][l16][t] * sr : 0.f);
                }
                corr = mfma(pa, cm128, corr);
                corr = mfma(pa, cm15, corr);
                const int rr = 32 * ks + 8 * g4 + (l16 >> 1);
#pragma unroll
                for (int bt = 0; bt < 2; ++bt) {
                    const uint32_t off = (uint32_t)(rr * 32 + ((bt ^ (g4 & 1)) * 16) + 8 * (l16 & 1));
                    const i32x2 raw = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_i32x2_t)(rs_w + off));
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        const uint32_t x0 = ((uint32_t)raw[0] >> (2 * c)) & 0x03030303u;
                        const uint32_t x1 = ((uint32_t)raw[1] >> (2 * c)) & 0x03030303u;
                        u32x4 bv;
                        bv[0] = __builtin_amdgcn_perm(0x43434343u, x0, 0x04010400u);
                        bv[1] = __builtin_amdgcn_perm(0x43434343u, x0, 0x04030402u);
                        bv[2] = __builtin_amdgcn_perm(0x43434343u, x1, 0x04010400u);
                        bv[3] = __builtin_amdgcn_perm(0x43434343u, x1, 0x04030402u);
                        rv[4 * bt + c] = mfma(pa, as_bf16x8(bv), rv[4 * bt + c]);
                    }
                }
            }
        }
#pragma unroll
        for (int ft = 0; ft < 8; ++ft) rv[ft] += corr;
    } else {
        // fp32 rows: per row, on the vector ALUs.
        static_assert(RDT == DT_F32, "bf16, int8 and 2-bit rows take the MFMA paths");
        for (int q0 = lo; q0 < hi; q0 += kResRows) {
            if (q0 != lo) {
                wait_lgkmcnt0();               // this wave's reads of the previous rows are done
                dma_res(q0);
            }
            const int n = min(kResRows, hi - q0);
            int tok = tok0;
            float scl = scl0;
            if (q0 != lo) res_meta(q0, tok, scl);
            tok -= t0;
            wait_vmcnt<0>();
            // Four rows per step, all their LDS reads first. Rows past n read the
            // zeros the copy left there; rows outside the block get weight zero.
            for (int r0 = 0; r0 < n; r0 += 4) {
                float pw[4][4], v[4][8];
    #pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int r = r0 + u;
                    const int t = __builtin_amdgcn_readlane(tok, r);
                    const bool ok = r < n && t >= 0 && t < nt;
                    applied += ok ? 1 : 0;
                    const int tc = ok ? t : 0;
                    const float wr = res_scaled(RDT) ? __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, scl), r)) : 1.f;
    #pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int j = 4 * g4 + i;
                        pw[u][i] = (ok && j < G) ? pl[w][j][tc] * wr : 0.f;
                    }
    #pragma unroll
                    for (int ft = 0; ft < 8; ++ft) {
                        const int f = ft * 16 + l16;
                        v[u][ft] = *reinterpret_cast<const float*>(rs_w + r * kResRowB + f * 4);
                    }
                }
    #pragma unroll
                for (int u = 0; u < 4; ++u)
    #pragma unroll
                    for (int i = 0; i < 4; ++i)
    #pragma unroll
                        for (int ft = 0; ft < 8; ++ft) rv[ft][i] += pw[u][i] * v[u][ft];
            }
        }
    }
    // Park the residual sums in this wave's quarter of sres (its rows are
    // consumed): resS[w][j][f] for f in 0..127, added to the value part below.
    float (*const resS)[kMaxG][kHeadDim] = reinterpret_cast<float (*)[kMaxG][kHeadDim]>(sres);
    static_assert(kWaves * kMaxG * kHeadDim * 4 <= kWaves * 4096, "residual sums overflow sres");
    wait_lgkmcnt0();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int j = 4 * g4 + i;
        if (j < G) {
#pragma unroll
            for (int ft = 0; ft < 8; ++ft)   // 2-bit rows: tile ft holds feature 4 (16 (ft / 4) + l16) + ft % 4
                resS[w][j][RDT == DT_I2 ? 64 * (ft >> 2) + 4 * l16 + (ft & 3) : ft * 16 + l16] = rv[ft][i];
        }
    }
    // Weight chunks go global -> registers -> LDS, loaded two chunks ahead:
    // chunk fc stores chunk fc+1 from one register set (loaded at the start
    // of chunk fc-1) and loads chunk fc+2 into the other; the two sets swap
    // roles from chunk to chunk, so no copy waits on a load in flight. Chunk
    // 0's loads start here, ahead of the value part.
    u32x4 preA[4], preB[4];
    stage_w(0, preA);

    // ---- 4b. The value part by linearity: sum_t p_t (k_t W_lin^T) =
    // (sum_t p_t k_t) W_lin^T. Each wave forms P K (query heads x 128
    // features) on MFMA; the contraction runs over tokens, which K holds across
    // lanes, so K goes through LDS once (this wave's 8 KB of a stage buffer,
    // 32 token rows of 256 bytes, 32-byte pair c of row r at pair c ^ (r & 7))
    // and comes back through the transposing read. The four waves' P K are
    // summed in fixed order, rounded to bf16 and multiplied by W_lin^T (two
    // 16-feature output tiles per wave); the residual sums are added and the
    // result is the record's value part.
    {
        // W_lin rows of this wave's output tiles: lane (l16, g4) of tile e,
        // k-step ks holds W_lin[16 (2w + e) + l16][32 ks + 8 g4 .. + 7].
        u32x4 wlf[2][4];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                wlf[e][ks] = *reinterpret_cast<const u32x4*>(wl + (int64_t)(16 * (2 * w + e) + l16) * kHeadDim + 32 * ks + 8 * g4);
        unsigned char* const kt_w = reinterpret_cast<unsigned char*>(w < 2 ? stg0 : stg1) + (w & 1) * 8192;
        f32x4 pk[8];
#pragma unroll
        for (int ft = 0; ft < 8; ++ft) pk[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < 2; ++u) {          // tokens 32 u .. 32 u + 31 (token tiles 2u, 2u + 1)
            // kf[tt][s] holds, for token 16 tt + l16, features 32 s + 4 g4 + (0..3)
            // (bytes 8 g4 of pair 2 s) and 32 s + 16 + 4 g4 + (0..3) (pair 2 s + 1).
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int rr = 16 * e + l16;
#pragma unroll
                for (int sg = 0; sg < 4; ++sg) {
                    const u32x4 v = __builtin_bit_cast(u32x4, kf[2 * u + e][sg]);
                    *reinterpret_cast<u32x2*>(kt_w + rr * 256 + (((2 * sg) ^ (rr & 7)) * 32) + 8 * g4) = u32x2{v[0], v[1]};
                    *reinterpret_cast<u32x2*>(kt_w + rr * 256 + (((2 * sg + 1) ^ (rr & 7)) * 32) + 8 * g4) = u32x2{v[2], v[3]};
                }
            }
            // B operand of tile ft: lane (l16, g4) takes feature 16 ft + l16 of
            // token rows 4 g4 + (0..3) and 16 + 4 g4 + (0..3), the k-slot order
            // of pf[u]; lanes 4 r' + c name row 4 g4 + r' at columns 16 ft + 4 c.
            const int r1 = 4 * g4 + (l16 >> 2), r2 = r1 + 16;
#pragma unroll
            for (int ft = 0; ft < 8; ++ft) {
                const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t)(kt_w + r1 * 256 + ((ft ^ (r1 & 7)) * 32) + 8 * (l16 & 3)));
                const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_t)(kt_w + r2 * 256 + ((ft ^ (r2 & 7)) * 32) + 8 * (l16 & 3)));
                u32x4 bv;
                bv[0] = (uint32_t)(uint16_t)lo[0] | ((uint32_t)(uint16_t)lo[1] << 16);
                bv[1] = (uint32_t)(uint16_t)lo[2] | ((uint32_t)(uint16_t)lo[3] << 16);
                bv[2] = (uint32_t)(uint16_t)hi[0] | ((uint32_t)(uint16_t)hi[1] << 16);
                bv[3] = (uint32_t)(uint16_t)hi[2] | ((uint32_t)(uint16_t)hi[3] << 16);
                pk[ft] = mfma(pf[u], as_bf16x8(bv), pk[ft]);
            }
            wait_lgkmcnt0();                   // this wave's reads are done before the next rows overwrite them
        }
        // P K of each wave, pk_w[j][f], in that wave's own 8 KB (its K rows are
        // read), so only one barrier orders the four waves' sums.
        auto pks = [&](int ww) {
            return reinterpret_cast<float (*)[kHeadDim]>(reinterpret_cast<unsigned char*>(ww < 2 ? stg0 : stg1) + (ww & 1) * 8192);
        };
        static_assert(kMaxG * kHeadDim * 4 <= 8192, "P K sums overflow a wave's space");
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = 4 * g4 + i;
            if (j < G) {
#pragma unroll
                for (int ft = 0; ft < 8; ++ft) pks(w)[j][ft * 16 + l16] = pk[ft][i];
            }
        }
        barrier_lds();
        // A operand: (sum over waves of P K)[j = l16][32 ks + 8 g4 .. + 7] in bf16.
        bf16x8 pa[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            float sum[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) sum[i] = 0.f;
            if (l16 < G) {
#pragma unroll
                for (int ww = 0; ww < kWaves; ++ww) {
                    const float* src = &pks(ww)[l16][32 * ks + 8 * g4];
#pragma unroll
                    for (int i = 0; i < 8; ++i) sum[i] += src[i];
                }
            }
#pragma unroll
            for (int i = 0; i < 8; ++i) pa[ks][i] = (__bf16)sum[i];
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            f32x4 ov = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) ov = mfma(pa[ks], as_bf16x8(wlf[e][ks]), ov);
            const int f = 16 * (2 * w + e) + l16;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * g4 + i;
                if (j < G)
                    rec0[j * rec_step + 2 + H + f] =
                        ov[i] + (((resS[0][j][f] + resS[1][j][f]) + resS[2][j][f]) + resS[3][j][f]);
            }
        }
    }
    // Past the value part's barrier every wave is done with the query rows and
    // softmax weights; their space holds the two per-wave O buffers of the
    // feature loop.
#pragma unroll
    for (int k = 0; k < kMaxHidden / kThreads; ++k) {
        const int e = tid + kThreads * k;
        if (e < H) b1s[e] = has_b1 ? __uint_as_float((uint32_t)b1_raw[k] << 16) : 0.f;
    }
    barrier_lds();               // every wave has read the P K sums in the stage buffers
    store_w(0, preA);
    stage_w(min(1, n_fchunks - 1), preA);
    __syncthreads();
    // One feature chunk of W1. No branch splits a tile's MFMAs from the GELU
    // of the tile before it, so the two interleave.
    auto fchunk = [&](int fc, u32x4 (&cur)[4], u32x4 (&nxt)[4]) {
        stage_w(min(fc + 2, n_fchunks - 1), nxt);    // unconditional; the last chunks reload the last
        const __bf16* sw = (fc & 1) ? stg1 : stg0;
        const int f0 = fc * kFc;
        // Z for one 16-feature tile; on the W1 part the accumulator starts at the bias.
        auto ztile = [&](int ft, f32x4 (&z)[4]) {
            bf16x8 wf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s)
                wf[s] = lds16(sw, (uint32_t)((ft * 16 + l16) * 256 + (((4 * s + g4) ^ l16) * 16)));
            const float bb = b1s[f0 + ft * 16 + l16];
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                z[tt] = f32x4{bb, bb, bb, bb};
#pragma unroll
                for (int s = 0; s < 4; ++s) z[tt] = mfma(kf[tt][s], wf[s], z[tt]);
            }
        };
        f32x4 o[4], zc[4], zn[4];
        ztile(0, zc);
#pragma unroll
        for (int ft = 0; ft < 4; ++ft) {
            if (ft + 1 < 4) ztile(ft + 1, zn);        // the next tile's MFMAs overlap this tile's GELU
            gelu_tail16(zc);
            o[ft] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 2; ++u) o[ft] = mfma(pf[u], pack8(zc[2 * u], zc[2 * u + 1]), o[ft]);
            if (ft + 1 < 4) {
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) zc[tt] = zn[tt];
            }
            {
                // Interleave: the next tile's 16 MFMAs each followed by a share
                // of this tile's GELU, so the matrix pipe and the vector ALU
                // work side by side.
                if (ft + 1 < 4) {
                    __builtin_amdgcn_sched_group_barrier(0x100, 5, 0);
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, 7, 0);
                    }
                }
                __builtin_amdgcn_sched_group_barrier(0x002, 40, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
            }
        }
        float (*const os)[kMaxG][kFc] = (fc & 1) ? oslot1 : oslot0;
#pragma unroll
        for (int ft = 0; ft < 4; ++ft)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 4 * g4 + i;
                if (j < G) os[w][j][ft * 16 + l16] = active ? o[ft][i] : 0.f;
            }
        store_w((fc + 1) & 1, cur);     // the other buffer: nobody reads it in this chunk
        __syncthreads();
        // Sum the four waves' O in fixed order. The next write of this buffer
        // comes two chunks later, after every wave has passed the next barrier.
        for (int e = tid; e < G * kFc; e += kThreads) {
            const int j = e / kFc, fl = e % kFc;
            float v = os[0][j][fl] + os[1][j][fl] + os[2][j][fl] + os[3][j][fl];
            rec0[j * rec_step + 2 + f0 + fl] = v;
        }
    };
    const int n_g = H / kFc;
    for (int fc = 0; fc < n_g; fc += 2) {
        fchunk(fc, preA, preB);
        if (fc + 1 < n_g) fchunk(fc + 1, preB, preA);
    }

    // ---- 5. record header and counts
    if (tid < G) {
        float m = -INFINITY, l = 0.f;
        for (int ww = 0; ww < kWaves; ++ww) m = fmaxf(m, mw[ww][tid]);
        for (int ww = 0; ww < kWaves; ++ww) l += lw[ww][tid];
        rec0[tid * rec_step + 0] = m;
        rec0[tid * rec_step + 1] = l;
    }
    if (lane == 0) {
        cnt_tok[w] = nt;
        cnt_res[w] = applied;
    }
    __syncthreads();
    if (tid == 0) {
        int32_t* c = p.counts + (((int64_t)b * p.n_kv + h) * p.n_split + split) * 2;
        c[0] = cnt_tok[0] + cnt_tok[1] + cnt_tok[2] + cnt_tok[3];
        c[1] = cnt_res[0] + cnt_res[1] + cnt_res[2] + cnt_res[3];
    }
}

bool mfma_supported(const DecodeParams& p, int act, int adt, int rdt) {
    (void)rdt;
    return act == DT_BF16 && (adt == DT_BF16 || adt == DT_I8) && p.group >= 1 && p.group <= kMaxG &&
           p.hidden % kFc == 0 && p.rank % kKc == 0;
}

int mfma_blocks_per_split() { return kWaves; }

template <int ADT>
static hipError_t launch_r(const DecodeParams& p, int rdt, hipStream_t s) {
    const int n_split_pad = (p.n_split + kXcd - 1) / kXcd * kXcd;
    const dim3 grid((unsigned)((int64_t)n_split_pad * p.n_kv * p.batch));
    switch (rdt) {
        case DT_F32: hipLaunchKernelGGL((decode_mfma_kernel<ADT, DT_F32>), grid, dim3(kThreads), 0, s, p, n_split_pad); break;
        case DT_BF16: hipLaunchKernelGGL((decode_mfma_kernel<ADT, DT_BF16>), grid, dim3(kThreads), 0, s, p, n_split_pad); break;
        case DT_I8: hipLaunchKernelGGL((decode_mfma_kernel<ADT, DT_I8>), grid, dim3(kThreads), 0, s, p, n_split_pad); break;
        default: hipLaunchKernelGGL((decode_mfma_kernel<ADT, DT_I2>), grid, dim3(kThreads), 0, s, p, n_split_pad); break;
    }
    return hipGetLastError();
}

hipError_t launch_decode_mfma(const DecodeParams& p, int adt, int rdt, hipStream_t s) {
    return adt == DT_I8 ? launch_r<DT_I8>(p, rdt, s) : launch_r<DT_BF16>(p, rdt, s);
}

}  // namespace lowram
