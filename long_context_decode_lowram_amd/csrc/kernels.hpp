// Host-side launchers of the liblowram kernels (one translation unit each).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace lowram {

// Attended-set assembly: att_list/att_count from sel and keep. Grid (B).
hipError_t launch_assemble(const DecodeParams& p, hipStream_t s);

// Validate mode: defect bits of the device-side index data into p.check_flags.
constexpr uint32_t kCheckSelOrder = 1, kCheckResRange = 2, kCheckResOrder = 4, kCheckResPtr = 8, kCheckWinLen = 16;
hipError_t launch_validate(const DecodeParams& p, hipStream_t s);

// Window append: one new exact key/value row per (layer, sequence) at slot
// win_len[l] of layer l's buffers, then win_len[l] += 1. Grid (n_layers).
struct WindowParams {
    int n_layers, batch, width, win_cap, elem_bytes;
    const void* new_k; const void* new_v;   // [L, B, width]
    void* win_k; void* win_v;               // [L, B, win_cap, width]
    int32_t* win_len;                       // [L]
};
hipError_t launch_window_append(const WindowParams& p, hipStream_t s);

// Generic fp32 SIMT kernel: one workgroup per (attended block, KV head, b).
hipError_t launch_decode_generic(const DecodeParams& p, int act, int adt, int rdt, hipStream_t s);

// bf16 MFMA kernel. Returns hipErrorInvalidValue for unsupported combinations.
bool mfma_supported(const DecodeParams& p, int act, int adt, int rdt);
int mfma_blocks_per_split();
hipError_t launch_decode_mfma(const DecodeParams& p, int adt, int rdt, hipStream_t s);

// Split-K combine, window tokens, deferred W2 / b2, stats. Grid (Hq, B).
size_t combine_smem_bytes(const DecodeParams& p);
hipError_t launch_combine(const DecodeParams& p, int act, hipStream_t s);

// Residual ranking.
struct RankParams {
    int n_slices, ctx_len, n_kv, n_res, n_blocks, in_dtype, res_dtype;
    const void* v; const void* v_hat;
    int32_t* res_idx; void* res_val; float* res_scale; int32_t* res_ptr;
    double* err;                 // [Lr, Hkv, T]
    unsigned long long* thr;     // [Lr*Hkv] threshold key
    int32_t* n_eq;               // [Lr*Hkv] ties at the threshold to take
};
hipError_t launch_rank_error(const RankParams& p, hipStream_t s);
hipError_t launch_rank_select(const RankParams& p, hipStream_t s);
hipError_t launch_rank_compact(const RankParams& p, hipStream_t s);
hipError_t launch_rank_gather(const RankParams& p, hipStream_t s);

// Fused prefill ranking: V_hat from the cache parameters, then the error
// (mode 0, every token) or the residual store (mode 1, chosen tokens).
struct PrefillParams {
    int n_slices, group, ctx_len, n_kv, rank, hidden, n_res, n_blocks, res_dtype;
    int n_groups;                // workgroups per (layer, head): 4 blocks, or 256 chosen tokens
    const void* a; const void* b_l; const void* w_lin; const void* w1; const void* b1;
    const void* w2; const void* b2; const void* v;
    double* err; float* v_hat;
    int32_t* res_idx; void* res_val; float* res_scale;
};
int prefill_groups(const PrefillParams& p, int mode);
hipError_t launch_prefill(const PrefillParams& p, int mode, hipStream_t s);

// Cross-layer key factors by subspace iteration on the Gram matrix, for a
// batch of independent problems (every pointer below has a leading batch
// dimension except omega, which all problems share).
struct XkvParams {
    int n_batch, n_layers, ctx_len, width, rank, n_iter;
    int n;                        // n_layers * width
    int nt, n_upper;              // 256-column tiles per side, tiles with I <= J
    int n_chunks, chunk_len;      // token chunks of the Gram partials
    int k_splits;                 // contraction splits of the r x r Gram products
    const __bf16* keys;           // [Bt, G, T, D]
    const double* omega;          // [n, r]
    __bf16* a;                    // [Bt, T, r]
    __bf16* b_l;                  // [Bt, n, r]
    double* basis;                // [Bt, n, r] or null
    // workspace
    float* partials;              // [Bt, n_chunks, n_upper, 256, 256]
    double* m;                    // [Bt, n, n]
    double* x;                    // [Bt, n, r]
    double* y;                    // [Bt, n, r]
    double* g;                    // [Bt, r, r]  Gram, then its Cholesky factor
    double* g_parts;              // [Bt, k_splits, r, r]
    double* rinv;                 // [Bt, r, r]  L^-T
    int32_t* dead;                // [Bt, r]
    __bf16* xt;                   // [Bt, r, n]
};
size_t xkv_partials_floats(const XkvParams& p);   // per problem
hipError_t launch_xkv_gram(const XkvParams& p, hipStream_t s);     // chunk partials of C^T C
hipError_t launch_xkv_factor(const XkvParams& p, hipStream_t s);   // M, iterations, A and B_l

// Test-time fit of the predictor's nonlinear branch by gradient descent, for
// P = n_layers * n_kv problems (one per layer and KV head).
struct FitParams {
    int n_layers, ctx_len, n_kv, hidden, n_steps;
    int n_probs;                  // n_layers * n_kv
    int m_tiles;                  // 64-token tiles (tiled forward, h > 256)
    int fwd_ranges;               // token ranges per problem of the resident-weight forward (h <= 256)
    int bwd_ranges;               // token ranges per problem and hidden slice of the backward
    int n_parts;                  // weight-gradient partials per problem: 2 * bwd_ranges
    int n_loss_parts;             // loss partials per problem
    float lr;
    const __bf16* keys;           // [L, T, Hkv*d]
    const __bf16* v;              // [L, T, Hkv, d]
    const __bf16* w_lin;          // [L, Hkv, d, d]
    float* w1; float* b1; float* w2; float* b2;   // [P, h, d], [P, h], [P, d, h], [P, d]
    float* losses;                // [P, n_steps + 1] or null
    // workspace, per problem
    __bf16* gb;                   // [P, T, d]  E = v_hat - v (the loss gradient is (2 / T) E)
    __bf16* w1b; __bf16* w2b; __bf16* w2tb;       // bf16 copies: [P, h, d], [P, d, h], [P, h, d]
    float* pw1;                   // [P, n_parts, h, d]  partial dZ^T K
    float* pw2;                   // [P, n_parts, h, d]  partial H^T E ([u][o], dW2 transposed)
    float* pb1;                   // [P, n_parts, h]     partial sum_t dZ
    float* pb2;                   // [P, n_parts, d]     partial sum_t E
    float* loss_p;                // [P, n_loss_parts]   sums of squared errors
};
hipError_t launch_fit(const FitParams& p, void* ev_begin, void* ev_end, hipStream_t s);

// W_lin = pinv(W_K) W_V per problem, from bf16 projections (binary64 inside).
struct PinvParams {
    int n_maps, hidden, d;
    const __bf16* w_k; const __bf16* w_v;   // [P, hidden, d]
    __bf16* w_lin;                          // [P, d, d] output-major
    double* w_lin64;                        // [P, d, d] output-major, or null
    double* wk64; double* wv64;             // [P, hidden, d]
    double* g; double* bm; double* rinv; double* t1; double* x;   // [P, d, d]
    double* g_parts;                        // [P, splits, d, d]
    int32_t* dead;                          // [P, d]
    int splits;
};
hipError_t launch_pinv(const PinvParams& p, hipStream_t s);

}  // namespace lowram
