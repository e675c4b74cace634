// liblowram C ABI: argument checks, workspace carving and launch sequence.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include <hip/hip_runtime.h>

#include "kernels.hpp"
#include "lowram.h"

using namespace lowram;

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof(g_err), fmt, ap);
    va_end(ap);
    return code;
}

bool misaligned(const void* p, uintptr_t a) { return p != nullptr && (reinterpret_cast<uintptr_t>(p) % a) != 0; }

size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

struct DecodePlan {
    bool mfma;
    int nb, n_cand, n_split, bps, part_stride;
    size_t off_list, off_count, off_part, off_counts, total;
};

int plan_decode(const lowram_decode_args* a, DecodePlan* pl) {
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->batch < 1 || a->ctx_len < 0 || a->n_q_heads < 1 || a->n_kv_heads < 1)
        return fail(LOWRAM_ERR_ARG, "batch/heads must be >= 1 and ctx_len >= 0");
    if (a->n_q_heads % a->n_kv_heads != 0)
        return fail(LOWRAM_ERR_ARG, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)", a->n_q_heads, a->n_kv_heads);
    if (a->head_dim != kHeadDim) return fail(LOWRAM_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", a->head_dim);
    if (a->block_size != kBlock) return fail(LOWRAM_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", a->block_size);
    if (a->rank < 32 || a->rank % 32 != 0) return fail(LOWRAM_ERR_UNSUPPORTED, "rank must be a positive multiple of 32 (got %d)", a->rank);
    if (a->mlp_hidden < 16 || a->mlp_hidden % 16 != 0 || a->mlp_hidden > 1024)
        return fail(LOWRAM_ERR_UNSUPPORTED, "mlp_hidden must be a multiple of 16 in [16, 1024] (got %d)", a->mlp_hidden);
    if (a->act_dtype != LOWRAM_F32 && a->act_dtype != LOWRAM_BF16) return fail(LOWRAM_ERR_ARG, "act_dtype must be F32 or BF16");
    if (a->a_dtype < LOWRAM_F32 || a->a_dtype > LOWRAM_I8) return fail(LOWRAM_ERR_ARG, "bad a_dtype");
    if (a->res_dtype < LOWRAM_F32 || a->res_dtype > LOWRAM_I2) return fail(LOWRAM_ERR_ARG, "bad res_dtype");
    if (a->n_res < 0 || a->n_res > a->ctx_len) return fail(LOWRAM_ERR_ARG, "n_res (%d) must be in [0, ctx_len]", a->n_res);
    if (a->win_len < 0 || a->win_cap < 0) return fail(LOWRAM_ERR_ARG, "win_len and win_cap must be >= 0");
    if (a->win_len > a->win_cap) return fail(LOWRAM_ERR_WINDOW_FULL, "win_len (%d) > win_cap (%d)", a->win_len, a->win_cap);
    if (a->win_len > 4096) return fail(LOWRAM_ERR_UNSUPPORTED, "win_len above 4096");
    if (a->flags & ~(LOWRAM_FLAG_GENERIC | LOWRAM_FLAG_VALIDATE)) return fail(LOWRAM_ERR_ARG, "unknown flag bits 0x%x", a->flags);
    const int g = a->n_q_heads / a->n_kv_heads;
    pl->nb = (a->ctx_len + kBlock - 1) / kBlock;
    if (a->sel != nullptr && (a->n_sel < 0 || a->n_sel > pl->nb))
        return fail(LOWRAM_ERR_ARG, "n_sel (%d) must be in [0, nb=%d]", a->n_sel, pl->nb);
    pl->n_cand = a->sel ? a->n_sel : pl->nb;
    if (pl->n_cand == 0 && a->win_len == 0) return fail(LOWRAM_ERR_EMPTY, "no block and no window token to attend");

    DecodeParams probe{};
    probe.group = g; probe.hidden = a->mlp_hidden; probe.rank = a->rank;
    pl->mfma = !(a->flags & LOWRAM_FLAG_GENERIC) && mfma_supported(probe, a->act_dtype, a->a_dtype, a->res_dtype);
    if (!pl->mfma && g > 8) return fail(LOWRAM_ERR_UNSUPPORTED, "GQA group above 8 needs the MFMA kernel");
    pl->bps = pl->mfma ? mfma_blocks_per_split() : 1;
    pl->n_split = (pl->n_cand + pl->bps - 1) / pl->bps;
    if (pl->n_split < 1) pl->n_split = 1;
    pl->part_stride = (2 + a->mlp_hidden + kHeadDim + 3) & ~3;
    DecodeParams sm{};
    sm.n_split = pl->n_split; sm.win_len = a->win_len; sm.hidden = a->mlp_hidden;
    const size_t smem = combine_smem_bytes(sm);
    if (smem > 65536) return fail(LOWRAM_ERR_UNSUPPORTED, "mlp_hidden too wide for the combine");

    const size_t B = a->batch;
    pl->off_list = 0;
    pl->off_count = up256(pl->off_list + B * pl->nb * sizeof(int32_t));
    pl->off_part = up256(pl->off_count + B * sizeof(int32_t));
    pl->off_counts = up256(pl->off_part + B * a->n_q_heads * (size_t)pl->n_split * pl->part_stride * sizeof(float));
    pl->total = up256(pl->off_counts + B * a->n_kv_heads * (size_t)pl->n_split * 2 * sizeof(int32_t));
    return LOWRAM_OK;
}

int check_decode_ptrs(const lowram_decode_args* a, const DecodePlan& pl) {
    if (!a->q || !a->a || !a->b_l || !a->w_lin || !a->w1 || !a->w2 || !a->out || !a->res_blk_ptr)
        return fail(LOWRAM_ERR_ARG, "q, a, b_l, w_lin, w1, w2, res_blk_ptr and out must be non-NULL");
    if (a->n_res > 0 && (!a->res_idx || !a->res_val)) return fail(LOWRAM_ERR_ARG, "res_idx and res_val must be non-NULL when n_res > 0");
    if (a->a_dtype == LOWRAM_I8 && !a->a_scale) return fail(LOWRAM_ERR_ARG, "int8 A needs a_scale");
    if ((a->res_dtype == LOWRAM_I8 || a->res_dtype == LOWRAM_I2) && a->n_res > 0 && !a->res_scale)
        return fail(LOWRAM_ERR_ARG, "int8 and 2-bit residuals need res_scale");
    if (a->win_len > 0 && (!a->win_k || !a->win_v)) return fail(LOWRAM_ERR_ARG, "win_k and win_v must be non-NULL when win_len > 0");
    if (a->combine_stream && !a->combine_ready) return fail(LOWRAM_ERR_ARG, "combine_stream needs combine_ready");
    if ((a->flags & LOWRAM_FLAG_VALIDATE) && !a->check_flags)
        return fail(LOWRAM_ERR_ARG, "LOWRAM_FLAG_VALIDATE needs check_flags");
    const void* v16[] = {a->q, a->a, a->b_l, a->w_lin, a->w1, a->w2, a->res_val, a->win_k, a->win_v, a->out, a->workspace};
    for (const void* p : v16)
        if (misaligned(p, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", p);
    const void* v4[] = {a->a_scale, a->b1, a->b2, a->res_idx, a->res_scale, a->res_blk_ptr, a->sel, a->stats,
                        a->win_len_dev, a->check_flags};
    for (const void* p : v4)
        if (misaligned(p, 4)) return fail(LOWRAM_ERR_ARG, "pointer %p is not 4-byte aligned", p);
    if (pl.total > 0 && (!a->workspace || a->workspace_bytes < pl.total))
        return fail(LOWRAM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total, a->workspace ? a->workspace_bytes : 0);
    return LOWRAM_OK;
}

struct RankPlan { size_t off_err, off_thr, off_neq, total; int nb; };

int plan_rank(const lowram_rank_args* a, RankPlan* pl) {
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->n_slices < 1 || a->ctx_len < 1 || a->n_kv_heads < 1)
        return fail(LOWRAM_ERR_ARG, "n_slices, ctx_len and n_kv_heads must be >= 1");
    if (a->head_dim != kHeadDim) return fail(LOWRAM_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", a->head_dim);
    if (a->block_size != kBlock) return fail(LOWRAM_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", a->block_size);
    if (a->n_res < 0 || a->n_res > a->ctx_len) return fail(LOWRAM_ERR_ARG, "n_res (%d) must be in [0, ctx_len]", a->n_res);
    if (a->in_dtype != LOWRAM_F32 && a->in_dtype != LOWRAM_BF16) return fail(LOWRAM_ERR_ARG, "in_dtype must be F32 or BF16");
    if (a->res_dtype < LOWRAM_F32 || a->res_dtype > LOWRAM_I2) return fail(LOWRAM_ERR_ARG, "bad res_dtype");
    pl->nb = (a->ctx_len + kBlock - 1) / kBlock;
    const size_t nseg = (size_t)a->n_slices * a->n_kv_heads;
    pl->off_err = 0;
    const size_t err_bytes = a->err ? 0 : nseg * a->ctx_len * sizeof(double);
    pl->off_thr = up256(err_bytes);
    pl->off_neq = up256(pl->off_thr + nseg * sizeof(unsigned long long));
    pl->total = up256(pl->off_neq + nseg * sizeof(int32_t));
    return LOWRAM_OK;
}

struct PrefillPlan { size_t off_err, off_thr, off_neq, total; int nb; };

int plan_prefill(const lowram_prefill_args* a, PrefillPlan* pl) {
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->n_slices < 1 || a->ctx_len < 1 || a->n_kv_heads < 1 || a->group < 1)
        return fail(LOWRAM_ERR_ARG, "n_slices, ctx_len, n_kv_heads and group must be >= 1");
    if (a->head_dim != kHeadDim) return fail(LOWRAM_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", a->head_dim);
    if (a->block_size != kBlock) return fail(LOWRAM_ERR_UNSUPPORTED, "block_size must be 64 (got %d)", a->block_size);
    if (a->rank < 64 || a->rank % 64 != 0) return fail(LOWRAM_ERR_UNSUPPORTED, "rank must be a positive multiple of 64 (got %d)", a->rank);
    if (a->mlp_hidden < 64 || a->mlp_hidden % 64 != 0 || a->mlp_hidden > 4096)
        return fail(LOWRAM_ERR_UNSUPPORTED, "mlp_hidden must be a multiple of 64 in [64, 4096] (got %d)", a->mlp_hidden);
    if ((int64_t)a->ctx_len * a->rank * 2 >= (int64_t(1) << 31))
        return fail(LOWRAM_ERR_UNSUPPORTED, "ctx_len * rank * 2 must stay below 2^31");
    if ((int64_t)a->ctx_len * a->n_kv_heads * a->head_dim * 2 >= (int64_t(1) << 31))
        return fail(LOWRAM_ERR_UNSUPPORTED, "ctx_len * n_kv_heads * head_dim * 2 must stay below 2^31");
    if (a->n_res < 0 || a->n_res > a->ctx_len) return fail(LOWRAM_ERR_ARG, "n_res (%d) must be in [0, ctx_len]", a->n_res);
    if (a->act_dtype != LOWRAM_BF16) return fail(LOWRAM_ERR_UNSUPPORTED, "act_dtype must be BF16");
    if (a->res_dtype < LOWRAM_F32 || a->res_dtype > LOWRAM_I2) return fail(LOWRAM_ERR_ARG, "bad res_dtype");
    pl->nb = (a->ctx_len + kBlock - 1) / kBlock;
    const size_t nseg = (size_t)a->n_slices * a->n_kv_heads;
    pl->off_err = 0;
    const size_t err_bytes = a->err ? 0 : nseg * a->ctx_len * sizeof(double);
    pl->off_thr = up256(err_bytes);
    pl->off_neq = up256(pl->off_thr + nseg * sizeof(unsigned long long));
    pl->total = up256(pl->off_neq + nseg * sizeof(int32_t));
    return LOWRAM_OK;
}

struct XkvPlan {
    XkvParams p;
    size_t off_part, off_m, off_x, off_y, off_g, off_gp, off_rinv, off_dead, off_xt, total;
};

int plan_xkv(const lowram_xkv_args* a, XkvPlan* pl) {
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->n_batch < 1 || a->n_batch > 65535) return fail(LOWRAM_ERR_ARG, "n_batch (%d) must be in [1, 65535]", a->n_batch);
    if (a->n_layers < 1 || a->n_layers > 16) return fail(LOWRAM_ERR_ARG, "n_layers (%d) must be in [1, 16]", a->n_layers);
    if (a->ctx_len < 1) return fail(LOWRAM_ERR_ARG, "ctx_len must be >= 1");
    if (a->width < 256 || a->width % 256 != 0 || a->width > 8192)
        return fail(LOWRAM_ERR_UNSUPPORTED, "width must be a multiple of 256 in [256, 8192] (got %d)", a->width);
    const int n = a->n_layers * a->width;
    if (n > 16384) return fail(LOWRAM_ERR_UNSUPPORTED, "n_layers * width must be at most 16384 (got %d)", n);
    if (a->rank < 64 || a->rank % 64 != 0 || a->rank > 1024 || a->rank > n)
        return fail(LOWRAM_ERR_UNSUPPORTED, "rank must be a multiple of 64 in [64, min(1024, n_layers * width)] (got %d)", a->rank);
    if (a->n_iter < 1 || a->n_iter > 16) return fail(LOWRAM_ERR_ARG, "n_iter (%d) must be in [1, 16]", a->n_iter);
    if ((int64_t)a->ctx_len * a->width * 2 >= (int64_t(1) << 31))
        return fail(LOWRAM_ERR_UNSUPPORTED, "ctx_len * width * 2 must stay below 2^31");
    XkvParams& p = pl->p;
    p = XkvParams{};
    p.n_batch = a->n_batch;
    p.n_layers = a->n_layers; p.ctx_len = a->ctx_len; p.width = a->width; p.rank = a->rank; p.n_iter = a->n_iter;
    p.n = n;
    p.nt = n / 256;
    p.n_upper = p.nt * (p.nt + 1) / 2;
    // About 2048 Gram workgroups over the batch, chunks of at least 64 tokens.
    const int max_chunks = (a->ctx_len + 63) / 64;
    const int64_t per_chunk = (int64_t)p.n_upper * a->n_batch;
    int nc = (int)((2048 + per_chunk - 1) / per_chunk);
    nc = nc < 1 ? 1 : (nc > 64 ? 64 : nc);
    nc = nc > max_chunks ? max_chunks : nc;
    p.chunk_len = ((a->ctx_len + nc - 1) / nc + 63) / 64 * 64;
    p.n_chunks = (a->ctx_len + p.chunk_len - 1) / p.chunk_len;
    const int tiles = ((p.rank + 127) / 128) * ((p.rank + 127) / 128) * a->n_batch;
    int ks = (512 + tiles - 1) / tiles;
    ks = ks > n / 256 ? n / 256 : ks;
    p.k_splits = ks < 1 ? 1 : ks;
    const size_t r = (size_t)p.rank, bt = (size_t)a->n_batch;
    pl->off_part = 0;
    pl->off_m = up256(pl->off_part + bt * xkv_partials_floats(p) * sizeof(float));
    pl->off_x = up256(pl->off_m + bt * n * n * sizeof(double));
    pl->off_y = up256(pl->off_x + bt * n * r * sizeof(double));
    pl->off_g = up256(pl->off_y + bt * n * r * sizeof(double));
    pl->off_gp = up256(pl->off_g + bt * r * r * sizeof(double));
    pl->off_rinv = up256(pl->off_gp + bt * p.k_splits * r * r * sizeof(double));
    pl->off_dead = up256(pl->off_rinv + bt * r * r * sizeof(double));
    pl->off_xt = up256(pl->off_dead + bt * r * sizeof(int32_t));
    pl->total = up256(pl->off_xt + bt * r * n * 2);
    return LOWRAM_OK;
}

struct PinvPlan { PinvParams p; size_t off[10]; size_t total; };

int plan_pinv(const lowram_pinv_args* a, PinvPlan* pl) {
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->n_maps < 1 || a->n_maps > 65535) return fail(LOWRAM_ERR_ARG, "n_maps (%d) must be in [1, 65535]", a->n_maps);
    if (a->head_dim != kHeadDim) return fail(LOWRAM_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", a->head_dim);
    if (a->hidden < a->head_dim || a->hidden > 65536)
        return fail(LOWRAM_ERR_ARG, "hidden (%d) must be in [head_dim, 65536]", a->hidden);
    PinvParams& p = pl->p;
    p = PinvParams{};
    p.n_maps = a->n_maps; p.hidden = a->hidden; p.d = a->head_dim;
    int sp = (512 + a->n_maps - 1) / a->n_maps;
    const int maxs = (a->hidden + 127) / 128;
    p.splits = sp > maxs ? maxs : (sp < 1 ? 1 : sp);
    const size_t P = a->n_maps, hd = (size_t)a->hidden * a->head_dim, dd = (size_t)a->head_dim * a->head_dim;
    const size_t sz[10] = {P * hd * 8, P * hd * 8, P * dd * 8, P * dd * 8, P * dd * 8, P * dd * 8, P * dd * 8,
                           P * p.splits * dd * 8, P * a->head_dim * 4, 0};
    size_t off = 0;
    for (int i = 0; i < 10; ++i) {
        pl->off[i] = off;
        off = up256(off + sz[i]);
    }
    pl->total = off;
    return LOWRAM_OK;
}

struct FitPlan { FitParams p; size_t off[9]; size_t total; };

int plan_fit(const lowram_fit_args* a, FitPlan* pl) {
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->n_layers < 1 || a->n_kv_heads < 1 || a->ctx_len < 1)
        return fail(LOWRAM_ERR_ARG, "n_layers, n_kv_heads and ctx_len must be >= 1");
    if (a->head_dim != kHeadDim) return fail(LOWRAM_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", a->head_dim);
    if (a->mlp_hidden < 128 || a->mlp_hidden % 128 != 0 || a->mlp_hidden > 1024)
        return fail(LOWRAM_ERR_UNSUPPORTED, "mlp_hidden must be a multiple of 128 in [128, 1024] (got %d)", a->mlp_hidden);
    if (a->n_steps < 0 || a->n_steps > 100000) return fail(LOWRAM_ERR_ARG, "n_steps (%d) must be in [0, 100000]", a->n_steps);
    if (!(a->lr == a->lr) || a->lr > 3.0e38f || a->lr < -3.0e38f) return fail(LOWRAM_ERR_ARG, "lr must be finite");
    if ((int64_t)a->ctx_len * a->n_kv_heads * a->head_dim * 2 >= (int64_t(1) << 31))
        return fail(LOWRAM_ERR_UNSUPPORTED, "ctx_len * n_kv_heads * head_dim * 2 must stay below 2^31");
    if ((int64_t)a->n_layers * a->n_kv_heads > 65535) return fail(LOWRAM_ERR_ARG, "n_layers * n_kv_heads above 65535");
    FitParams& p = pl->p;
    p = FitParams{};
    p.n_layers = a->n_layers; p.ctx_len = a->ctx_len; p.n_kv = a->n_kv_heads; p.hidden = a->mlp_hidden;
    p.n_steps = a->n_steps; p.lr = a->lr;
    p.n_probs = a->n_layers * a->n_kv_heads;
    p.m_tiles = (a->ctx_len + 63) / 64;
    // Token ranges: enough workgroups for the 256 CUs (one per CU each).
    const int P = p.n_probs, T = a->ctx_len, H = a->mlp_hidden, d = a->head_dim;
    const int fwd_tiles = (T + 31) / 32, bwd_tiles = (T + 63) / 64;
    p.fwd_ranges = std::max(1, std::min((256 + P - 1) / P, (fwd_tiles + 7) / 8));
    const int per_q = H / 128;
    p.bwd_ranges = std::max(1, std::min((256 + P * per_q - 1) / (P * per_q), bwd_tiles));
    p.n_parts = 2 * p.bwd_ranges;
    p.n_loss_parts = H <= 256 ? 8 * p.fwd_ranges : p.m_tiles;
    const size_t Pz = P, Tz = T, Hz = H, dz = d, np = p.n_parts;
    const size_t sz[9] = {Pz * Tz * dz * 2,                                   // gb
                          Pz * Hz * dz * 2, Pz * Hz * dz * 2, Pz * Hz * dz * 2, // w1b w2b w2tb
                          Pz * np * Hz * dz * 4, Pz * np * Hz * dz * 4,        // pw1 pw2
                          Pz * np * Hz * 4, Pz * np * dz * 4,                  // pb1 pb2
                          Pz * (size_t)p.n_loss_parts * 4};                    // loss_p
    size_t off = 0;
    for (int i = 0; i < 9; ++i) {
        pl->off[i] = off;
        off = up256(off + sz[i]);
    }
    pl->total = off;
    return LOWRAM_OK;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(LOWRAM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int decode_launch_all(const lowram_decode_args* a, const DecodePlan& pl, char* ws, void* stream);

// Scratch of lowram_decode_step_noalloc: a static device array, one copy per
// GPU, alive until the process ends. In host code its name is only a
// stand-in; the device address of each GPU's copy comes from
// hipGetSymbolAddress, taken once per device (with that device current) at
// the first call on it and kept here.
static __device__ __align__(256) unsigned char scratch[LOWRAM_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[kMaxDevices] = {};

int scratch_for_current_device(char** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(LOWRAM_ERR_UNSUPPORTED, "device %d above the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (ptr == nullptr || (reinterpret_cast<uintptr_t>(ptr) & 255) != 0)
            return fail(LOWRAM_ERR_HIP, "scratch array address %p is not 256-byte aligned", ptr);
        g_scratch_ptr[dev] = static_cast<char*>(ptr);
    }
    *out = g_scratch_ptr[dev];
    return LOWRAM_OK;
}

}  // namespace

extern "C" {

const char* lowram_status_string(int s) {
    switch (s) {
        case LOWRAM_OK: return "ok";
        case LOWRAM_ERR_ARG: return "invalid argument";
        case LOWRAM_ERR_UNSUPPORTED: return "unsupported shape or dtype combination";
        case LOWRAM_ERR_WORKSPACE: return "workspace missing or too small";
        case LOWRAM_ERR_WINDOW_FULL: return "window length exceeds its capacity";
        case LOWRAM_ERR_EMPTY: return "nothing to attend";
        case LOWRAM_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* lowram_last_error(void) { return g_err; }

size_t lowram_decode_workspace_size(const lowram_decode_args* a) {
    DecodePlan pl;
    return plan_decode(a, &pl) == LOWRAM_OK ? pl.total : 0;
}

int lowram_decode_step(const lowram_decode_args* a, void* stream) {
    g_err[0] = 0;
    DecodePlan pl;
    int rc = plan_decode(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    rc = check_decode_ptrs(a, pl);
    if (rc != LOWRAM_OK) return rc;
    return decode_launch_all(a, pl, static_cast<char*>(a->workspace), stream);
}

int lowram_decode_step_noalloc(const lowram_decode_args* a, void* stream) {
    g_err[0] = 0;
    DecodePlan pl;
    int rc = plan_decode(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    if (pl.total > (size_t)LOWRAM_NOALLOC_SCRATCH_BYTES)
        return fail(LOWRAM_ERR_WORKSPACE, "these shapes need %zu bytes of scratch, above the %zu of the static array "
                    "(use lowram_decode_step with a workspace)", pl.total, (size_t)LOWRAM_NOALLOC_SCRATCH_BYTES);
    lowram_decode_args chk = *a;          // the caller's workspace fields are ignored
    chk.workspace = reinterpret_cast<void*>(uintptr_t(256));
    chk.workspace_bytes = LOWRAM_NOALLOC_SCRATCH_BYTES;
    rc = check_decode_ptrs(&chk, pl);     // every host check before the first HIP call
    if (rc != LOWRAM_OK) return rc;
    char* ws = nullptr;
    rc = scratch_for_current_device(&ws);
    if (rc != LOWRAM_OK) return rc;
    return decode_launch_all(a, pl, ws, stream);
}

}  // extern "C"

namespace {

int decode_launch_all(const lowram_decode_args* a, const DecodePlan& pl, char* ws, void* stream) {
    DecodeParams p{};
    p.batch = a->batch; p.ctx_len = a->ctx_len; p.n_q = a->n_q_heads; p.n_kv = a->n_kv_heads;
    p.group = a->n_q_heads / a->n_kv_heads; p.rank = a->rank; p.hidden = a->mlp_hidden; p.n_res = a->n_res;
    p.n_blocks = pl.nb; p.win_len = a->win_len; p.win_cap = a->win_cap; p.part_stride = pl.part_stride;
    p.n_split = pl.n_split; p.blocks_per_split = pl.bps; p.scale = 0.08838834764831845f;  // 1/sqrt(128)
    p.q = a->q; p.a = a->a; p.a_scale = a->a_scale; p.b_l = a->b_l; p.w_lin = a->w_lin; p.w1 = a->w1;
    p.b1 = a->b1; p.w2 = a->w2; p.b2 = a->b2; p.res_idx = a->res_idx; p.res_val = a->res_val;
    p.res_scale = a->res_scale; p.res_ptr = a->res_blk_ptr; p.sel = a->sel; p.keep = a->keep;
    p.win_k = a->win_k; p.win_v = a->win_v; p.out = a->out; p.stats = a->stats; p.n_sel = a->n_sel;
    p.win_len_dev = a->win_len_dev;
    p.check_flags = (a->flags & LOWRAM_FLAG_VALIDATE) ? a->check_flags : nullptr;
    p.att_list = reinterpret_cast<int32_t*>(ws + pl.off_list);
    p.att_count = reinterpret_cast<int32_t*>(ws + pl.off_count);
    p.partials = reinterpret_cast<float*>(ws + pl.off_part);
    p.counts = reinterpret_cast<int32_t*>(ws + pl.off_counts);

    hipStream_t s = static_cast<hipStream_t>(stream);
    // Without eviction flags the kernels read the selection in place; the
    // compaction pass runs only when some selected blocks may be dropped.
    p.att_direct = a->keep == nullptr;
    hipError_t e = hipSuccess;
    if (p.check_flags) {
        e = launch_validate(p, s);
        if (e != hipSuccess) return hip_fail(e, "validate launch");
    }
    if (!p.att_direct) {
        e = launch_assemble(p, s);
        if (e != hipSuccess) return hip_fail(e, "assemble launch");
    }
    if (a->ev_main_begin) {
        e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_begin), s);
        if (e != hipSuccess) return hip_fail(e, "event record");
    }
    e = pl.mfma ? launch_decode_mfma(p, a->a_dtype, a->res_dtype, s)
                : launch_decode_generic(p, a->act_dtype, a->a_dtype, a->res_dtype, s);
    if (e != hipSuccess) return hip_fail(e, "decode kernel launch");
    if (a->ev_main_end) {
        e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_end), s);
        if (e != hipSuccess) return hip_fail(e, "event record");
    }
    hipStream_t cs = s;
    if (a->combine_stream) {
        cs = static_cast<hipStream_t>(a->combine_stream);
        e = hipEventRecord(static_cast<hipEvent_t>(a->combine_ready), s);
        if (e != hipSuccess) return hip_fail(e, "event record");
        e = hipStreamWaitEvent(cs, static_cast<hipEvent_t>(a->combine_ready), 0);
        if (e != hipSuccess) return hip_fail(e, "stream wait");
    }
    e = launch_combine(p, a->act_dtype, cs);
    if (e != hipSuccess) return hip_fail(e, "combine launch");
    return LOWRAM_OK;
}

}  // namespace

extern "C" {

int lowram_window_append(const lowram_window_args* a, void* stream) {
    g_err[0] = 0;
    if (a == nullptr) return fail(LOWRAM_ERR_ARG, "args is NULL");
    if (a->n_layers < 1 || a->n_layers > 65535 || a->batch < 1 || a->win_cap < 1)
        return fail(LOWRAM_ERR_ARG, "n_layers must be in [1, 65535], batch and win_cap >= 1");
    if (a->act_dtype != LOWRAM_F32 && a->act_dtype != LOWRAM_BF16) return fail(LOWRAM_ERR_ARG, "act_dtype must be F32 or BF16");
    const int eb = a->act_dtype == LOWRAM_F32 ? 4 : 2;
    if (a->width < 8 || (a->width * eb) % 16 != 0) return fail(LOWRAM_ERR_ARG, "width (%d) must fill whole 16-byte pieces", a->width);
    if (!a->new_k || !a->new_v || !a->win_k || !a->win_v || !a->win_len_dev)
        return fail(LOWRAM_ERR_ARG, "new_k, new_v, win_k, win_v and win_len_dev must be non-NULL");
    const void* v16[] = {a->new_k, a->new_v, a->win_k, a->win_v};
    for (const void* q : v16)
        if (misaligned(q, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", q);
    if (misaligned(a->win_len_dev, 4)) return fail(LOWRAM_ERR_ARG, "win_len_dev is not 4-byte aligned");
    WindowParams p{};
    p.n_layers = a->n_layers; p.batch = a->batch; p.width = a->width; p.win_cap = a->win_cap; p.elem_bytes = eb;
    p.new_k = a->new_k; p.new_v = a->new_v; p.win_k = a->win_k; p.win_v = a->win_v; p.win_len = a->win_len_dev;
    const hipError_t e = launch_window_append(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWRAM_OK : hip_fail(e, "window append launch");
}

size_t lowram_rank_workspace_size(const lowram_rank_args* a) {
    RankPlan pl;
    return plan_rank(a, &pl) == LOWRAM_OK ? pl.total : 0;
}

int lowram_rank_residuals(const lowram_rank_args* a, void* stream) {
    g_err[0] = 0;
    RankPlan pl;
    int rc = plan_rank(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    if (!a->v || !a->v_hat || !a->res_blk_ptr)
        return fail(LOWRAM_ERR_ARG, "v, v_hat and res_blk_ptr must be non-NULL");
    if (a->n_res > 0 && (!a->res_idx || !a->res_val))
        return fail(LOWRAM_ERR_ARG, "res_idx and res_val must be non-NULL when n_res > 0");
    if ((a->res_dtype == LOWRAM_I8 || a->res_dtype == LOWRAM_I2) && a->n_res > 0 && !a->res_scale)
        return fail(LOWRAM_ERR_ARG, "int8 and 2-bit residuals need res_scale");
    const void* v16[] = {a->v, a->v_hat, a->res_val, a->workspace};
    for (const void* p : v16)
        if (misaligned(p, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", p);
    const void* v8[] = {a->err};
    for (const void* p : v8)
        if (misaligned(p, 8)) return fail(LOWRAM_ERR_ARG, "err pointer %p is not 8-byte aligned", p);
    if (misaligned(a->res_idx, 4) || misaligned(a->res_blk_ptr, 4) || misaligned(a->res_scale, 4))
        return fail(LOWRAM_ERR_ARG, "index/scale pointers must be 4-byte aligned");
    if (!a->workspace || a->workspace_bytes < pl.total)
        return fail(LOWRAM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total, a->workspace ? a->workspace_bytes : 0);

    char* ws = static_cast<char*>(a->workspace);
    RankParams p{};
    p.n_slices = a->n_slices; p.ctx_len = a->ctx_len; p.n_kv = a->n_kv_heads; p.n_res = a->n_res;
    p.n_blocks = pl.nb; p.in_dtype = a->in_dtype; p.res_dtype = a->res_dtype;
    p.v = a->v; p.v_hat = a->v_hat; p.res_idx = a->res_idx; p.res_val = a->res_val;
    p.res_scale = a->res_scale; p.res_ptr = a->res_blk_ptr;
    p.err = a->err ? a->err : reinterpret_cast<double*>(ws + pl.off_err);
    p.thr = reinterpret_cast<unsigned long long*>(ws + pl.off_thr);
    p.n_eq = reinterpret_cast<int32_t*>(ws + pl.off_neq);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (a->ev_main_begin && (e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_begin), s)) != hipSuccess)
        return hip_fail(e, "event record");
    if ((e = launch_rank_error(p, s)) != hipSuccess) return hip_fail(e, "rank error launch");
    if (a->ev_main_end && (e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_end), s)) != hipSuccess)
        return hip_fail(e, "event record");
    if ((e = launch_rank_select(p, s)) != hipSuccess) return hip_fail(e, "rank select launch");
    if ((e = launch_rank_compact(p, s)) != hipSuccess) return hip_fail(e, "rank compact launch");
    if ((e = launch_rank_gather(p, s)) != hipSuccess) return hip_fail(e, "rank gather launch");
    return LOWRAM_OK;
}

size_t lowram_prefill_workspace_size(const lowram_prefill_args* a) {
    g_err[0] = 0;
    PrefillPlan pl;
    return plan_prefill(a, &pl) == LOWRAM_OK ? pl.total : 0;
}

int lowram_prefill_rank(const lowram_prefill_args* a, void* stream) {
    g_err[0] = 0;
    PrefillPlan pl;
    int rc = plan_prefill(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    if (!a->a || !a->b_l || !a->w_lin || !a->w1 || !a->w2 || !a->v || !a->res_blk_ptr)
        return fail(LOWRAM_ERR_ARG, "a, b_l, w_lin, w1, w2, v and res_blk_ptr must be non-NULL");
    if (a->n_res > 0 && (!a->res_idx || !a->res_val))
        return fail(LOWRAM_ERR_ARG, "res_idx and res_val must be non-NULL when n_res > 0");
    if ((a->res_dtype == LOWRAM_I8 || a->res_dtype == LOWRAM_I2) && a->n_res > 0 && !a->res_scale)
        return fail(LOWRAM_ERR_ARG, "int8 and 2-bit residuals need res_scale");
    const void* v16[] = {a->a, a->b_l, a->w_lin, a->w1, a->w2, a->v, a->res_val, a->v_hat, a->workspace};
    for (const void* p : v16)
        if (misaligned(p, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", p);
    if (misaligned(a->b1, 2) || misaligned(a->b2, 2)) return fail(LOWRAM_ERR_ARG, "bias pointers must be 2-byte aligned");
    if (misaligned(a->err, 8)) return fail(LOWRAM_ERR_ARG, "err pointer is not 8-byte aligned");
    if (misaligned(a->res_idx, 4) || misaligned(a->res_blk_ptr, 4) || misaligned(a->res_scale, 4))
        return fail(LOWRAM_ERR_ARG, "index/scale pointers must be 4-byte aligned");
    if (!a->workspace || a->workspace_bytes < pl.total)
        return fail(LOWRAM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total, a->workspace ? a->workspace_bytes : 0);

    char* ws = static_cast<char*>(a->workspace);
    PrefillParams p{};
    p.n_slices = a->n_slices; p.group = a->group; p.ctx_len = a->ctx_len; p.n_kv = a->n_kv_heads;
    p.rank = a->rank; p.hidden = a->mlp_hidden; p.n_res = a->n_res; p.n_blocks = pl.nb; p.res_dtype = a->res_dtype;
    p.a = a->a; p.b_l = a->b_l; p.w_lin = a->w_lin; p.w1 = a->w1; p.b1 = a->b1; p.w2 = a->w2; p.b2 = a->b2; p.v = a->v;
    p.err = a->err ? a->err : reinterpret_cast<double*>(ws + pl.off_err);
    p.v_hat = a->v_hat;
    p.res_idx = a->res_idx; p.res_val = a->res_val; p.res_scale = a->res_scale;

    RankParams r{};
    r.n_slices = a->n_slices; r.ctx_len = a->ctx_len; r.n_kv = a->n_kv_heads; r.n_res = a->n_res;
    r.n_blocks = pl.nb; r.in_dtype = LOWRAM_BF16; r.res_dtype = a->res_dtype;
    r.res_idx = a->res_idx; r.res_ptr = a->res_blk_ptr; r.err = p.err;
    r.thr = reinterpret_cast<unsigned long long*>(ws + pl.off_thr);
    r.n_eq = reinterpret_cast<int32_t*>(ws + pl.off_neq);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (a->ev_main_begin && (e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_begin), s)) != hipSuccess)
        return hip_fail(e, "event record");
    p.n_groups = prefill_groups(p, 0);
    if ((e = launch_prefill(p, 0, s)) != hipSuccess) return hip_fail(e, "prefill error launch");
    if (a->ev_main_end && (e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_end), s)) != hipSuccess)
        return hip_fail(e, "event record");
    if ((e = launch_rank_select(r, s)) != hipSuccess) return hip_fail(e, "rank select launch");
    if ((e = launch_rank_compact(r, s)) != hipSuccess) return hip_fail(e, "rank compact launch");
    if (a->n_res > 0) {
        p.n_groups = prefill_groups(p, 1);
        if ((e = launch_prefill(p, 1, s)) != hipSuccess) return hip_fail(e, "prefill residual launch");
    }
    return LOWRAM_OK;
}

size_t lowram_xkv_workspace_size(const lowram_xkv_args* a) {
    g_err[0] = 0;
    XkvPlan pl;
    return plan_xkv(a, &pl) == LOWRAM_OK ? pl.total : 0;
}

int lowram_xkv_factorize(const lowram_xkv_args* a, void* stream) {
    g_err[0] = 0;
    XkvPlan pl;
    int rc = plan_xkv(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    if (!a->keys || !a->omega || !a->a || !a->b_l) return fail(LOWRAM_ERR_ARG, "keys, omega, a and b_l must be non-NULL");
    const void* v16[] = {a->keys, a->omega, a->a, a->b_l, a->basis, a->workspace};
    for (const void* q : v16)
        if (misaligned(q, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", q);
    if (!a->workspace || a->workspace_bytes < pl.total)
        return fail(LOWRAM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total, a->workspace ? a->workspace_bytes : 0);
    char* ws = static_cast<char*>(a->workspace);
    XkvParams p = pl.p;
    p.keys = static_cast<const __bf16*>(a->keys);
    p.omega = a->omega;
    p.a = static_cast<__bf16*>(a->a);
    p.b_l = static_cast<__bf16*>(a->b_l);
    p.basis = a->basis;
    p.partials = reinterpret_cast<float*>(ws + pl.off_part);
    p.m = reinterpret_cast<double*>(ws + pl.off_m);
    p.x = reinterpret_cast<double*>(ws + pl.off_x);
    p.y = reinterpret_cast<double*>(ws + pl.off_y);
    p.g = reinterpret_cast<double*>(ws + pl.off_g);
    p.g_parts = reinterpret_cast<double*>(ws + pl.off_gp);
    p.rinv = reinterpret_cast<double*>(ws + pl.off_rinv);
    p.dead = reinterpret_cast<int32_t*>(ws + pl.off_dead);
    p.xt = reinterpret_cast<__bf16*>(ws + pl.off_xt);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if (a->ev_main_begin && (e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_begin), s)) != hipSuccess)
        return hip_fail(e, "event record");
    if ((e = launch_xkv_gram(p, s)) != hipSuccess) return hip_fail(e, "xkv gram launch");
    if (a->ev_main_end && (e = hipEventRecord(static_cast<hipEvent_t>(a->ev_main_end), s)) != hipSuccess)
        return hip_fail(e, "event record");
    if ((e = launch_xkv_factor(p, s)) != hipSuccess) return hip_fail(e, "xkv iteration launch");
    return LOWRAM_OK;
}

size_t lowram_pinv_workspace_size(const lowram_pinv_args* a) {
    g_err[0] = 0;
    PinvPlan pl;
    return plan_pinv(a, &pl) == LOWRAM_OK ? pl.total : 0;
}

int lowram_pinv_value_map(const lowram_pinv_args* a, void* stream) {
    g_err[0] = 0;
    PinvPlan pl;
    int rc = plan_pinv(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    if (!a->w_k || !a->w_v || !a->w_lin) return fail(LOWRAM_ERR_ARG, "w_k, w_v and w_lin must be non-NULL");
    const void* v16[] = {a->w_k, a->w_v, a->w_lin, a->w_lin64, a->workspace};
    for (const void* q : v16)
        if (misaligned(q, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", q);
    if (!a->workspace || a->workspace_bytes < pl.total)
        return fail(LOWRAM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total, a->workspace ? a->workspace_bytes : 0);
    char* ws = static_cast<char*>(a->workspace);
    PinvParams p = pl.p;
    p.w_k = static_cast<const __bf16*>(a->w_k);
    p.w_v = static_cast<const __bf16*>(a->w_v);
    p.w_lin = static_cast<__bf16*>(a->w_lin);
    p.w_lin64 = a->w_lin64;
    auto dbl = [&](int i) { return reinterpret_cast<double*>(ws + pl.off[i]); };
    p.wk64 = dbl(0); p.wv64 = dbl(1); p.g = dbl(2); p.bm = dbl(3); p.rinv = dbl(4); p.t1 = dbl(5); p.x = dbl(6);
    p.g_parts = dbl(7);
    p.dead = reinterpret_cast<int32_t*>(ws + pl.off[8]);
    hipError_t e = launch_pinv(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWRAM_OK : hip_fail(e, "pinv launch");
}

size_t lowram_fit_workspace_size(const lowram_fit_args* a) {
    g_err[0] = 0;
    FitPlan pl;
    return plan_fit(a, &pl) == LOWRAM_OK ? pl.total : 0;
}

int lowram_fit_predictor(const lowram_fit_args* a, void* stream) {
    g_err[0] = 0;
    FitPlan pl;
    int rc = plan_fit(a, &pl);
    if (rc != LOWRAM_OK) return rc;
    if (!a->keys || !a->v || !a->w_lin || !a->w1 || !a->b1 || !a->w2 || !a->b2)
        return fail(LOWRAM_ERR_ARG, "keys, v, w_lin, w1, b1, w2 and b2 must be non-NULL");
    const void* v16[] = {a->keys, a->v, a->w_lin, a->w1, a->b1, a->w2, a->b2, a->workspace};
    for (const void* q : v16)
        if (misaligned(q, 16)) return fail(LOWRAM_ERR_ARG, "tensor pointer %p is not 16-byte aligned", q);
    if (misaligned(a->losses, 4)) return fail(LOWRAM_ERR_ARG, "losses must be 4-byte aligned");
    if (!a->workspace || a->workspace_bytes < pl.total)
        return fail(LOWRAM_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", pl.total, a->workspace ? a->workspace_bytes : 0);
    char* ws = static_cast<char*>(a->workspace);
    FitParams p = pl.p;
    p.keys = static_cast<const __bf16*>(a->keys);
    p.v = static_cast<const __bf16*>(a->v);
    p.w_lin = static_cast<const __bf16*>(a->w_lin);
    p.w1 = a->w1; p.b1 = a->b1; p.w2 = a->w2; p.b2 = a->b2; p.losses = a->losses;
    p.gb = reinterpret_cast<__bf16*>(ws + pl.off[0]);
    p.w1b = reinterpret_cast<__bf16*>(ws + pl.off[1]);
    p.w2b = reinterpret_cast<__bf16*>(ws + pl.off[2]);
    p.w2tb = reinterpret_cast<__bf16*>(ws + pl.off[3]);
    p.pw1 = reinterpret_cast<float*>(ws + pl.off[4]);
    p.pw2 = reinterpret_cast<float*>(ws + pl.off[5]);
    p.pb1 = reinterpret_cast<float*>(ws + pl.off[6]);
    p.pb2 = reinterpret_cast<float*>(ws + pl.off[7]);
    p.loss_p = reinterpret_cast<float*>(ws + pl.off[8]);
    hipError_t e = launch_fit(p, a->ev_main_begin, a->ev_main_end, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOWRAM_OK : hip_fail(e, "fit launch");
}

}  // extern "C"
