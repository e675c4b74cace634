/*
 * lowram.h -- C ABI of liblowram, the MI355X (gfx950) decode-time path of
 * LowRAM KV-cache compression.
 *
 * What the cache holds (project site, Figure 1; explainer, mechanism
 * paragraph): low-rank keys, a per-head value predictor fitted to the
 * context, and exact residuals for the tokens the predictor gets worst.
 * Keys are K_l = A . B_l with A shared by a group of adjacent layers and B_l
 * per layer (project site, Figure 3; explainer, keys paragraph).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller, row-major
 *     and contiguous in the shapes written below, 16-byte aligned. The library
 *     never allocates, frees or synchronises; work is enqueued on `stream`
 *     (a hipStream_t passed as void*, NULL = the null stream) and runs
 *     asynchronously.
 *   - Every weight matrix is stored output-major, the layout of
 *     torch.nn.Linear.weight: [out_features, in_features].
 *   - Host-side argument checks run before any HIP call; on failure nothing is
 *     launched and a negative status is returned. lowram_last_error() then
 *     holds a message (thread-local).
 *   - Device data that the host cannot check (block lists, residual indices,
 *     block pointers) is bounds-guarded in the kernels: out-of-range entries
 *     are skipped, never dereferenced.
 *   - Offsets are computed in 64-bit.
 */
#ifndef LOWRAM_H
#define LOWRAM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LOWRAM_OK               0
#define LOWRAM_ERR_ARG         -1  /* null pointer, bad shape, misalignment      */
#define LOWRAM_ERR_UNSUPPORTED -2  /* dtype combination or shape not built       */
#define LOWRAM_ERR_WORKSPACE   -3  /* workspace missing or smaller than required */
#define LOWRAM_ERR_WINDOW_FULL -4  /* win_len > win_cap                          */
#define LOWRAM_ERR_EMPTY       -5  /* nothing to attend (no block and no window) */
#define LOWRAM_ERR_HIP         -6  /* a HIP launch or runtime call failed        */

/* Element types. */
#define LOWRAM_F32  0
#define LOWRAM_BF16 1
#define LOWRAM_I8   2   /* symmetric codes with a float32 scale per row */
/* 2-bit residual codes (residuals only; explainer, comparison table: LowRAM
 * combined with quantization stores 2-bit residuals). Four codes per byte,
 * element i in bits 2(i mod 4) of byte i / 4, so a d-element row takes d / 4
 * bytes; value (q - 1.5) s with a float32 scale s per row. */
#define LOWRAM_I2   3

/* Flags for lowram_decode_args.flags. */
#define LOWRAM_FLAG_GENERIC  1  /* use the fp32 SIMT kernel even where the MFMA kernel applies */
#define LOWRAM_FLAG_VALIDATE 2  /* check the device-side index data first; defects set bits of
                                   *check_flags (LOWRAM_CHECK_*), the step still runs, guarded */

/* Bits that the validate mode ORs into *check_flags. The library only sets
 * bits: the caller clears the word (e.g. with a fill kernel) before the call
 * and reads it once the stream has passed the call. */
#define LOWRAM_CHECK_SEL_ORDER  1   /* sel: the in-range entries of a row are not strictly ascending */
#define LOWRAM_CHECK_RES_RANGE  2   /* res_idx: an entry outside [0, ctx_len)                        */
#define LOWRAM_CHECK_RES_ORDER  4   /* res_idx: a row is not strictly ascending                     */
#define LOWRAM_CHECK_RES_PTR    8   /* res_blk_ptr: not the block CSR of res_idx                    */
#define LOWRAM_CHECK_WIN_LEN   16   /* *win_len_dev outside [0, win_len]                            */

/*
 * One layer's decode step for a batch (explainer, prefill/decode paragraph:
 * only the chunks the current query selects are rebuilt; paper page,
 * Abstract: a selected subset of KV pairs per step).
 *
 * For each sequence b the attended compressed tokens are the 64-token blocks
 * listed in sel[b] (every block when sel is NULL) that keep[b] marks kept
 * (every listed block when keep is NULL); block i covers tokens
 * [64 i, min(64 i + 64, ctx_len)). For each attended token t and KV head h:
 *   k_t      = a_t . B_l                      (a_t = q_t * a_scale[t] for int8)
 *   k_{t,h}  = k_t[h d : h d + d]
 *   v_{t,h}  = k_{t,h} W_lin + gelu(k_{t,h} W1 + b1) W2 + b2
 *              + R[slot] when t is stored among h's residuals
 * (explainer, mechanism and Slim Attention paragraphs), plus win_len exact
 * recent tokens (win_k, win_v) per head. Query head j attends over KV head
 * j / (n_q_heads / n_kv_heads) with scale 1/sqrt(head_dim):
 *   out[b, j] = softmax(q_j . K^T / sqrt(d)) . V.
 * gelu is the exact error-function form.
 *
 * Shapes (B = batch, T = ctx_len, r = rank, h = mlp_hidden, d = head_dim,
 * Hq = n_q_heads, Hkv = n_kv_heads, k = n_res, nb = ceil(T / block_size)):
 */
typedef struct lowram_decode_args {
    int32_t batch, ctx_len, n_q_heads, n_kv_heads, head_dim, rank, mlp_hidden, block_size;
    int32_t n_res;        /* residual slots per (b, KV head), 0..T                   */
    int32_t n_sel;        /* entries per sel row (ignored when sel is NULL)          */
    int32_t win_len;      /* exact window tokens attended, 0..win_cap               */
    int32_t win_cap;      /* rows allocated per sequence in win_k / win_v           */
    int32_t act_dtype;    /* F32 | BF16: q, b_l, w_*, b*, win_*, out                */
    int32_t a_dtype;      /* F32 | BF16 | I8                                        */
    int32_t res_dtype;    /* F32 | BF16 | I8 | I2                                   */
    int32_t flags;        /* LOWRAM_FLAG_*                                          */

    const void    *q;           /* [B, Hq, d]                                       */
    const void    *a;           /* [B, T, r]   this layer's group factor A          */
    const float   *a_scale;     /* [B, T]      int8 A only, else NULL               */
    const void    *b_l;         /* [B, Hkv*d, r]  B_l output-major (= B_l^T)        */
    const void    *w_lin;       /* [B, Hkv, d, d]                                   */
    const void    *w1;          /* [B, Hkv, h, d]                                   */
    const void    *b1;          /* [B, Hkv, h]  or NULL (= 0)                       */
    const void    *w2;          /* [B, Hkv, d, h]                                   */
    const void    *b2;          /* [B, Hkv, d]  or NULL (= 0)                       */
    const int32_t *res_idx;     /* [B, Hkv, k] strictly ascending (NULL if k == 0) */
    const void    *res_val;     /* [B, Hkv, k, d] (I2: [B, Hkv, k, d/4] bytes; NULL if k == 0) */
    const float   *res_scale;   /* [B, Hkv, k] I8 / I2 residuals only, else NULL    */
    const int32_t *res_blk_ptr; /* [B, Hkv, nb+1] slots of block i: [p[i], p[i+1])  */
    const int32_t *sel;         /* [B, n_sel] ascending block indices, or NULL;
                                   entries outside [0, nb) are padding and skipped */
    const uint8_t *keep;        /* [B, nb] 1 = kept, 0 = evicted, or NULL           */
    const void    *win_k;       /* [B, win_cap, Hkv*d] or NULL when win_len == 0    */
    const void    *win_v;       /* [B, win_cap, Hkv*d]                              */

    void          *out;         /* [B, Hq, d] output, act_dtype                     */
    int32_t       *stats;       /* [B, Hkv, 2] or NULL: (tokens attended incl.
                                   window, residuals applied)                       */
    void          *workspace;   /* device scratch, >= lowram_decode_workspace_size  */
    size_t         workspace_bytes;

    void          *ev_main_begin; /* optional hipEvent_t recorded right before and  */
    void          *ev_main_end;   /* after the fused reconstruct+attend kernel       */

    void          *combine_stream; /* optional hipStream_t for the split-K combine,
                                      or NULL (the combine follows on `stream`)      */
    void          *combine_ready;  /* hipEvent_t, required with combine_stream      */

    const int32_t *win_len_dev;    /* optional: one int32 in device memory holding the
                                      number of window tokens to attend, read when the
                                      kernels run (so one captured graph serves a
                                      growing window); win_len is then its upper bound
                                      and values outside [0, win_len] are clamped.
                                      NULL: win_len itself is attended.              */
    uint32_t      *check_flags;    /* device word for LOWRAM_FLAG_VALIDATE, else NULL */
} lowram_decode_args;

/* Enqueue one layer's decode step. Returns LOWRAM_OK or a negative status.
 * A sequence with nothing to attend (its blocks all evicted and no window)
 * gets a zero output row and zero stats; LOWRAM_ERR_EMPTY is returned only
 * when the host can see that every sequence is empty (ctx_len == 0 or
 * n_sel == 0, and win_len == 0). The call only launches kernels (and
 * records the optional events), so it may be captured into a HIP graph;
 * replays read the argument buffers as they are at replay time.
 *
 * With combine_stream set, the call records combine_ready on `stream` after
 * the fused kernel, makes combine_stream wait for it and runs the split-K
 * combine (which reads the workspace and writes out and stats) there, so
 * that it can overlap the caller's next work on `stream`. The caller then
 * orders on combine_stream whatever reuses this workspace or reads out or
 * stats (for example the next layer's call with the same workspace); a
 * next call with another workspace may run on `stream` at once. */
int lowram_decode_step(const lowram_decode_args *args, void *stream);

/* Bytes of workspace lowram_decode_step needs for these shapes; 0 when the
 * arguments are invalid (see lowram_last_error). */
size_t lowram_decode_workspace_size(const lowram_decode_args *args);

/*
 * lowram_decode_step without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, kernels and results as
 * lowram_decode_step; workspace and workspace_bytes are ignored. The step's
 * scratch (attended-block lists, split-K partial records, counts) lives in a
 * static device array of LOWRAM_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process ends; the call itself allocates
 * and frees nothing. Its device address is looked up once per device, at the
 * first call on that device (make that first call outside graph capture).
 * Shapes whose lowram_decode_workspace_size exceeds the array are rejected
 * with LOWRAM_ERR_WORKSPACE before any HIP call (e.g. batch 12 with every one
 * of 2048 blocks a candidate; the 131072- and 262144-token shapes with a
 * selection of 256 blocks fit up to batch 8 and beyond). Nothing in the
 * scratch has to start at zero: every value the kernels read was written
 * earlier in the same call. All calls on one GPU share its array, so calls
 * that may overlap there (on different streams, or a combine_stream that
 * overlaps the next call) race: order them on one stream.
 */
#define LOWRAM_NOALLOC_SCRATCH_BYTES (64u << 20)
int lowram_decode_step_noalloc(const lowram_decode_args *args, void *stream);

/*
 * Validate mode (flags & LOWRAM_FLAG_VALIDATE, check_flags non-NULL). Before
 * the step's kernels, one more kernel reads the device-side index data the
 * host cannot see and ORs a LOWRAM_CHECK_* bit into *check_flags for every
 * kind of defect it finds:
 *   - a row of sel whose in-range entries are not strictly ascending
 *     (padding entries outside [0, nb) are allowed anywhere);
 *   - a res_idx entry outside [0, ctx_len), or a (b, h) row of res_idx that
 *     is not strictly ascending;
 *   - a res_blk_ptr row that is not the block CSR of its res_idx row
 *     (ptr[0] = 0, ptr[nb] = n_res, non-decreasing, and every slot s lies in
 *     [ptr[i], ptr[i+1]) for the block i = res_idx[s] / 64 of its token);
 *   - *win_len_dev outside [0, win_len].
 * The step itself runs as usual: its kernels are bounds-guarded and never
 * read outside the documented shapes, so a defect gives a wrong output
 * (e.g. residuals outside their block are skipped), not a fault. The check
 * costs one pass over the indices (about 1 MB per call at 131072 tokens);
 * the call neither synchronises nor reads the word back.
 */

/*
 * Window append (explainer, prefill/decode paragraph: newly generated tokens
 * are kept exactly, uncompressed). For each of n_layers recent-window
 * buffers and each sequence b, writes the step's new key and value rows
 *   win_k[l, b, pos_l, :] = new_k[l, b, :],  win_v[l, b, pos_l, :] = new_v[l, b, :]
 * at pos_l = win_len_dev[l], then sets win_len_dev[l] = pos_l + 1, so a
 * decode call that follows on the stream with that counter as its
 * win_len_dev attends the token. A buffer that is full (pos_l outside
 * [0, win_cap)) is left as it is, counter included. One launch, no
 * allocation and no synchronisation: it may be captured into a HIP graph
 * with the decode calls, and each replay appends at the counter's current
 * value. Layer l's buffers win_k[l], win_v[l] are what its decode call
 * takes as win_k, win_v.
 * Shapes: new_k, new_v [n_layers, B, width] (width = n_kv_heads * head_dim,
 * a multiple of 8) and win_k, win_v [n_layers, B, win_cap, width] in
 * act_dtype; win_len_dev int32 [n_layers]. Pointers 16-byte aligned
 * (win_len_dev 4).
 */
typedef struct lowram_window_args {
    int32_t n_layers, batch, width, win_cap;
    int32_t act_dtype;          /* F32 | BF16                                         */
    const void *new_k;          /* [n_layers, B, width]                               */
    const void *new_v;          /* [n_layers, B, width]                               */
    void       *win_k;          /* [n_layers, B, win_cap, width]                      */
    void       *win_v;          /* [n_layers, B, win_cap, width]                      */
    int32_t    *win_len_dev;    /* [n_layers] in/out fill counts                      */
} lowram_window_args;

int lowram_window_append(const lowram_window_args *args, void *stream);

/*
 * Prefill-side residual ranking (paper page, Abstract: residuals for the
 * tokens the predictor reconstructs worst; explainer, three-details
 * paragraph: ranking by error). For each slice s and KV head h of
 * V, V_hat [Lr, T, Hkv, d]:
 *   e_t  = sum_i (V[s,t,h,i] - V_hat[s,t,h,i])^2, accumulated in index order
 *          in binary64, one rounding per multiply and per add;
 *   I    = the n_res tokens with the largest e_t, ties to the lower index,
 *          stored in ascending order;
 *   R    = V - V_hat at those tokens, computed exactly in binary64 and stored
 *          as res_dtype: F32 / BF16 rounded to nearest-even in one step, or
 *          I8 with s = float32(max|R| / 127) and q = clamp(rint(R / s), +-127),
 *          or I2 with s = float32(max|R| / 1.5) and
 *          q = clamp(rint(R / s + 1.5), 0, 3) (q = 2 for a zero row), the
 *          quotient and sum in binary64;
 *   ptr  = block CSR: ptr[i] = #{t in I : t < i * block_size}, ptr[nb] = n_res.
 */
typedef struct lowram_rank_args {
    int32_t n_slices, ctx_len, n_kv_heads, head_dim, block_size, n_res;
    int32_t in_dtype;           /* F32 | BF16                                       */
    int32_t res_dtype;          /* F32 | BF16 | I8 | I2                             */

    const void *v;              /* [Lr, T, Hkv, d]                                  */
    const void *v_hat;          /* [Lr, T, Hkv, d]                                  */

    int32_t    *res_idx;        /* [Lr, Hkv, k]      (may be NULL when k == 0)      */
    void       *res_val;        /* [Lr, Hkv, k, d]  res_dtype, I2: [.., d/4] bytes  */
    float      *res_scale;      /* [Lr, Hkv, k]  I8 / I2 only, else NULL            */
    int32_t    *res_blk_ptr;    /* [Lr, Hkv, nb+1]                                  */
    double     *err;            /* [Lr, Hkv, T] or NULL (then kept in workspace)    */

    void       *workspace;
    size_t      workspace_bytes;

    void       *ev_main_begin;  /* optional hipEvent_t around the error kernel      */
    void       *ev_main_end;
} lowram_rank_args;

int    lowram_rank_residuals(const lowram_rank_args *args, void *stream);
size_t lowram_rank_workspace_size(const lowram_rank_args *args);

/*
 * Fused prefill ranking: the same residual store as lowram_rank_residuals,
 * with V_hat computed in the library from the cache's own parameters instead
 * of read from memory (explainer, mechanism paragraph: the value predictor
 * applied to the reconstructed keys; three-details paragraph: per-head
 * predictors and ranking by error; project site, Figure 3: keys from a factor
 * shared by a group of layers times a per-layer factor). For slice (layer) l,
 * KV head h and token t:
 *   k       = a[l / group][t] . b_l[l][h*d .. h*d+d)^T       (row vectors)
 *   V_hat   = k W_lin^T + gelu(k W1^T + b1) W2^T + b2        (weights output-major)
 *   e_t, I, R, ptr as for lowram_rank_residuals with this V_hat.
 * V_hat is evaluated in bf16 MFMA products with fp32 accumulation: k and the
 * hidden activations are rounded to bf16 before the next product, the GELU is
 * the float32 tail evaluation of the decode kernel, and V_hat is fp32. It is
 * computed twice (for every token, then again for the chosen ones) by the
 * same instructions, so R uses bit-for-bit the V_hat that was ranked; pass a
 * v_hat buffer to receive that fp32 V_hat for every token.
 * Requirements: head_dim 128, block_size 64, rank % 64 == 0, mlp_hidden % 64
 * == 0, act_dtype BF16, T * rank * 2 < 2^31 and T * n_kv_heads * head_dim * 2
 * < 2^31 (32-bit buffer offsets into A and V). All tensors caller-owned device
 * memory, 16-byte aligned (err 8, index/scale 4).
 */
typedef struct lowram_prefill_args {
    int32_t n_slices;           /* Lr layers                                          */
    int32_t group;              /* layers per shared key factor: slice l uses a[l/group] */
    int32_t ctx_len, n_kv_heads, head_dim, rank, mlp_hidden, block_size, n_res;
    int32_t act_dtype;          /* BF16: a, b_l, weights, biases and v                */
    int32_t res_dtype;          /* F32 | BF16 | I8 | I2                               */

    const void *a;              /* [ceil(Lr/group), T, r]                             */
    const void *b_l;            /* [Lr, Hkv*d, r]                                     */
    const void *w_lin;          /* [Lr, Hkv, d, d]                                    */
    const void *w1;             /* [Lr, Hkv, h, d]                                    */
    const void *b1;             /* [Lr, Hkv, h] or NULL (zero)                        */
    const void *w2;             /* [Lr, Hkv, d, h]                                    */
    const void *b2;             /* [Lr, Hkv, d] or NULL (zero)                        */
    const void *v;              /* [Lr, T, Hkv, d] true values                        */

    int32_t    *res_idx;        /* [Lr, Hkv, k]      (may be NULL when k == 0)        */
    void       *res_val;        /* [Lr, Hkv, k, d]  res_dtype, I2: [.., d/4] bytes    */
    float      *res_scale;      /* [Lr, Hkv, k]  I8 / I2 only, else NULL              */
    int32_t    *res_blk_ptr;    /* [Lr, Hkv, nb+1]                                    */
    double     *err;            /* [Lr, Hkv, T] or NULL (then kept in workspace)      */
    float      *v_hat;          /* [Lr, T, Hkv, d] fp32 copy of V_hat, or NULL        */

    void       *workspace;
    size_t      workspace_bytes;

    void       *ev_main_begin;  /* optional hipEvent_t around the all-token pass      */
    void       *ev_main_end;
} lowram_prefill_args;

int    lowram_prefill_rank(const lowram_prefill_args *args, void *stream);
size_t lowram_prefill_workspace_size(const lowram_prefill_args *args);

/*
 * Cross-layer key factors of n_batch independent layer groups (project site,
 * Figure 3: K ~ A . B with A shared by a group of adjacent layers and a
 * smaller factor per layer; explainer, keys paragraph: xKV, one low-rank basis
 * for adjacent layers). With C = [K_1 | ... | K_G] (T x n, n = G D) and its
 * Gram matrix M = C^T C, randomized subspace iteration (Halko, Martinsson and
 * Tropp, "Finding structure with randomness", SIAM Review 2011, Algorithm 4.4)
 * from the caller's draw omega:
 *   X_0 = omega,  X_i = orth(M X_{i-1}) for i = 1 .. n_iter,
 *   A = C X,      B_l = (rows l D .. l D + D - 1 of X)^T,
 * so K_l ~ A B_l with the reconstruction C X X^T, which approaches the best
 * rank-r fit (the truncated SVD) as n_iter grows. orth is CholeskyQR applied
 * twice, M is accumulated in float32 per token chunk and summed in binary64,
 * the iteration runs in binary64, A = C X in bf16 products with float32 sums.
 * A Cholesky pivot at or below r 2^-52 times the largest diagonal entry drops
 * that basis column (zero column of X, A and B_l): the block is numerically
 * rank deficient there (e.g. fewer tokens than the rank, or zero keys), and
 * the dropped direction carries none of the keys' energy.
 *
 * Shapes (Bt = n_batch problems, e.g. the layer groups of a model, or of
 * several sequences, all of length T): keys [Bt, G, T, D] bf16 (layer-major,
 * each layer's keys [T, D] with D = Hkv d); omega [n, r] binary64, one draw
 * shared by every problem, e.g. standard normal; outputs a [Bt, T, r] bf16
 * (the factor the decode step reads as this group's A for every layer of it)
 * and b_l [Bt, G, D, r] bf16 (layer l's B_l output-major, as the decode step
 * reads it); basis [Bt, n, r] binary64 (X) if not NULL. Limits: G <= 16, D a
 * multiple of 256, n <= 16384, r a multiple of 64 in [64, min(1024, n)],
 * n_iter in [1, 16], T D 2 < 2^31. Buffers are caller-owned device memory,
 * 16-byte aligned; the call allocates nothing. The problems run side by side
 * in every kernel (the r x r Cholesky factorisations, one workgroup each,
 * then overlap).
 */
typedef struct lowram_xkv_args {
    int32_t n_batch;            /* Bt, independent problems                         */
    int32_t n_layers;           /* G, layers sharing A                              */
    int32_t ctx_len;            /* T                                                */
    int32_t width;              /* D = n_kv_heads * head_dim                        */
    int32_t rank;               /* r                                                */
    int32_t n_iter;             /* subspace iterations                              */

    const void   *keys;         /* [Bt, G, T, D] bf16                               */
    const double *omega;        /* [G*D, r] starting block                          */

    void         *a;            /* [Bt, T, r] bf16 out                              */
    void         *b_l;          /* [Bt, G, D, r] bf16 out                           */
    double       *basis;        /* [Bt, G*D, r] out, or NULL                        */

    void         *workspace;    /* >= lowram_xkv_workspace_size bytes               */
    size_t        workspace_bytes;

    void         *ev_main_begin; /* optional hipEvent_t around the Gram MFMA kernel */
    void         *ev_main_end;
} lowram_xkv_args;

int    lowram_xkv_factorize(const lowram_xkv_args *args, void *stream);
size_t lowram_xkv_workspace_size(const lowram_xkv_args *args);

/*
 * Pseudoinverse start of the per-head linear value map (explainer, Slim
 * Attention paragraph: the predictor starts from the best linear guess the
 * projections allow). For each of n_maps problems (e.g. layer x KV head),
 * with row vectors k = x W_K and v = x W_V over the model width:
 *   W_lin = pinv(W_K) W_V = (W_K^T W_K)^-1 W_K^T W_V,
 * computed in binary64 (Cholesky of W_K^T W_K; a pivot at or below
 * d 2^-52 times the largest diagonal entry drops that direction, which is
 * the pseudoinverse on a rank-deficient W_K's range). Output w_lin is
 * output-major [d, d] = W_lin^T, the layout the decode step reads, rounded to
 * bf16 once; w_lin64 the same in binary64 if not NULL.
 * Shapes: w_k, w_v [P, hidden, d] bf16; hidden in [d, 65536], d = 128.
 */
typedef struct lowram_pinv_args {
    int32_t n_maps;             /* P                                                */
    int32_t hidden;             /* model width                                      */
    int32_t head_dim;           /* d                                                */
    const void *w_k;            /* [P, hidden, d] bf16                              */
    const void *w_v;            /* [P, hidden, d] bf16                              */
    void       *w_lin;          /* [P, d, d] bf16 out                               */
    double     *w_lin64;        /* [P, d, d] out, or NULL                           */
    void       *workspace;
    size_t      workspace_bytes;
} lowram_pinv_args;

int    lowram_pinv_value_map(const lowram_pinv_args *args, void *stream);
size_t lowram_pinv_workspace_size(const lowram_pinv_args *args);

/*
 * Test-time fit of the predictor's nonlinear branch (explainer, mechanism
 * paragraph: a small two-layer network per head fitted during prefill to this
 * context; Slim Attention paragraph: it learns what the linear map leaves;
 * cost paragraph: a number of gradient steps per context). The pages name
 * neither loss nor optimiser; this library takes the mean over tokens of the
 * squared L2 value error,
 *   L = (1/T) sum_t || k_t W_lin + gelu(k_t W1 + b1) W2 + b2 - v_t ||^2,
 * and n_steps of plain gradient descent theta <- theta - lr dL/dtheta on
 * W1, b1, W2, b2 (W_lin fixed), for every (layer, KV head) at once. Products
 * in bf16 with float32 sums (keys, values, the bf16 copies of the weights and
 * the intermediate activations and gradients are bf16); the parameters are
 * float32 masters updated in place. gelu is the exact erf form (the kernels
 * evaluate it, and its derivative, from a fitted normal tail to within 6e-5).
 * losses[l, h, i] is L before step i and losses[l, h, n_steps] after the
 * last step; with losses NULL no loss is written and the loss-only forward
 * pass after the last step is skipped (the parameters are the same).
 * Shapes (L layers, T tokens, Hkv heads, d = 128, h = mlp_hidden, a multiple
 * of 128 in [128, 1024]): keys [L, T, Hkv*d] bf16 (e.g. A B_l), v [L, T, Hkv,
 * d] bf16, w_lin [L, Hkv, d, d] bf16 output-major; w1 [L, Hkv, h, d], b1
 * [L, Hkv, h], w2 [L, Hkv, d, h], b2 [L, Hkv, d] float32 in/out (output-major,
 * as the decode step reads them after a bf16 conversion). T Hkv d 2 < 2^31.
 */
typedef struct lowram_fit_args {
    int32_t n_layers, ctx_len, n_kv_heads, head_dim, mlp_hidden, n_steps;
    float   lr;
    const void *keys;           /* [L, T, Hkv*d] bf16                               */
    const void *v;              /* [L, T, Hkv, d] bf16                              */
    const void *w_lin;          /* [L, Hkv, d, d] bf16                              */
    float      *w1;             /* [L, Hkv, h, d] float32 in/out                    */
    float      *b1;             /* [L, Hkv, h]                                      */
    float      *w2;             /* [L, Hkv, d, h]                                   */
    float      *b2;             /* [L, Hkv, d]                                      */
    float      *losses;         /* [L, Hkv, n_steps + 1] out, or NULL               */
    void       *workspace;
    size_t      workspace_bytes;
    void       *ev_main_begin;  /* optional hipEvent_t around the gradient steps    */
    void       *ev_main_end;
} lowram_fit_args;

int    lowram_fit_predictor(const lowram_fit_args *args, void *stream);
size_t lowram_fit_workspace_size(const lowram_fit_args *args);

/* Static description of a status code. */
const char *lowram_status_string(int status);

/* Message for the last failed call on this thread ("" if none). */
const char *lowram_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LOWRAM_H */
