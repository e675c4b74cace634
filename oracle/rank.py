"""Oracle for the prefill-side residual ranking (float64, plain definitions).

Test infrastructure only (see the package docstring). The paper page's
Abstract and the explainer's mechanism and three-details paragraphs say that
exact residuals are kept for the tokens the per-head predictor reconstructs
worst, ranked by error, at a fixed budget. Readings taken where the pages are
silent: the error is the squared L2 norm of V - V_hat summed in index order in
binary64 (no fused multiply-add, no square root, so the order equals the
norm's); ties go to the lower token index; stored residuals are in ascending
token order with a block CSR over them.
"""
import numpy as np

_BF16_MIN_EXP = -133      # exponent of the smallest bf16 subnormal quantum
_BF16_SIG_BITS = 8        # significant bits of a normal bf16 (7 stored + 1)


def residual_error(v, v_hat):
    """e = sum_i (v_i - v_hat_i)^2 over the last axis, accumulated left to
    right from 0 with one binary64 rounding per multiply and per add.

    The difference of two stored values is exact in binary64 for bf16 and
    float32 inputs. numpy performs each elementwise operation separately
    (no contraction), so the loop below is the stated operation sequence.
    """
    delta = np.asarray(v).astype(np.float64) - np.asarray(v_hat).astype(np.float64)
    e = np.zeros(delta.shape[:-1])
    for i in range(delta.shape[-1]):
        e = e + delta[..., i] * delta[..., i]
    return e


def select_worst(err, k):
    """Indices of the k largest errors, ordered by (error desc, index asc),
    returned in ascending index order."""
    err = np.asarray(err, np.float64)
    order = np.lexsort((np.arange(err.size), -err))
    return np.sort(order[:k]).astype(np.int64)


def round_bf16(x):
    """Round binary64 values to the nearest bfloat16, ties to even, in one
    step (no intermediate float32 rounding). bfloat16 keeps 8 significant bits
    down to 2**-126 and a fixed quantum of 2**-133 below; results at or above
    2**128 overflow to infinity."""
    x = np.asarray(x, np.float64)
    _, e = np.frexp(x)
    q = np.maximum(e - _BF16_SIG_BITS, _BF16_MIN_EXP)
    r = np.ldexp(np.rint(np.ldexp(x, -q)), q)
    return np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, x), r)


def round_f32(x):
    """Round binary64 values to the nearest float32, ties to even."""
    return np.asarray(x, np.float64).astype(np.float32).astype(np.float64)


def quantize_int8_rows(r):
    """Symmetric per-row int8 code: s = float32(max|r| / 127) (binary64
    division, one rounding to float32), q = clamp(rint(r / s), -127, 127) in
    binary64 with ties to even. An all-zero row gets s = 0 and q = 0.
    Returns (q int8 [..., d], s float32 [...])."""
    r = np.asarray(r, np.float64)
    amax = np.max(np.abs(r), axis=-1)
    s = (amax / 127.0).astype(np.float32)
    s64 = s.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s64 > 0, np.rint(r / np.where(s64 > 0, s64, 1.0)), 0.0)
    return np.clip(qf, -127, 127).astype(np.int8), s


def dequantize_int8_rows(q, s):
    """Exact value of an int8 row code: q * s in binary64."""
    return np.asarray(q).astype(np.float64) * np.asarray(s).astype(np.float64)[..., None]


def quantize_i2_rows(r):
    """Per-row 2-bit code (the explainer's comparison table names 2-bit
    residuals without a codec; the reading here is the symmetric mid-rise
    4-level quantizer): levels (q - 1.5) s for q in 0..3 with
    s = float32(max|r| / 1.5) (binary64 division, one rounding to float32),
    q = clamp(rint(r / s + 1.5), 0, 3) in binary64 (division, then addition,
    ties to even). An all-zero row gets s = 0 and q = 2 (level 0).
    Returns (q uint8 [..., d] in 0..3, s float32 [...])."""
    r = np.asarray(r, np.float64)
    amax = np.max(np.abs(r), axis=-1)
    s = (amax / 1.5).astype(np.float32)
    s64 = s.astype(np.float64)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        qf = np.where(s64 > 0, np.rint(r / np.where(s64 > 0, s64, 1.0) + 1.5), 2.0)
    return np.clip(qf, 0, 3).astype(np.uint8), s


def dequantize_i2_rows(q, s):
    """Exact value of a 2-bit row code: (q - 1.5) s in binary64."""
    return (np.asarray(q).astype(np.float64) - 1.5) * np.asarray(s).astype(np.float64)[..., None]


def pack_i2(q):
    """Four 2-bit codes per byte: element i in bits 2(i mod 4) .. 2(i mod 4)+1
    of byte i // 4. q [..., d] with d a multiple of 4 -> uint8 [..., d/4]."""
    q = np.asarray(q).astype(np.uint8)
    q4 = q.reshape(q.shape[:-1] + (q.shape[-1] // 4, 4))
    return (q4[..., 0] | (q4[..., 1] << 2) | (q4[..., 2] << 4) | (q4[..., 3] << 6)).astype(np.uint8)


def unpack_i2(b):
    """Inverse of pack_i2: uint8 [..., d/4] -> codes uint8 [..., d]."""
    b = np.asarray(b).astype(np.uint8)
    return np.stack([(b >> (2 * j)) & 3 for j in range(4)], axis=-1).reshape(b.shape[:-1] + (4 * b.shape[-1],))


def block_ptr(idx, n_tokens, block):
    """Block CSR over ascending residual indices: ptr[i] = #{t in idx : t < i*block}
    for i = 0..nb, nb = ceil(T/block); so block i owns slots ptr[i]..ptr[i+1]."""
    idx = np.asarray(idx, np.int64)
    nb = -(-n_tokens // block)
    return np.array([int(np.count_nonzero(idx < min(i * block, n_tokens))) if i < nb
                     else int(idx.size) for i in range(nb + 1)], dtype=np.int64)


def rank_residuals(v, v_hat, k, block, res_dtype):
    """Residual store for each slice l and KV head h of V, V_hat [Lr, T, Hkv, d].

    Per (l, h): errors over all T tokens; the k worst tokens (ties to the
    lower index) in ascending order; residuals R = V - V_hat at those tokens
    (exact in binary64, then stored as ``res_dtype``: 'f32', 'bf16', 'i8', or
    'i2' packed four codes per byte);
    and the block CSR. Returns a dict with idx [Lr, Hkv, k], val [Lr, Hkv, k, d]
    (float64 value of the stored element, or int8 codes for 'i8'), scale
    [Lr, Hkv, k] float32 ('i8' only), ptr [Lr, Hkv, nb+1], err [Lr, Hkv, T].
    """
    v = np.asarray(v)
    v_hat = np.asarray(v_hat)
    n_sl, n_tok, n_kv, d = v.shape
    nb = -(-n_tok // block)
    idx = np.zeros((n_sl, n_kv, k), np.int64)
    ptr = np.zeros((n_sl, n_kv, nb + 1), np.int64)
    err = np.zeros((n_sl, n_kv, n_tok))
    if res_dtype == "i2":
        val = np.zeros((n_sl, n_kv, k, d // 4), np.uint8)
    else:
        val = np.zeros((n_sl, n_kv, k, d), np.int8 if res_dtype == "i8" else np.float64)
    scale = np.zeros((n_sl, n_kv, k), np.float32) if res_dtype in ("i8", "i2") else None
    for sl in range(n_sl):
        for h in range(n_kv):
            e = residual_error(v[sl, :, h, :], v_hat[sl, :, h, :])
            err[sl, h] = e
            sel = select_worst(e, k)
            idx[sl, h] = sel
            ptr[sl, h] = block_ptr(sel, n_tok, block)
            r = v[sl, sel, h, :].astype(np.float64) - v_hat[sl, sel, h, :].astype(np.float64)
            if res_dtype == "i8":
                val[sl, h], scale[sl, h] = quantize_int8_rows(r)
            elif res_dtype == "i2":
                q2, scale[sl, h] = quantize_i2_rows(r)
                val[sl, h] = pack_i2(q2)
            elif res_dtype == "bf16":
                val[sl, h] = round_bf16(r)
            elif res_dtype == "f32":
                val[sl, h] = round_f32(r)
            else:
                raise ValueError(res_dtype)
    return {"idx": idx, "val": val, "scale": scale, "ptr": ptr, "err": err}
