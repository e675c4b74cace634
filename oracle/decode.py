"""Oracle for one decode step of one layer (float64, plain definitions).

Test infrastructure only (see the package docstring). Layout conventions are
those of the compressed cache the library consumes: every weight matrix is
stored output-major, like ``torch.nn.Linear.weight`` ([out_features,
in_features]); the oracle transposes explicitly where the mathematics uses the
row-vector convention ``y = x . W``.
"""
import math

import numpy as np
from scipy.special import erf

from .rank import dequantize_i2_rows, unpack_i2


def gelu(x):
    """GELU in its exact error-function form, 0.5*x*(1 + erf(x/sqrt(2))).

    The pages call the predictor's second branch a small two-layer nonlinear
    network without naming the activation (explainer, mechanism and Slim
    Attention paragraphs); the exact erf form is the reading taken here.
    """
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def _f64(x, scale=None):
    """Exact upcast of a stored tensor; int8 rows times their float32 scale."""
    y = np.asarray(x).astype(np.float64)
    if scale is not None:
        y = y * np.asarray(scale).astype(np.float64)[..., None]
    return y


def _residual_rows(val, scale):
    """Stored residual rows as float64: uint8 rows are 2-bit codes packed four
    per byte ((q - 1.5) s), int8 rows are q s, float rows are exact."""
    val = np.asarray(val)
    if val.dtype == np.uint8:
        return dequantize_i2_rows(unpack_i2(val), scale)
    return _f64(val, scale)


def reconstruct_keys(a_rows, bl):
    """Keys of one layer from the cross-layer factors: K_l = A . B_l.

    project site, Figure 3: a factor shared by a group of layers times a
    per-layer factor; explainer, keys paragraph (xKV basis shared by adjacent
    layers). ``a_rows`` is [n, r]; ``bl`` is B_l stored output-major
    [Hkv*d, r], so B_l = bl^T.
    """
    return np.asarray(a_rows, np.float64) @ np.asarray(bl, np.float64).T


def predict_values(k_h, w_lin, w1, w2, b1=None, b2=None):
    """Per-KV-head value predictor on the keys of that head.

    v_hat = k . W_lin + gelu(k . W1 + b1) . W2 + b2 (row vectors), with the
    linear map from the Slim Attention paragraph of the explainer
    (pseudoinverse start) plus the small two-layer nonlinear branch of its
    mechanism paragraph; one predictor per head (three-details paragraph).
    Stored output-major: w_lin [d, d] = W_lin^T, w1 [h, d] = W1^T,
    w2 [d, h] = W2^T. Missing biases are zero.
    """
    k_h = np.asarray(k_h, np.float64)
    pre = k_h @ np.asarray(w1, np.float64).T
    if b1 is not None:
        pre = pre + np.asarray(b1, np.float64)
    v = k_h @ np.asarray(w_lin, np.float64).T + gelu(pre) @ np.asarray(w2, np.float64).T
    if b2 is not None:
        v = v + np.asarray(b2, np.float64)
    return v


def attended_blocks(n_tokens, block, sel=None, keep=None):
    """Blocks a decode step attends: the selected ones (all if no selection)
    that the eviction mask keeps.

    explainer, prefill/decode paragraph: only the chunks the current query
    selects are rebuilt; paper page, Abstract: a selected subset per step and
    composition with eviction. Blocks are [i*block, min((i+1)*block, T)).
    Selection entries outside [0, nb) are padding (a row of a batch that
    selects fewer blocks than the widest row) and name no block.
    """
    nb = -(-n_tokens // block)
    cand = range(nb) if sel is None else [int(i) for i in sel if 0 <= int(i) < nb]
    return [i for i in cand if keep is None or bool(keep[i])]


def attention(qv, keys, vals):
    """Softmax attention of one query over given keys and values, scale
    1/sqrt(d), no positional term or mask (the cached tokens all precede the
    query). The explainer's mechanism paragraph feeds the rebuilt pairs to
    ordinary attention."""
    qv = np.asarray(qv, np.float64)
    s = keys @ qv / math.sqrt(qv.shape[0])
    p = np.exp(s - s.max())
    p = p / p.sum()
    return p @ vals


def decode_batch_element(q, a, bl, w_lin, w1, w2, res_idx, res_val, *, block,
                         a_scale=None, b1=None, b2=None, res_scale=None,
                         sel=None, keep=None, win_k=None, win_v=None):
    """One layer's decode output for one sequence.

    Shapes: q [Hq, d]; a [T, r] (int8 codes when ``a_scale`` [T] is given);
    bl [Hkv*d, r]; w_lin [Hkv, d, d]; w1 [Hkv, h, d]; w2 [Hkv, d, h];
    b1 [Hkv, h] | None; b2 [Hkv, d] | None; res_idx [Hkv, k] ascending token
    indices; res_val [Hkv, k, d] (int8 codes when ``res_scale`` [Hkv, k] is
    given); sel [n_sel] | None; keep [nb] | None; win_k, win_v [w, Hkv*d] |
    None (exact recent tokens).

    Steps: attended tokens (``attended_blocks``); keys rebuilt from the factors;
    per KV head, values predicted from that head's keys and the stored
    residual added where the token has one (explainer, mechanism paragraph);
    the exact window tokens joined to them (explainer, prefill/decode
    paragraph: new tokens stored exactly); ordinary softmax attention for each
    query head j on KV head j // (Hq/Hkv).

    Returns (out [Hq, d] float64, stats [Hkv, 2] int64) with stats[h] =
    (attended tokens including the window, residuals applied). With nothing
    to attend the output row is zero.
    """
    q = np.asarray(q, np.float64)
    n_q, d = q.shape
    n_tok = np.asarray(a).shape[0]
    n_kv = np.asarray(bl).shape[0] // d
    g = n_q // n_kv
    blocks = attended_blocks(n_tok, block, sel, keep)
    tau = np.array([t for i in blocks for t in range(i * block, min((i + 1) * block, n_tok))],
                   dtype=np.int64)
    pos = np.full(n_tok, -1, dtype=np.int64)
    pos[tau] = np.arange(tau.size)

    a_rows = _f64(np.asarray(a)[tau], None if a_scale is None else np.asarray(a_scale)[tau])
    keys_all = reconstruct_keys(a_rows, bl)
    n_win = 0 if win_k is None else np.asarray(win_k).shape[0]

    out = np.zeros((n_q, d))
    stats = np.zeros((n_kv, 2), dtype=np.int64)
    for h in range(n_kv):
        k_h = keys_all[:, h * d:(h + 1) * d]
        v_h = predict_values(k_h, w_lin[h], w1[h], w2[h],
                             None if b1 is None else b1[h], None if b2 is None else b2[h])
        rv = _residual_rows(res_val[h], None if res_scale is None else res_scale[h])
        rows = pos[np.asarray(res_idx[h], dtype=np.int64)] if tau.size else np.full(len(res_idx[h]), -1)
        hit = rows >= 0
        v_h[rows[hit]] += rv[hit]
        if n_win:
            k_h = np.concatenate([k_h, _f64(win_k)[:, h * d:(h + 1) * d]])
            v_h = np.concatenate([v_h, _f64(win_v)[:, h * d:(h + 1) * d]])
        stats[h] = (tau.size + n_win, int(hit.sum()))
        if k_h.shape[0] == 0:
            continue
        for j in range(h * g, (h + 1) * g):
            out[j] = attention(q[j], k_h, v_h)
    return out, stats


def decode_step(batch):
    """``decode_batch_element`` over a batch. ``batch`` maps argument names to
    arrays with a leading batch axis (``block`` is an int; optional entries
    may be missing or None; ``win_len`` cuts the window buffers)."""
    n_b = np.asarray(batch["q"]).shape[0]
    outs, stats = [], []
    w = batch.get("win_len", 0) or 0
    for b in range(n_b):
        def opt(name):
            v = batch.get(name)
            return None if v is None else v[b]
        o, s = decode_batch_element(
            batch["q"][b], batch["a"][b], batch["bl"][b], batch["w_lin"][b],
            batch["w1"][b], batch["w2"][b], batch["res_idx"][b], batch["res_val"][b],
            block=batch["block"], a_scale=opt("a_scale"), b1=opt("b1"), b2=opt("b2"),
            res_scale=opt("res_scale"), sel=opt("sel"), keep=opt("keep"),
            win_k=None if w == 0 else batch["win_k"][b][:w],
            win_v=None if w == 0 else batch["win_v"][b][:w])
        outs.append(o)
        stats.append(s)
    return np.stack(outs), np.stack(stats)
