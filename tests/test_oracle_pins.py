"""Pins for the float64 oracle: each check ties an oracle function to
something other than itself (a closed form, a library routine it does not
call, a printed number, or a pure-Python brute force)."""
import itertools
import json
import math
import os
import random
import struct

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _softmax_attend(qv, keys, vals):
    # Independent plain attention: lists of python floats.
    d = len(qv)
    s = [sum(qv[i] * k[i] for i in range(d)) / math.sqrt(d) for k in keys]
    m = max(s)
    p = [math.exp(x - m) for x in s]
    z = sum(p)
    return [sum(p[t] * vals[t][i] for t in range(len(keys))) / z for i in range(len(vals[0]))]


# ---------------------------------------------------------------- Slim Attention
def test_slim_attention_exact_recovery():
    """explainer, Slim Attention paragraph: with a square invertible key
    projection, values follow from keys exactly through pinv(W_K) W_V. Keys
    are x W_K (the factor A is x itself, B_l stacks the heads' W_K), the
    nonlinear branch is zero and no residuals are stored; the decode must then
    equal attention over the true (x W_K, x W_V)."""
    rng = np.random.default_rng(1)
    n_tok, d, n_kv, n_q, hid = 150, 16, 2, 4, 8
    x = rng.standard_normal((n_tok, d))
    w_k = [rng.standard_normal((d, d)) + 3 * np.eye(d) for _ in range(n_kv)]
    w_v = [rng.standard_normal((d, d)) for _ in range(n_kv)]
    bl = np.concatenate([w.T for w in w_k], axis=0)            # [Hkv*d, r=d], output-major
    w_lin = np.stack([oracle.pinv_value_map(w_k[h], w_v[h]) for h in range(n_kv)])
    for h in range(n_kv):
        v_hat = oracle.predict_values(x @ w_k[h], w_lin[h], np.zeros((hid, d)), np.zeros((d, hid)))
        np.testing.assert_allclose(v_hat, x @ w_v[h], rtol=0, atol=1e-10)
    q = rng.standard_normal((n_q, d))
    out, stats = oracle.decode_batch_element(
        q, x, bl, w_lin, np.zeros((n_kv, hid, d)), np.zeros((n_kv, d, hid)),
        np.zeros((n_kv, 0), np.int64), np.zeros((n_kv, 0, d)), block=64)
    for j in range(n_q):
        h = j // (n_q // n_kv)
        ref = _softmax_attend(list(q[j]), (x @ w_k[h]).tolist(), (x @ w_v[h]).tolist())
        np.testing.assert_allclose(out[j], ref, rtol=0, atol=1e-10)
    assert stats.tolist() == [[n_tok, 0]] * n_kv


# --------------------------------------------------------- exact V with k = T
@pytest.mark.parametrize("with_window", [False, True])
def test_residuals_everywhere_give_exact_values(with_window):
    """explainer, mechanism paragraph: value = prediction + residual where one
    exists. With a residual for every token equal to V - V_hat the decode must
    return attention over the true values, whatever the predictor."""
    rng = np.random.default_rng(2)
    n_tok, d, r, n_kv, n_q, hid, blk = 200, 8, 6, 2, 4, 5, 64
    x = rng.standard_normal((n_tok, r))
    w_k = [rng.standard_normal((r, d)) for _ in range(n_kv)]
    bl = np.concatenate([w.T for w in w_k], axis=0)
    v_true = rng.standard_normal((n_kv, n_tok, d))
    w_lin = rng.standard_normal((n_kv, d, d))
    w1 = rng.standard_normal((n_kv, hid, d))
    w2 = rng.standard_normal((n_kv, d, hid))
    b1 = rng.standard_normal((n_kv, hid))
    b2 = rng.standard_normal((n_kv, d))
    res = np.stack([v_true[h] - oracle.predict_values(x @ w_k[h], w_lin[h], w1[h], w2[h], b1[h], b2[h])
                    for h in range(n_kv)])
    idx = np.tile(np.arange(n_tok), (n_kv, 1))
    sel = [0, 2, 3]
    wk = rng.standard_normal((3, n_kv * d)) if with_window else None
    wv = rng.standard_normal((3, n_kv * d)) if with_window else None
    q = rng.standard_normal((n_q, d))
    out, stats = oracle.decode_batch_element(q, x, bl, w_lin, w1, w2, idx, res, block=blk,
                                             b1=b1, b2=b2, sel=sel, win_k=wk, win_v=wv)
    tau = [t for i in sel for t in range(i * blk, min((i + 1) * blk, n_tok))]
    for j in range(n_q):
        h = j // 2
        keys = (x[tau] @ w_k[h]).tolist()
        vals = v_true[h][tau].tolist()
        if with_window:
            keys += wk[:, h * d:(h + 1) * d].tolist()
            vals += wv[:, h * d:(h + 1) * d].tolist()
        np.testing.assert_allclose(out[j], _softmax_attend(list(q[j]), keys, vals), rtol=0, atol=1e-10)
    assert stats[:, 1].tolist() == [len(tau)] * n_kv
    assert stats[:, 0].tolist() == [len(tau) + (3 if with_window else 0)] * n_kv


# ------------------------------------------------- factor layout: exact K at full rank
def test_xkv_full_rank_exact_and_eckart_young_tail():
    """project site, Figure 3: K_l ~ A . B_l with A shared by the group. At
    full rank the factors rebuild every layer's keys exactly; below it the
    Frobenius error is the tail of the singular values (Eckart-Young), here
    taken from the eigenvalues of the Gram matrix, a different routine."""
    rng = np.random.default_rng(3)
    n_tok, width, n_layers = 80, 16, 4
    keys = [rng.standard_normal((n_tok, width)) @ rng.standard_normal((width, width)) for _ in range(n_layers)]
    a, bls, _ = oracle.xkv_factorize(keys, n_layers * width)
    for l in range(n_layers):
        np.testing.assert_allclose(oracle.reconstruct_keys(a, bls[l]), keys[l], rtol=0, atol=1e-10)
    cat = np.concatenate(keys, axis=1)
    eig = np.sort(np.linalg.eigvalsh(cat.T @ cat))[::-1]
    for rank in (5, 20, 40):
        a, bls, _ = oracle.xkv_factorize(keys, rank)
        rec = np.concatenate([oracle.reconstruct_keys(a, b) for b in bls], axis=1)
        tail = math.sqrt(max(0.0, float(np.sum(eig[rank:]))))
        assert abs(np.linalg.norm(cat - rec) - tail) < 1e-8 * max(1.0, tail)


def _xkv_case(rng, n_tok, width, n_layers, decay, floor):
    """Keys whose concatenation has a decaying spectrum: Z diag(s) W with
    s_i = exp(-i / decay) + floor."""
    m = n_layers * width
    z = rng.standard_normal((n_tok, m)) * (np.exp(-np.arange(m) / decay) + floor)
    cat = z @ rng.standard_normal((m, m)) / math.sqrt(m)
    return [cat[:, l * width:(l + 1) * width] for l in range(n_layers)], cat


def _rebuild(a, bls):
    return np.concatenate([oracle.reconstruct_keys(a, b) for b in bls], axis=1)


def test_xkv_iteration_exact_cases():
    """Full rank (r = n), keys of exact rank r, and fewer tokens than the rank:
    in each the span of M X holds the whole row space of C after one step, so
    the factors rebuild every layer exactly; the basis is orthonormal and A is
    C times it."""
    rng = np.random.default_rng(40)
    keys, cat = _xkv_case(rng, 90, 8, 3, 5.0, 0.1)
    a, bls, x = oracle.xkv_subspace_iteration(keys, 24, rng.standard_normal((24, 24)), 1)
    np.testing.assert_allclose(_rebuild(a, bls), cat, atol=1e-10)
    low = rng.standard_normal((90, 6)) @ rng.standard_normal((6, 24))
    keys = [low[:, l * 8:(l + 1) * 8] for l in range(3)]
    a, bls, x = oracle.xkv_subspace_iteration(keys, 6, rng.standard_normal((24, 6)), 1)
    np.testing.assert_allclose(_rebuild(a, bls), low, atol=1e-9)
    np.testing.assert_allclose(x.T @ x, np.eye(6), atol=1e-12)
    np.testing.assert_allclose(a, low @ x, atol=1e-12)
    short = rng.standard_normal((5, 24))                     # T = 5 < r = 8
    keys = [short[:, l * 8:(l + 1) * 8] for l in range(3)]
    a, bls, _ = oracle.xkv_subspace_iteration(keys, 8, rng.standard_normal((24, 8)), 2)
    np.testing.assert_allclose(_rebuild(a, bls), short, atol=1e-10)


def test_xkv_iteration_reaches_the_truncated_svd_across_a_gap():
    """Rank-r signal plus noise 1e-6 below it: the iteration converges to the
    truncated SVD (the plain definition, pinned above) geometrically in the
    squared singular-value ratio; three steps match it to 1e-9."""
    rng = np.random.default_rng(41)
    sig = rng.standard_normal((200, 10)) @ rng.standard_normal((10, 48))
    cat = sig + 1e-6 * rng.standard_normal((200, 48))
    keys = [cat[:, l * 16:(l + 1) * 16] for l in range(3)]
    a, bls, _ = oracle.xkv_factorize(keys, 10)
    best = _rebuild(a, bls)
    a, bls, _ = oracle.xkv_subspace_iteration(keys, 10, rng.standard_normal((48, 10)), 3)
    assert np.linalg.norm(_rebuild(a, bls) - best) <= 1e-9 * np.linalg.norm(best)


def test_xkv_iteration_eckart_young_bounds_and_basis_independence():
    """On a smoothly decaying spectrum the error never beats the singular-value
    tail (Eckart-Young), shrinks with every step, and is within 5% of it after
    three; the result depends on the span only: an orthonormalisation by
    Cholesky (X = Y L^-T, L L^T = Y^T Y) instead of QR gives the same factors'
    product."""
    rng = np.random.default_rng(42)
    keys, cat = _xkv_case(rng, 600, 32, 4, 20.0, 0.02)
    tail = math.sqrt(float(np.sum(np.linalg.svd(cat, compute_uv=False)[24:] ** 2)))
    om = rng.standard_normal((128, 24))
    errs = []
    for q in (1, 2, 3):
        a, bls, _ = oracle.xkv_subspace_iteration(keys, 24, om, q)
        errs.append(np.linalg.norm(cat - _rebuild(a, bls)))
    assert tail <= errs[2] < errs[1] < errs[0] and errs[2] <= 1.05 * tail
    x = om
    m = cat.T @ cat
    for _ in range(3):
        y = m @ x
        x = np.linalg.solve(np.linalg.cholesky(y.T @ y), y.T).T
    np.testing.assert_allclose(cat @ x @ x.T, cat - (cat - _rebuild(a, bls)), rtol=0, atol=1e-9 * np.abs(cat).max())


# ---------------------------------------------------------- brute force, tiny
def _gelu_py(v):
    return 0.5 * v * (1.0 + math.erf(v / math.sqrt(2.0)))


def _brute_decode(q, a, a_scale, bl, w_lin, w1, b1, w2, b2, idx, rv, rs, sel, keep, wk, wv, blk):
    """Scalar-loop decode for one sequence, written from the definitions with
    python floats and math.erf; no numpy arithmetic."""
    n_q, d = len(q), len(q[0])
    n_tok, r = len(a), len(a[0])
    n_kv = len(bl) // d
    g = n_q // n_kv
    nb = (n_tok + blk - 1) // blk
    blocks = list(range(nb)) if sel is None else [i for i in sel if 0 <= i < nb]
    blocks = [i for i in blocks if keep is None or keep[i]]
    tau = [t for i in blocks for t in range(i * blk, min(i * blk + blk, n_tok))]
    out = [[0.0] * d for _ in range(n_q)]
    stats = []
    for h in range(n_kv):
        keys, vals = [], []
        napplied = 0
        for t in tau:
            arow = [a[t][c] * (1.0 if a_scale is None else a_scale[t]) for c in range(r)]
            k = [sum(arow[c] * bl[h * d + n][c] for c in range(r)) for n in range(d)]
            hidv = [sum(k[n] * w1[h][u][n] for n in range(d)) + (0.0 if b1 is None else b1[h][u])
                    for u in range(len(w1[h]))]
            gv = [_gelu_py(x) for x in hidv]
            v = [sum(k[n] * w_lin[h][o][n] for n in range(d)) + sum(gv[u] * w2[h][o][u] for u in range(len(gv)))
                 + (0.0 if b2 is None else b2[h][o]) for o in range(d)]
            for p, tt in enumerate(idx[h]):
                if tt == t:
                    sc = 1.0 if rs is None else rs[h][p]
                    v = [v[o] + rv[h][p][o] * sc for o in range(d)]
                    napplied += 1
            keys.append(k)
            vals.append(v)
        for u in range(len(wk)):
            keys.append(list(wk[u][h * d:(h + 1) * d]))
            vals.append(list(wv[u][h * d:(h + 1) * d]))
        stats.append([len(keys), napplied])
        if keys:
            for j in range(h * g, (h + 1) * g):
                out[j] = _softmax_attend(q[j], keys, vals)
    return out, stats


def _tiny_case(rng, n_tok, int8_a=False, int8_r=False, biases=True):
    d, r, n_kv, n_q, hid = 8, 4, 2, 4, 4
    case = dict(
        q=rng.standard_normal((n_q, d)),
        a=(rng.integers(-127, 128, (n_tok, r)).astype(np.int8) if int8_a else rng.standard_normal((n_tok, r))),
        a_scale=(rng.uniform(0.01, 0.02, n_tok).astype(np.float32) if int8_a else None),
        bl=rng.standard_normal((n_kv * d, r)),
        w_lin=rng.standard_normal((n_kv, d, d)) * 0.3,
        w1=rng.standard_normal((n_kv, hid, d)) * 0.5,
        b1=rng.standard_normal((n_kv, hid)) if biases else None,
        w2=rng.standard_normal((n_kv, d, hid)) * 0.5,
        b2=rng.standard_normal((n_kv, d)) if biases else None,
    )
    k = n_tok // 5
    case["idx"] = np.stack([np.sort(rng.choice(n_tok, k, replace=False)) for _ in range(n_kv)])
    if int8_r:
        case["rv"] = rng.integers(-127, 128, (n_kv, k, d)).astype(np.int8)
        case["rs"] = rng.uniform(0.001, 0.01, (n_kv, k)).astype(np.float32)
    else:
        case["rv"] = rng.standard_normal((n_kv, k, d)) * 0.1
        case["rs"] = None
    return case


def _run_both(case, sel, keep, n_win, rng):
    n_kv, d = case["w_lin"].shape[:2]
    wk = rng.standard_normal((n_win, n_kv * d))
    wv = rng.standard_normal((n_win, n_kv * d))
    got, gstats = oracle.decode_batch_element(
        case["q"], case["a"], case["bl"], case["w_lin"], case["w1"], case["w2"], case["idx"], case["rv"],
        block=64, a_scale=case["a_scale"], b1=case["b1"], b2=case["b2"], res_scale=case["rs"],
        sel=sel, keep=keep, win_k=wk if n_win else None, win_v=wv if n_win else None)
    tl = lambda x: None if x is None else np.asarray(x, np.float64).tolist()
    ref, rstats = _brute_decode(
        tl(case["q"]), tl(case["a"]), tl(case["a_scale"]), tl(case["bl"]), tl(case["w_lin"]), tl(case["w1"]),
        tl(case["b1"]), tl(case["w2"]), tl(case["b2"]), case["idx"].tolist(), tl(case["rv"]), tl(case["rs"]),
        sel, None if keep is None else list(keep), wk.tolist(), wv.tolist(), 64)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-11, atol=1e-12)
    assert gstats.tolist() == rstats


@pytest.mark.parametrize("n_tok", [128, 100])
def test_brute_force_every_block_subset_and_window(n_tok):
    rng = np.random.default_rng(4 + n_tok)
    case = _tiny_case(rng, n_tok)
    nb = (n_tok + 63) // 64
    for m in range(1, nb + 1):
        for sel in itertools.combinations(range(nb), m):
            for n_win in range(4):
                _run_both(case, list(sel), None, n_win, rng)
    _run_both(case, None, None, 0, rng)          # no selection = all blocks


def test_brute_force_int8_keep_and_no_bias():
    rng = np.random.default_rng(5)
    case = _tiny_case(rng, 200, int8_a=True, int8_r=True, biases=False)
    _run_both(case, None, np.array([1, 0, 1, 1], np.uint8), 2, rng)
    _run_both(case, [0, 1, 3], np.array([1, 1, 0, 1], np.uint8), 0, rng)
    # Everything evicted and no window: nothing to attend, output zero.
    out, stats = oracle.decode_batch_element(
        case["q"], case["a"], case["bl"], case["w_lin"], case["w1"], case["w2"], case["idx"], case["rv"],
        block=64, a_scale=case["a_scale"], res_scale=case["rs"], keep=np.zeros(4, np.uint8))
    assert not out.any() and stats.tolist() == [[0, 0], [0, 0]]


def test_brute_force_two_bit_residuals():
    """Packed 2-bit residual rows in the decode: the scalar decoder reads each
    code with plain bit operations, element o in bits 2(o mod 4) of byte
    o // 4, and applies (q - 1.5) s."""
    rng = np.random.default_rng(6)
    case = _tiny_case(rng, 150)
    n_kv, k, d = case["rv"].shape
    packed = rng.integers(0, 256, (n_kv, k, d // 4)).astype(np.uint8)
    scale = rng.uniform(0.05, 0.2, (n_kv, k)).astype(np.float32)
    levels = [[[((int(packed[h, p, o // 4]) >> (2 * (o % 4))) & 3) - 1.5 for o in range(d)]
               for p in range(k)] for h in range(n_kv)]
    wk = rng.standard_normal((1, n_kv * d))
    wv = rng.standard_normal((1, n_kv * d))
    got, gstats = oracle.decode_batch_element(
        case["q"], case["a"], case["bl"], case["w_lin"], case["w1"], case["w2"], case["idx"], packed,
        block=64, b1=case["b1"], b2=case["b2"], res_scale=scale, win_k=wk, win_v=wv)
    tl = lambda x: None if x is None else np.asarray(x, np.float64).tolist()  # noqa: E731
    ref, rstats = _brute_decode(
        tl(case["q"]), tl(case["a"]), None, tl(case["bl"]), tl(case["w_lin"]), tl(case["w1"]), tl(case["b1"]),
        tl(case["w2"]), tl(case["b2"]), case["idx"].tolist(), levels, tl(scale), None, None,
        wk.tolist(), wv.tolist(), 64)
    np.testing.assert_allclose(got, np.array(ref), rtol=1e-11, atol=1e-12)
    assert gstats.tolist() == rstats


@pytest.mark.parametrize("enc", ["float", "int8", "i2"])
def test_decode_step_routes_every_sequence(enc):
    """decode_step over a batch of three sequences, each with its own query,
    factor A (and int8 row scales), B_l, predictor, residual set and scales,
    padded selection row, eviction row and window rows, the window buffers
    holding more rows than win_len. Every sequence must equal the scalar brute
    force on that sequence's own data and exactly its first win_len window
    rows (explainer, mechanism paragraph; prefill/decode paragraph: the recent
    tokens are stored exactly)."""
    rng = np.random.default_rng(11 + len(enc))
    n_b, n_tok, win_cap, win_len = 3, 200, 6, 4
    cases = [_tiny_case(rng, n_tok, int8_a=enc == "int8", int8_r=enc == "int8") for _ in range(n_b)]
    n_kv, d = cases[0]["w_lin"].shape[:2]
    k = cases[0]["idx"].shape[1]
    if enc == "i2":
        for c in cases:
            c["rv"] = rng.integers(0, 256, (n_kv, k, d // 4)).astype(np.uint8)
            c["rs"] = rng.uniform(0.05, 0.2, (n_kv, k)).astype(np.float32)
    sels = [[0, 2, 3, -1], [1, 3, -1, -1], [0, 1, 2, 3]]
    keeps = [np.array([1, 1, 1, 1], np.uint8), np.array([1, 1, 1, 1], np.uint8), np.array([1, 0, 1, 1], np.uint8)]
    wk = rng.standard_normal((n_b, win_cap, n_kv * d))
    wv = rng.standard_normal((n_b, win_cap, n_kv * d))
    batch = {name: np.stack([c[src] for c in cases]) for name, src in
             (("q", "q"), ("a", "a"), ("bl", "bl"), ("w_lin", "w_lin"), ("w1", "w1"), ("w2", "w2"),
              ("b1", "b1"), ("b2", "b2"), ("res_idx", "idx"), ("res_val", "rv"))}
    if enc == "int8":
        batch["a_scale"] = np.stack([c["a_scale"] for c in cases])
    if enc != "float":
        batch["res_scale"] = np.stack([c["rs"] for c in cases])
    batch.update(sel=np.array(sels, np.int32), keep=np.stack(keeps), win_k=wk, win_v=wv, win_len=win_len, block=64)
    tl = lambda x: None if x is None else np.asarray(x, np.float64).tolist()  # noqa: E731

    def rows(c):
        # 2-bit codes read with plain bit operations: element o in bits
        # 2(o mod 4) of byte o // 4, level q - 1.5.
        if enc != "i2":
            return tl(c["rv"])
        return [[[((int(c["rv"][h, p, o // 4]) >> (2 * (o % 4))) & 3) - 1.5 for o in range(d)]
                 for p in range(k)] for h in range(n_kv)]

    def brute(b, n_win):
        c = cases[b]
        return _brute_decode(
            tl(c["q"]), tl(c["a"]), tl(c["a_scale"]), tl(c["bl"]), tl(c["w_lin"]), tl(c["w1"]), tl(c["b1"]),
            tl(c["w2"]), tl(c["b2"]), c["idx"].tolist(), rows(c), tl(c["rs"]), sels[b], list(keeps[b]),
            wk[b, :n_win].tolist(), wv[b, :n_win].tolist(), 64)

    for n_win in (win_len, 0):
        batch["win_len"] = n_win
        got, gstats = oracle.decode_step(batch)
        assert got.shape == (n_b, cases[0]["q"].shape[0], d)
        for b in range(n_b):
            ref, rstats = brute(b, n_win)
            np.testing.assert_allclose(got[b], np.array(ref), rtol=1e-11, atol=1e-12)
            assert gstats[b].tolist() == rstats


# ------------------------------------------------------------ invariants
def test_selection_invariants():
    rng = np.random.default_rng(6)
    case = _tiny_case(rng, 300)
    args = (case["q"], case["a"], case["bl"], case["w_lin"], case["w1"], case["w2"], case["idx"], case["rv"])
    kw = dict(block=64, b1=case["b1"], b2=case["b2"])
    full, _ = oracle.decode_batch_element(*args, **kw)
    all_sel, _ = oracle.decode_batch_element(*args, sel=[0, 1, 2, 3, 4], **kw)
    np.testing.assert_array_equal(full, all_sel)
    a1, _ = oracle.decode_batch_element(*args, sel=[0, 2, 4], **kw)
    a2, _ = oracle.decode_batch_element(*args, sel=[4, 0, 2], **kw)
    np.testing.assert_allclose(a1, a2, rtol=1e-13, atol=1e-14)
    a3, _ = oracle.decode_batch_element(*args, keep=np.array([1, 0, 1, 0, 1], np.uint8), **kw)
    np.testing.assert_allclose(a1, a3, rtol=0, atol=0)
    # Padding entries (outside [0, nb)) in a selection row name no block.
    a4, s4 = oracle.decode_batch_element(*args, sel=[-1, 0, 2, 4, 5, 99], **kw)
    _, s1 = oracle.decode_batch_element(*args, sel=[0, 2, 4], **kw)
    np.testing.assert_array_equal(a1, a4)
    assert s4.tolist() == s1.tolist()
    a5, s5 = oracle.decode_batch_element(*args, sel=[-1, -1], **kw)
    assert not a5.any() and not s5.any()


def test_split_softmax_merge_equals_single_pass():
    """Flash-decoding merge identity the GPU combine relies on:
    o = sum_s e^{m_s - M} o_s / sum_s e^{m_s - M} l_s."""
    rng = np.random.default_rng(7)
    keys = rng.standard_normal((90, 8)) * 3
    vals = rng.standard_normal((90, 5))
    qv = rng.standard_normal(8)
    whole = oracle.attention(qv, keys, vals)
    parts = []
    for lo, hi in ((0, 30), (30, 64), (64, 90)):
        s = keys[lo:hi] @ qv / math.sqrt(8)
        m = s.max()
        p = np.exp(s - m)
        parts.append((m, p.sum(), p @ vals[lo:hi]))
    mm = max(p[0] for p in parts)
    num = sum(np.exp(m - mm) * o for m, _, o in parts)
    den = sum(np.exp(m - mm) * l for m, l, _ in parts)
    np.testing.assert_allclose(num / den, whole, rtol=1e-13)


# ----------------------------------------------------------------- GELU
def test_gelu_identities():
    xs = np.linspace(-6, 6, 101)
    assert oracle.gelu(0.0) == 0.0
    np.testing.assert_allclose(oracle.gelu(xs) - oracle.gelu(-xs), xs, rtol=0, atol=1e-14)
    np.testing.assert_allclose(oracle.gelu(xs), [_gelu_py(float(x)) for x in xs], rtol=1e-14, atol=1e-16)
    # x * Phi(x) at x = 1: Phi(1) = 0.8413447460685429 (normal CDF table value).
    assert abs(float(oracle.gelu(1.0)) - 0.8413447460685429) < 1e-15


# ------------------------------------------------------------ ranking
def _brute_rank(v, vh, k):
    errs = []
    for t in range(len(v)):
        e = 0.0
        for i in range(len(v[t])):
            dlt = float(v[t][i]) - float(vh[t][i])
            e = e + dlt * dlt
        errs.append(e)
    top = sorted(range(len(v)), key=lambda t: (-errs[t], t))[:k]
    return errs, sorted(top)


@pytest.mark.parametrize("k", [0, 1, 7, 20, 49, 50])
def test_ranking_brute_force(k):
    rng = np.random.default_rng(8)
    n_tok, n_kv, d = 50, 2, 4
    vh = rng.standard_normal((1, n_tok, n_kv, d)).astype(np.float32)
    v = (vh + rng.standard_normal(vh.shape).astype(np.float32) * 0.3).astype(np.float32)
    v[0, 10] = v[0, 3]; vh[0, 10] = vh[0, 3]          # exact duplicates -> equal errors
    v[0, 40] = v[0, 3]; vh[0, 40] = vh[0, 3]
    got = oracle.rank_residuals(v, vh, k, 16, "f32")
    for h in range(n_kv):
        errs, top = _brute_rank(v[0, :, h].tolist(), vh[0, :, h].tolist(), k)
        assert got["err"][0, h].tolist() == errs
        assert got["idx"][0, h].tolist() == top
        ptr = [sum(1 for t in top if t < i * 16) for i in range(4)] + [len(top)]
        assert got["ptr"][0, h].tolist() == ptr
        f32 = lambda x: struct.unpack("f", struct.pack("f", x))[0]
        want = [[f32(float(v[0, t, h, i]) - float(vh[0, t, h, i])) for i in range(d)] for t in top]
        np.testing.assert_array_equal(got["val"][0, h], np.array(want).reshape(-1, d))


def test_ranking_special_cases():
    rng = np.random.default_rng(9)
    n_tok, d = 40, 4
    vh = rng.standard_normal((1, n_tok, 1, d)).astype(np.float32).astype(np.float64)
    same = vh + 0.5                                  # every error equal: lowest indices win
    r = oracle.rank_residuals(same, vh, 7, 16, "f32")
    assert r["idx"][0, 0].tolist() == list(range(7))
    assert oracle.rank_residuals(same, vh, 0, 16, "f32")["idx"].shape == (1, 1, 0)
    assert oracle.rank_residuals(same, vh, n_tok, 16, "f32")["idx"][0, 0].tolist() == list(range(n_tok))
    # A tie group straddling the k-th place: tokens 30..35 share the 3rd-largest error.
    v = vh.copy()
    v[0, 5] += 9.0
    v[0, 17] += 8.0
    for t in range(30, 36):
        v[0, t] = vh[0, t] + 4.0
    r = oracle.rank_residuals(v, vh, 4, 16, "f32")
    assert r["idx"][0, 0].tolist() == [5, 17, 30, 31]


# --------------------------------------------------------- rounding and int8
def test_bf16_rounding_matches_library_and_closed_forms():
    rng = np.random.default_rng(10)
    xs = np.concatenate([rng.standard_normal(5000) * 10.0 ** rng.integers(-40, 38, 5000),
                         [0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.0e38, 1e-40, -2.5e-39]]).astype(np.float32)
    ref = torch.from_numpy(xs).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(oracle.round_bf16(xs.astype(np.float64)), ref)
    # One rounding step, not two: 1 + 2^-8 + 2^-40 is above the bf16 midpoint
    # between 1 and 1 + 2^-7, so it rounds up, while a float32 detour would
    # land exactly on the midpoint and round to even (down).
    assert oracle.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert oracle.round_bf16(1.0 + 2.0 ** -8) == 1.0                     # tie to even
    assert oracle.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6     # tie to even, upward
    assert np.isinf(oracle.round_bf16(3.4e38))


def test_int8_code_invariants():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((300, 16)) * rng.uniform(1e-3, 10, (300, 1))
    x[7] = 0.0
    q, s = oracle.quantize_int8_rows(x)
    deq = oracle.dequantize_int8_rows(q, s)
    assert np.all(np.abs(deq - x) <= s.astype(np.float64)[:, None] / 2 * (1 + 1e-12) + 1e-300)
    assert s[7] == 0 and not q[7].any()
    assert np.abs(q).max() == 127
    q2, s2 = oracle.quantize_int8_rows(deq)
    np.testing.assert_array_equal(q2, q)
    np.testing.assert_array_equal(s2, s)


# ------------------------------------------------------- printed numbers
def test_memory_budget_worked_example():
    with open(os.path.join(GOLDEN, "memory_budget.json")) as f:
        g = json.load(f)["cases"]
    b = oracle.value_budget(32768)
    assert (b["dense"], b["budget"], b["predictor"], b["remaining"]) == (
        g[0]["dense"], g[0]["budget"], g[0]["predictor"], g[0]["remaining"])
    assert round(b["residuals"]) == g[0]["residuals_printed"]
    assert int(100 * b["token_fraction"]) == g[0]["token_percent_printed"]
    b = oracle.value_budget(4096)
    assert (b["budget"], b["predictor"]) == (g[1]["budget"], g[1]["predictor"])
    assert round(b["residuals"]) == g[1]["residuals_printed"]
    assert int(100 * b["token_fraction"]) == g[1]["token_percent_printed"]
    b = oracle.value_budget(2048)
    assert abs(b["predictor_share"] - g[2]["predictor_share_printed"]) < 0.01


def test_dense_kv_bytes_per_token():
    with open(os.path.join(GOLDEN, "dense_kv_per_token.json")) as f:
        g = json.load(f)
    sh = g["shape"]
    nbytes = oracle.dense_kv_bytes_per_token(sh["layers"], sh["kv_heads"], sh["head_dim"], sh["elem_bytes"])
    assert round(nbytes / 1000, 2) == g["kb_per_token_printed"]


# ------------------------------------------------ fused prefill: V_hat everywhere
def test_predicted_values_slim_case_per_layer():
    """explainer, Slim Attention paragraph, for every layer of a group sharing
    one key factor: with A = x, B_l = the layer's invertible W_K and
    W_lin = pinv(W_K) W_V (nonlinear branch zero), every token's predicted
    value is x W_V exactly."""
    rng = np.random.default_rng(21)
    n_tok, d, n_kv, hid, n_l = 40, 8, 2, 4, 3
    x = rng.standard_normal((n_tok, d))
    w_k = rng.standard_normal((n_l, n_kv, d, d)) + 3 * np.eye(d)
    w_v = rng.standard_normal((n_l, n_kv, d, d))
    bl = np.stack([np.concatenate([w_k[l, h].T for h in range(n_kv)], axis=0) for l in range(n_l)])
    w_lin = np.stack([[oracle.pinv_value_map(w_k[l, h], w_v[l, h]) for h in range(n_kv)] for l in range(n_l)])
    zeros1, zeros2 = np.zeros((n_l, n_kv, hid, d)), np.zeros((n_l, n_kv, d, hid))
    vh = oracle.predicted_values(x[None], bl, w_lin, zeros1, zeros2, group=4)
    for l in range(n_l):
        for h in range(n_kv):
            np.testing.assert_allclose(vh[l, :, h, :], x @ w_v[l, h], rtol=0, atol=1e-10)


def test_predicted_values_brute_force_groups_and_biases():
    """Pure-Python loops with math.erf on tiny inputs: five layers in groups of
    four (layer 4 reads the second factor), nonzero biases."""
    rng = np.random.default_rng(22)
    n_l, grp, n_tok, r, d, n_kv, hid = 5, 4, 3, 3, 2, 2, 3
    a = rng.standard_normal((2, n_tok, r))
    bl = rng.standard_normal((n_l, n_kv * d, r))
    w_lin = rng.standard_normal((n_l, n_kv, d, d))
    w1 = rng.standard_normal((n_l, n_kv, hid, d))
    w2 = rng.standard_normal((n_l, n_kv, d, hid))
    b1 = rng.standard_normal((n_l, n_kv, hid))
    b2 = rng.standard_normal((n_l, n_kv, d))
    vh = oracle.predicted_values(a, bl, w_lin, w1, w2, b1, b2, group=grp)
    for l in range(n_l):
        for t in range(n_tok):
            for h in range(n_kv):
                key = [sum(a[l // grp, t, c] * bl[l, h * d + i, c] for c in range(r)) for i in range(d)]
                hidden = []
                for j in range(hid):
                    z = sum(key[i] * w1[l, h, j, i] for i in range(d)) + b1[l, h, j]
                    hidden.append(0.5 * z * (1.0 + math.erf(z / math.sqrt(2.0))))
                for o in range(d):
                    want = (sum(key[i] * w_lin[l, h, o, i] for i in range(d)) +
                            sum(hidden[j] * w2[l, h, o, j] for j in range(hid)) + b2[l, h, o])
                    assert abs(vh[l, t, h, o] - want) <= 1e-12 * max(1.0, abs(want))


# ------------------------------------------------------------- 2-bit residuals
def test_i2_levels_closed_form():
    """A row on the four levels comes back exactly: (-1.5, -0.5, 0.5, 1.5) c
    with c = 1/8 gives s = c and q = 0, 1, 2, 3."""
    c = 0.125
    row = np.array([[-1.5, -0.5, 0.5, 1.5, 1.5, -1.5, 0.5, -0.5]]) * c
    q, s = oracle.quantize_i2_rows(row)
    assert s.tolist() == [np.float32(c)]
    assert q.tolist() == [[0, 1, 2, 3, 3, 0, 2, 1]]
    np.testing.assert_array_equal(oracle.dequantize_i2_rows(q, s), row)


def test_i2_error_bound_and_zero_row():
    """Every element lies within the level range (max level = max|r|), so the
    round-to-nearest level is within s/2 of it; an all-zero row is level 0."""
    rng = np.random.default_rng(31)
    r = rng.standard_normal((300, 128)) * np.exp(rng.standard_normal((300, 1)))
    q, s = oracle.quantize_i2_rows(r)
    assert q.min() >= 0 and q.max() <= 3
    err = np.abs(oracle.dequantize_i2_rows(q, s) - r)
    assert np.all(err <= s.astype(np.float64)[:, None] / 2 * (1 + 1e-6) + 1e-300)
    q0, s0 = oracle.quantize_i2_rows(np.zeros((2, 8)))
    assert s0.tolist() == [0.0, 0.0] and q0.tolist() == [[2] * 8] * 2
    np.testing.assert_array_equal(oracle.dequantize_i2_rows(q0, s0), np.zeros((2, 8)))


def test_i2_packing_layout():
    """Element i sits in bits 2(i mod 4) of byte i // 4; pack/unpack invert."""
    q = np.array([[1, 2, 3, 0, 0, 0, 0, 3]], np.uint8)
    b = oracle.pack_i2(q)
    assert b.tolist() == [[1 | (2 << 2) | (3 << 4), 3 << 6]]
    rng = np.random.default_rng(32)
    qq = rng.integers(0, 4, size=(5, 7, 128)).astype(np.uint8)
    np.testing.assert_array_equal(oracle.unpack_i2(oracle.pack_i2(qq)), qq)


def test_rank_residuals_i2_matches_its_codec():
    """The ranking's 'i2' store is the codec above applied to V - V_hat at the
    chosen tokens (same tokens as any other encoding)."""
    rng = np.random.default_rng(33)
    v = rng.standard_normal((2, 90, 2, 8)).astype(np.float32)
    vh = rng.standard_normal((2, 90, 2, 8)).astype(np.float32)
    a = oracle.rank_residuals(v, vh, 11, 64, "i2")
    b = oracle.rank_residuals(v, vh, 11, 64, "f32")
    np.testing.assert_array_equal(a["idx"], b["idx"])
    for sl in range(2):
        for h in range(2):
            r = v[sl, a["idx"][sl, h], h].astype(np.float64) - vh[sl, a["idx"][sl, h], h].astype(np.float64)
            q, s = oracle.quantize_i2_rows(r)
            np.testing.assert_array_equal(oracle.unpack_i2(a["val"][sl, h]), q)
            np.testing.assert_array_equal(a["scale"][sl, h], s)


# ------------------------------------------------------------ predictor fit
def _fit_case(rng, n_tok=7, d=3, hid=4):
    return dict(k=rng.standard_normal((n_tok, d)), v=rng.standard_normal((n_tok, d)),
                w_lin=rng.standard_normal((d, d)) * 0.5, w1=rng.standard_normal((hid, d)) * 0.7,
                b1=rng.standard_normal(hid) * 0.3, w2=rng.standard_normal((d, hid)) * 0.6,
                b2=rng.standard_normal(d) * 0.2)


def _loss_py(c):
    """Scalar loop from the definitions: mean over tokens of the squared error
    of the predictor (math.erf GELU, no numpy arithmetic)."""
    tl = lambda x: np.asarray(x, np.float64).tolist()  # noqa: E731
    k, v, wl, w1, b1, w2, b2 = (tl(c[n]) for n in ("k", "v", "w_lin", "w1", "b1", "w2", "b2"))
    tot = 0.0
    for t in range(len(k)):
        hid = [_gelu_py(sum(k[t][i] * w1[u][i] for i in range(len(k[t]))) + b1[u]) for u in range(len(w1))]
        for o in range(len(v[t])):
            vh = sum(k[t][i] * wl[o][i] for i in range(len(k[t]))) + sum(hid[u] * w2[o][u] for u in range(len(hid))) + b2[o]
            tot += (vh - v[t][o]) ** 2
    return tot / len(k)


def test_fit_gradient_matches_central_differences():
    """One gradient step recovers the gradient, (theta0 - theta1) / lr, which
    must match central differences of the scalar-loop loss for every
    parameter of a tiny case."""
    rng = np.random.default_rng(50)
    c = _fit_case(rng)
    lr = 1e-3
    w1, b1, w2, b2, losses = oracle.fit_predictor(c["k"], c["v"], c["w_lin"], c["w1"], c["b1"], c["w2"], c["b2"], lr, 1)
    assert abs(losses[0] - _loss_py(c)) < 1e-12
    got = {"w1": (c["w1"] - w1) / lr, "b1": (c["b1"] - b1) / lr, "w2": (c["w2"] - w2) / lr, "b2": (c["b2"] - b2) / lr}
    eps = 1e-6
    for name, g in got.items():
        num = np.zeros_like(g)
        for idx in np.ndindex(g.shape):
            cp = {kk: np.array(vv, np.float64) for kk, vv in c.items()}
            cm = {kk: np.array(vv, np.float64) for kk, vv in c.items()}
            cp[name][idx] += eps
            cm[name][idx] -= eps
            num[idx] = (_loss_py(cp) - _loss_py(cm)) / (2 * eps)
        np.testing.assert_allclose(g, num, rtol=1e-6, atol=1e-8)


def test_fit_special_cases():
    """No steps leave the parameters as they are; values that the linear map
    already predicts exactly (w2 = 0, b2 = 0) give zero loss and zero
    gradients, so steps change nothing; on a generic case a small rate lowers
    the loss at every step."""
    rng = np.random.default_rng(51)
    c = _fit_case(rng, n_tok=40)
    out = oracle.fit_predictor(c["k"], c["v"], c["w_lin"], c["w1"], c["b1"], c["w2"], c["b2"], 0.1, 0)
    for a, b in zip(out[:4], (c["w1"], c["b1"], c["w2"], c["b2"])):
        np.testing.assert_array_equal(a, b)
    assert len(out[4]) == 1
    v_lin = c["k"] @ c["w_lin"].T
    out = oracle.fit_predictor(c["k"], v_lin, c["w_lin"], c["w1"], c["b1"], np.zeros_like(c["w2"]),
                               np.zeros_like(c["b2"]), 0.5, 3)
    np.testing.assert_array_equal(out[0], c["w1"])
    np.testing.assert_array_equal(out[2], 0.0)
    assert np.all(out[4] < 1e-28)
    losses = oracle.fit_predictor(c["k"], c["v"], c["w_lin"], c["w1"], c["b1"], c["w2"], c["b2"], 0.02, 25)[4]
    assert np.all(np.diff(losses) < 0)


def test_gelu_grad_closed_form():
    """gelu'(0) = 1/2; gelu'(z) + gelu'(-z) = 1 (from gelu(z) - gelu(-z) = z);
    central differences of the oracle's gelu."""
    z = np.linspace(-6, 6, 121)
    assert oracle.gelu_grad(0.0) == 0.5
    np.testing.assert_allclose(oracle.gelu_grad(z) + oracle.gelu_grad(-z), 1.0, atol=1e-15)
    h = 1e-6
    np.testing.assert_allclose(oracle.gelu_grad(z), (oracle.gelu(z + h) - oracle.gelu(z - h)) / (2 * h), atol=1e-8)
