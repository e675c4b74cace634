"""Oracle helpers that produce the path's factor inputs (float64).

Test infrastructure only (see the package docstring). ``xkv_factorize`` and
``pinv_value_map`` are the plain definitions; ``xkv_subspace_iteration`` is
the iterative prefill step the library runs, written out step by step.
"""
import numpy as np


def xkv_factorize(keys, rank):
    """Cross-layer low-rank factors of a layer group's keys.

    project site, Figure 3, and the explainer's keys paragraph: one factor is
    shared by a group of adjacent layers and each layer keeps its own smaller
    factor, K_l ~ A . B_l. Here the group's keys [K_1 | ... | K_G] (T x G*D)
    get a truncated SVD U S V^T; A = U_r S_r (T x r) and B_l is layer l's
    column slice of V_r^T (r x D). By Eckart-Young this is the best rank-r
    fit of the concatenation in the Frobenius norm.

    ``keys`` is a list of [T, D] arrays. Returns (A [T, r], [bl_l]) with each
    B_l stored output-major, bl_l = B_l^T [D, r], and the singular values.
    """
    cat = np.concatenate([np.asarray(k, np.float64) for k in keys], axis=1)
    u, s, vt = np.linalg.svd(cat, full_matrices=False)
    a = u[:, :rank] * s[:rank]
    width = np.asarray(keys[0]).shape[1]
    bls = [vt[:rank, l * width:(l + 1) * width].T.copy() for l in range(len(keys))]
    return a, bls, s


def pinv_value_map(w_k, w_v):
    """Linear value map from keys: W_lin = pinv(W_K) . W_V, the best linear
    guess the projections allow (explainer, Slim Attention paragraph). With
    x . W_K = k and x . W_V = v it gives k . W_lin = v exactly when W_K is
    square and invertible. W_K, W_V are [hidden, d] in the row-vector
    convention; the result is returned output-major ([d_out, d_in])."""
    return (np.linalg.pinv(np.asarray(w_k, np.float64)) @ np.asarray(w_v, np.float64)).T


def xkv_subspace_iteration(keys, rank, omega, n_iter):
    """Cross-layer key factors by randomized subspace iteration.

    The factors of ``xkv_factorize`` (project site, Figure 3; explainer, keys
    paragraph: one basis for a group of adjacent layers) computed the way the
    library does: Halko, Martinsson and Tropp, "Finding structure with
    randomness" (SIAM Review 2011), Algorithm 4.4, run on the row space. With
    C = [K_1 | ... | K_G] (T x n) and its Gram matrix M = C^T C:
        X_0 = omega  (n x r, the caller's Gaussian draw),
        X_i = orth(M X_{i-1})  for i = 1 .. n_iter,
        A   = C X_q,   B_l = (rows l*D .. l*D+D-1 of X_q)^T,
    so K_l ~ A B_l with K_l's reconstruction C X_q X_q^T restricted to layer
    l's columns. orth returns an orthonormal basis of the span (Householder
    QR here); the span, hence A B_l, does not depend on which basis.

    ``keys`` is a list of G arrays [T, D]. Returns (A [T, r], [bl_l] with
    bl_l = B_l^T [D, r], X_q [n, r])."""
    cat = np.concatenate([np.asarray(k, np.float64) for k in keys], axis=1)
    m = cat.T @ cat
    x = np.asarray(omega, np.float64)
    assert x.shape == (cat.shape[1], rank) and n_iter >= 1
    for _ in range(n_iter):
        x = np.linalg.qr(m @ x)[0]
    a = cat @ x
    width = np.asarray(keys[0]).shape[1]
    bls = [x[l * width:(l + 1) * width].copy() for l in range(len(keys))]
    return a, bls, x
