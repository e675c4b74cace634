"""Oracle helpers that produce the path's factor inputs (float64).

Test infrastructure only (see the package docstring). These are not on the
decode path; they exist so the pins can drive the decode oracle with factors
whose exact result is known.
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
