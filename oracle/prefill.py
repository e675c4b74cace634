"""Oracle of the fused prefill ranking: the predictor's values for every
cached token, then the ranking of oracle.rank (float64, plain definitions).

Test infrastructure only (see the package docstring).
"""
import numpy as np

from .decode import predict_values, reconstruct_keys
from .rank import rank_residuals


def predicted_values(a, bl, w_lin, w1, w2, b1=None, b2=None, group=4):
    """V_hat for every token, layer and KV head.

    project site, Figure 3 (K_l = A_group . B_l, one factor shared by a group
    of layers); explainer, mechanism paragraph (the per-head predictor applied
    to the keys). ``a`` is [ceil(Lr/group), T, r]; ``bl`` [Lr, Hkv*d, r];
    ``w_lin`` [Lr, Hkv, d, d], ``w1`` [Lr, Hkv, h, d], ``w2`` [Lr, Hkv, d, h]
    output-major; biases [Lr, Hkv, h] / [Lr, Hkv, d] or None. Returns
    [Lr, T, Hkv, d].
    """
    bl = np.asarray(bl)
    n_l, hkv = bl.shape[0], np.asarray(w_lin).shape[1]
    d = bl.shape[1] // hkv
    t = np.asarray(a).shape[1]
    out = np.zeros((n_l, t, hkv, d))
    for l in range(n_l):
        keys = reconstruct_keys(np.asarray(a)[l // group], bl[l])          # [T, Hkv*d]
        for h in range(hkv):
            out[l, :, h, :] = predict_values(
                keys[:, h * d:(h + 1) * d], np.asarray(w_lin)[l, h], np.asarray(w1)[l, h], np.asarray(w2)[l, h],
                None if b1 is None else np.asarray(b1)[l, h], None if b2 is None else np.asarray(b2)[l, h])
    return out


def prefill_rank(v, v_hat, k, block, res_dtype):
    """The ranking of the fused path: oracle.rank_residuals on the true values
    against the given V_hat (explainer, three-details paragraph: residuals
    for the tokens the predictor reconstructs worst)."""
    return rank_residuals(v, v_hat, k, block, res_dtype)
