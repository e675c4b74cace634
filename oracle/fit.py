"""Test-time fit of the per-head value predictor (float64).

Test infrastructure only (see the package docstring). The explainer's
Slim Attention paragraph starts the predictor from the best linear map the
projection weights allow (a pseudoinverse, ``factor.pinv_value_map``) and lets
the small nonlinear branch learn the rest from the current context; its cost
paragraph says the fit runs gradient steps per context at prefill (150 for the
full fit, 2 from a meta-learned start). The pages name neither the loss nor
the optimiser. The reading taken here: the loss is the mean over tokens of the
squared L2 error of the predicted values (the ranking's error measure),

    L = (1 / T) sum_t || v_hat_t - v_t ||^2,

minimised by plain gradient descent with a fixed rate on the nonlinear
branch's W1, b1, W2, b2, with W_lin held at its start.
"""
import math

import numpy as np

from .decode import gelu, predict_values


def gelu_grad(z):
    """d gelu / dz = Phi(z) + z phi(z) for the exact erf form."""
    z = np.asarray(z, np.float64)
    from scipy.special import erf
    return 0.5 * (1.0 + erf(z / math.sqrt(2.0))) + z * np.exp(-0.5 * z * z) / math.sqrt(2.0 * math.pi)


def predictor_loss_and_grads(k, v, w_lin, w1, b1, w2, b2):
    """Loss L and its gradients with respect to (w1, b1, w2, b2).

    Row vectors, weights stored output-major as in ``predict_values``:
    z = k w1^T + b1, h = gelu(z), v_hat = k w_lin^T + h w2^T + b2,
    g = (2 / T) (v_hat - v), dL/dw2 = g^T h, dL/db2 = sum_t g,
    dh = g w2, dz = dh * gelu'(z), dL/dw1 = dz^T k, dL/db1 = sum_t dz."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    w1, b1, w2, b2 = (np.asarray(x, np.float64) for x in (w1, b1, w2, b2))
    n_tok = k.shape[0]
    z = k @ w1.T + b1
    hid = gelu(z)
    v_hat = k @ np.asarray(w_lin, np.float64).T + hid @ w2.T + b2
    e = v_hat - v
    loss = float(np.sum(e * e)) / n_tok
    g = (2.0 / n_tok) * e
    dz = (g @ w2) * gelu_grad(z)
    return loss, (dz.T @ k, dz.sum(axis=0), g.T @ hid, g.sum(axis=0))


def fit_predictor(k, v, w_lin, w1, b1, w2, b2, lr, n_steps):
    """``n_steps`` steps of theta <- theta - lr dL/dtheta on (w1, b1, w2, b2).

    Returns (w1, b1, w2, b2, losses) with losses[i] the loss before step i
    and losses[n_steps] the loss after the last step."""
    w1, b1, w2, b2 = (np.array(x, np.float64) for x in (w1, b1, w2, b2))
    losses = []
    for _ in range(n_steps):
        loss, (g1, gb1, g2, gb2) = predictor_loss_and_grads(k, v, w_lin, w1, b1, w2, b2)
        losses.append(loss)
        w1 -= lr * g1
        b1 -= lr * gb1
        w2 -= lr * g2
        b2 -= lr * gb2
    e = predict_values(k, w_lin, w1, w2, b1, b2) - np.asarray(v, np.float64)
    losses.append(float(np.sum(e * e)) / np.asarray(k).shape[0])
    return w1, b1, w2, b2, np.array(losses)
