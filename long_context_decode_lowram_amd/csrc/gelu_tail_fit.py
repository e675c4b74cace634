"""Derive the constants of the device normal tail and GELU.

GELU(x) = x * Phi(x). With Q(a) = 1 - Phi(a) = erfc(a / sqrt 2) / 2 for a >= 0,
GELU(x) = x - x Q(x) for x >= 0 and x Q(-x) for x < 0, i.e.
GELU(x) = max(x, 0) - |x| Q(|x|). The device evaluates log2 Q(a) by a
polynomial in a and takes one exp2. Two fits:

* normal_tail (used where Q itself is needed, for GELU and its derivative in
  the predictor fit): degree 4 on [0, 6], with a clamped to 6 (6 Q(6) < 1e-8).
* gelu_tail16 (the decode kernel's GELU): degree 3 on [0, 6] with a negative
  cubic coefficient, so 2^P(a) falls to zero by itself as a grows and no clamp
  is needed; one multiply-add and the clamp fewer per element.

Each fit is a least-squares fit on Chebyshev nodes of the interval, weighted by
a Q(a) (the size of the term the polynomial's error scales), then reweighted a
few dozen times toward the nodes with the largest absolute GELU error (Lawson's
iteration towards the minimax fit). The script prints the coefficients, the
worst absolute GELU error of the float32 evaluation against scipy's erfc over
[-12, 12], and for the unclamped fit the largest a 2^P(a) over [6, 1e4].

python long_context_decode_lowram_amd/csrc/gelu_tail_fit.py
"""
import numpy as np
from scipy.special import erfc

X, ROUNDS = 6.0, 30


def fit(deg):
    n = 6000
    a = np.cos(np.pi * (np.arange(n) + 0.5) / n) * X / 2 + X / 2
    q = 0.5 * erfc(a / np.sqrt(2.0))
    y = np.log2(q)
    w = a * q + 1e-3
    c = np.polynomial.polynomial.polyfit(a, y, deg, w=w)
    for _ in range(ROUNDS):
        err = np.abs(a * (np.exp2(np.polynomial.polynomial.polyval(a, c)) - q))
        w = w * (1.0 + 5.0 * err / err.max())
        c = np.polynomial.polynomial.polyfit(a, y, deg, w=w)
    return c.astype(np.float32)


def gelu_f32(x, c, clamp):
    x = np.asarray(x, np.float32)
    a = np.abs(x)
    if clamp:
        a = np.minimum(a, np.float32(X))
    p = np.float32(c[-1])
    for k in range(len(c) - 2, -1, -1):
        p = (p * a + c[k]).astype(np.float32)
    q = np.exp2(p).astype(np.float32)
    t = (a * q).astype(np.float32)
    return (np.maximum(x, np.float32(0)) - t).astype(np.float32)


def max_error(c, clamp):
    x = np.linspace(-12, 12, 2_000_001)
    ref = x * (1.0 - 0.5 * erfc(x / np.sqrt(2.0)))
    return float(np.max(np.abs(gelu_f32(x, c, clamp).astype(np.float64) - ref)))


if __name__ == "__main__":
    for name, deg, clamp in (("normal_tail", 4, True), ("gelu_tail16", 3, False)):
        c = fit(deg)
        print(name, "coefficients c0..c%d:" % deg, ", ".join(f"{float(v)!r}f" for v in c))
        print("  max |gelu error| =", max_error(c, clamp))
        if not clamp:
            assert c[-1] < 0
            t = np.linspace(X, 1e4, 100001)
            print("  max a 2^P(a) over [6, 1e4] =", float(np.max(t * np.exp2(np.polynomial.polynomial.polyval(t, c.astype(np.float64))))))
