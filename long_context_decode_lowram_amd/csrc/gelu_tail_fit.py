"""Derive the constants of the device GELU used by the bf16 MFMA kernel.

GELU(x) = x * Phi(x). With Q(a) = 1 - Phi(a) = erfc(a / sqrt 2) / 2 for a >= 0,
GELU(x) = x - x Q(x) for x >= 0 and x Q(-x) for x < 0, i.e.
GELU(x) = max(x, 0) - |x| Q(|x|). The kernel evaluates log2 Q(a) on [0, 6] by
a degree-4 polynomial in a, clamps a to 6 (6 Q(6) < 1e-8, so beyond 6 the
product min(|x|, 6) Q is below that bound), and takes one exp2. The fit is a
least-squares fit on Chebyshev nodes of the interval, weighted by a Q(a)
(the size of the term the polynomial's error scales), then reweighted a few
dozen times toward the nodes with the largest absolute GELU error (Lawson's
iteration towards the minimax fit). This script prints the coefficients and
the worst absolute GELU error of the float32 evaluation against scipy's erfc
over [-12, 12].

python long_context_decode_lowram_amd/csrc/gelu_tail_fit.py
"""
import numpy as np
from scipy.special import erfc

X, DEG, SHIFT, ROUNDS = 6.0, 4, 0.0, 30


def fit():
    n = 6000
    a = np.cos(np.pi * (np.arange(n) + 0.5) / n) * X / 2 + X / 2
    q = 0.5 * erfc(a / np.sqrt(2.0))
    y = np.log2(q)
    w = a * q + 1e-3
    c = np.polynomial.polynomial.polyfit(a - SHIFT, y, DEG, w=w)
    for _ in range(ROUNDS):
        err = np.abs(a * (np.exp2(np.polynomial.polynomial.polyval(a - SHIFT, c)) - q))
        w = w * (1.0 + 5.0 * err / err.max())
        c = np.polynomial.polynomial.polyfit(a - SHIFT, y, DEG, w=w)
    return c.astype(np.float32)


def gelu_f32(x, c):
    x = np.asarray(x, np.float32)
    a = np.minimum(np.abs(x), np.float32(X)) - np.float32(SHIFT)
    p = np.float32(c[-1])
    for k in range(len(c) - 2, -1, -1):
        p = (p * a + c[k]).astype(np.float32)
    q = np.exp2(p).astype(np.float32)
    t = (np.minimum(np.abs(x), np.float32(X)) * q).astype(np.float32)
    return (np.maximum(x, np.float32(0)) - t).astype(np.float32)


def max_error(c):
    x = np.linspace(-12, 12, 2_000_001)
    ref = x * (1.0 - 0.5 * erfc(x / np.sqrt(2.0)))
    return float(np.max(np.abs(gelu_f32(x, c).astype(np.float64) - ref)))


if __name__ == "__main__":
    c = fit()
    for k, v in enumerate(c):
        print(f"    constexpr float kGeluTail{k} = {float(v)!r}f;")
    print("max |gelu error| =", max_error(c))
