"""Fit of the complementary error function used by the GeLU epilogues.

    python megatron_tensor_transformer_rank_amd/csrc/fit_erfc.py

For x >= 0 the kernels evaluate

    erfc(x) = t * P(t) * exp(-x^2),   t = 1 / (1 + p x),   P of degree 7,

so that the normal CDF and density of the GeLU and its derivative share one
exponential: Phi(u) = 0.5 erfc(|u| / sqrt 2) for u < 0 (1 minus it for
u >= 0) and phi(u) = exp(-u^2 / 2) / sqrt(2 pi).  The scaled function
erfc(x) exp(x^2) is smooth and bounded on t in (0, 1] and behaves like
p t / sqrt(pi) as t -> 0, so t * P(t) fits it closely with no constant term.

P is fitted here on the relative error at Chebyshev-spaced points of t by
Lawson's algorithm (iteratively reweighted least squares, which tends to the
minimax fit), with scipy's erfcx as the target.  This prints the
coefficients pasted into common.h and the maximum relative error of
erfc(x) for x in [0, 30], evaluated in float64 and in float32 Horner form
(tests/test_erfc_fit.py checks the pasted values against the same bound).
"""
import numpy as np
from scipy.special import erfcx

P_SCALE = 0.46
DEGREE = 7          # P has DEGREE + 1 coefficients: t * P(t) is of degree 8


def fit(p=P_SCALE, degree=DEGREE, n=6000, iters=300):
    k = np.arange(n)
    t = 0.5 * (1 - np.cos(np.pi * (k + 0.5) / n))
    t = t[t > 1e-7]
    f = erfcx((1 / t - 1) / p)
    V = np.vander(t, degree + 2, increasing=True)[:, 1:] / f[:, None]   # t^1 .. t^(degree+1), relative
    b = np.ones_like(t)
    w = np.full_like(t, 1 / len(t))
    for _ in range(iters):
        sw = np.sqrt(w)
        c, *_ = np.linalg.lstsq(V * sw[:, None], b * sw, rcond=None)
        r = np.abs(V @ c - b)
        w = w * r
        w /= w.sum()
    return c


def erfc_approx(x, c, p=P_SCALE, dtype=np.float64):
    x = np.asarray(x, dtype)
    t = (dtype(1) / (dtype(1) + dtype(p) * x)).astype(dtype)
    acc = np.full_like(t, dtype(c[-1]))
    for ci in c[-2::-1]:
        acc = (acc * t + dtype(ci)).astype(dtype)
    return (acc * t * np.exp(-(x * x).astype(dtype))).astype(dtype)


if __name__ == "__main__":
    from scipy.special import erfc
    c = fit()
    print("coefficients (t^1 .. t^8):", ", ".join(f"{v:.9e}" for v in c))
    x = np.concatenate([np.linspace(0, 9, 200001), np.geomspace(1e-6, 9, 20001)]).astype(np.float32)
    ref = erfc(x.astype(np.float64))      # at the float32 arguments the kernels see
    for dt in (np.float64, np.float32):
        got = erfc_approx(x, c, dtype=dt).astype(np.float64)
        for lo, hi in ((0, 4), (4, 9)):
            m = (x >= lo) & (x <= hi)
            print(dt.__name__, f"max relative error of erfc on [{lo}, {hi}]:", f"{np.abs(got[m] / ref[m] - 1).max():.2e}")
