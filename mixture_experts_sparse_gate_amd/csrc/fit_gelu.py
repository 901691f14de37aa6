"""Derives the GELU constants in gemm.hip (run by hand; nothing builds from it).

GELU(u) = u * Phi(u) with Phi(u) = erfc(-u / sqrt(2)) / 2. For x = |u| / sqrt(2):
    Phi(u) = 1 - erfc(x) / 2   (u >= 0)        Phi(u) = erfc(x) / 2   (u < 0)
and erfc(x) = R(x) exp(-x^2), where the scaled complement R(x) = erfc(x) exp(x^2)
is smooth and decreasing from 1 towards 1 / (x sqrt(pi)). R is fitted as a
degree-9 polynomial in t = 1 / (1 + 0.35 x) by least squares on its relative
error over x in [0, 9.3] (past 9.3, exp(-x^2) is below fp32's normal range).
A relative error in R is the same relative error in erfc, so Phi keeps its
relative accuracy in the negative tail, where 1 + erf(x) would cancel.

    python fit_gelu.py        prints the constants as C literals
"""
import numpy as np
from scipy.special import erfcx

P = 0.35
DEG = 9
X_MAX = 9.3


def fit():
    x = np.linspace(0.0, X_MAX, 400001)
    r = erfcx(x)
    t = 1.0 / (1.0 + P * x)
    v = np.vander(t, DEG + 1, increasing=True)
    w = 1.0 / r
    c, *_ = np.linalg.lstsq(v * w[:, None], r * w, rcond=None)
    return c.astype(np.float32)


if __name__ == "__main__":
    c = fit()
    print(", ".join("%.9ef" % v for v in c))
