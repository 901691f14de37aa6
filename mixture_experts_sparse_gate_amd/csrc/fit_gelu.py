"""Derives the GELU constants in gemm.hip (run by hand; nothing builds from it).

GELU(u) = u * Phi(u) with Phi(u) = erfc(-u / sqrt(2)) / 2. For x = |u| / sqrt(2):
    Phi(u) = 1 - erfc(x) / 2   (u >= 0)        Phi(u) = erfc(x) / 2   (u < 0)
and erfc(x) = R(x) exp(-x^2), where the scaled complement R(x) = erfc(x) exp(x^2)
is smooth and decreasing from 1 towards 1 / (x sqrt(pi)). R is fitted as a
degree-7 polynomial in t = 1 / (1 + 0.35 x) by least squares on its relative
error over x in [0, 9.3] (past 9.3, exp(-x^2) is below fp32's normal range);
the largest relative error is 2.3e-6. A relative error in R is the same
relative error in erfc, so Phi keeps its relative accuracy in the negative
tail, where 1 + erf(x) would cancel. The kernel uses the coefficients of
R / 2 (kernel_constants), so that the polynomial gives erfc(x) / 2 after
one multiplication by exp(-x^2).

    python fit_gelu.py        prints the kernel's constants as C literals
"""
import numpy as np
from scipy.special import erfcx

P = 0.35
DEG = 7
X_MAX = 9.3


def fit():
    x = np.linspace(0.0, X_MAX, 400001)
    r = erfcx(x)
    t = 1.0 / (1.0 + P * x)
    v = np.vander(t, DEG + 1, increasing=True)
    w = 1.0 / r
    c, *_ = np.linalg.lstsq(v * w[:, None], r * w, rcond=None)
    return c.astype(np.float32)


def kernel_constants():
    # halving is exact in fp32
    return (np.float32(0.5) * fit()).astype(np.float32)


if __name__ == "__main__":
    c = kernel_constants()
    print(", ".join("%.9ef" % v for v in c))
