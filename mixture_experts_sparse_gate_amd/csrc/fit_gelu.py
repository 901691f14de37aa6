"""Derives the GELU constants in gelu.hpp (run by hand; nothing builds from it).

GELU(u) = u * Phi(u) with Phi(u) = erfc(-u / sqrt(2)) / 2. With a = |u| and
Q(a) = Phi(-a) = erfc(a / sqrt(2)) / 2, GELU(u) = max(u, 0) - a Q(a): u - u Q(u)
for u >= 0 and u Q(-u) for u < 0, and a relative error in Q stays a relative
error in the negative tail, where 1 + erf would cancel. Two forms of Q:

fp32 results (gelu_erf, constants h). With x = a / sqrt(2), erfc(x) =
R(x) exp(-x^2), where the scaled complement R(x) = erfc(x) exp(x^2) is smooth
and decreasing from 1 towards 1 / (x sqrt(pi)). R is fitted as a degree-7
polynomial in t = 1 / (1 + 0.35 x) by least squares on its relative error over
x in [0, 9.3] (past 9.3, exp(-x^2) is below fp32's normal range); the largest
relative error is 2.3e-6. The kernel uses the coefficients of R / 2
(kernel_constants), so that the polynomial gives Q after one multiplication by
exp(-x^2).

bf16 results (gelu_erf_bf16, constants g). Q(a) = p(a)^32, p a degree-6
polynomial in a fitted by least squares on its relative error to Q^(1/32)
over a in [0, 6]; the kernel clamps a at 6 (Q(6) = 1e-9). Q^(1/32) falls
slowly, from 0.979 to 0.52, so a low degree fits it well; five squarings give
Q without a reciprocal or an exponential. Largest relative error of Q 1e-5
(about 2e-5 after fp32 rounding), far below bf16's 2^-9.

    python fit_gelu.py        prints both sets of kernel constants as C literals
"""
import numpy as np
from scipy.special import erfcx, log_ndtr

P = 0.35
DEG = 7
X_MAX = 9.3

POW = 32
DEG_BF16 = 6
A_MAX = 6.0


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


def kernel_constants_bf16():
    a = np.linspace(0.0, A_MAX, 400001)
    target = np.exp(log_ndtr(-a) / POW)  # Q(a)^(1/32), computed in the log domain
    v = np.vander(a, DEG_BF16 + 1, increasing=True)
    w = 1.0 / target
    c, *_ = np.linalg.lstsq(v * w[:, None], target * w, rcond=None)
    return c.astype(np.float32)


if __name__ == "__main__":
    print("h:", ", ".join("%.9ef" % v for v in kernel_constants()))
    print("g:", ", ".join("%.9ef" % v for v in kernel_constants_bf16()))
