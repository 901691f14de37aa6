// The expert's GELU (erf form) as the kernels evaluate it; the fitted
// constants come from fit_gelu.py beside this file.
#pragma once

#include "common.hpp"

namespace moe {

// GELU(u) = u Phi(u), Phi the standard normal CDF (the erf form of GELU).
// With x = |u| / sqrt(2) and e = erfc(x) / 2 = Phi(-|u|),
//     GELU(u) = max(u, 0) - |u| e
// (u - u e for u >= 0, u e for u < 0), one fma with one rounding. erfc is
// R(t) exp(-x^2), t = 1 / (1 + 0.35 x), R a degree-7 polynomial fitted to
// the scaled complement erfc(x) exp(x^2) on x in [0, 9.3] (fit_gelu.py
// beside this file derives the constants, which are R's halved). Relative
// error of R below 2.3e-6 everywhere, including the negative tail that
// 0.5 u (1 + erf(x)) loses to cancellation; 13 VALU operations and two
// transcendental ones, against about 45 for erff and its two-path branch.
// kGeluR: R's coefficients (halved), lowest degree first.
constexpr float kGeluR[8] = {1.738272113e-04f, 9.559800476e-02f, 1.226225942e-01f, -7.414813619e-03f, 3.312253952e-01f, -3.146309555e-01f, 3.652992249e-01f, -9.287211299e-02f};

__device__ inline float gelu_erf(float u) {
  const float a = fabsf(u);
  // t = 1 / (1 + 0.35 |u| / sqrt(2))
  const float t = __builtin_amdgcn_rcpf(fmaf(a, 0.24748737341529164f, 1.f));
  float r = kGeluR[7];
#pragma unroll
  for (int i = 6; i >= 0; --i) r = fmaf(r, t, kGeluR[i]);
  // exp(-x^2) = 2^(-u^2 log2(e) / 2); below -126 it gives zero (|u| > 13.4)
  const float e = r * __builtin_amdgcn_exp2f((u * -0.72134752044448170f) * u);
  return fmaf(-a, e, fmaxf(u, 0.f));
}

// GELU for results rounded to bf16 afterwards (2^-9 relative). With
// a = |u|, GELU(u) = max(u, 0) - a Q(a) where Q(a) = Phi(-a) is taken as
// p(a)^32: Q^(1/32) falls slowly from 0.979 to 0.52 over a in [0, 6] and a
// degree-6 polynomial p fits it with small relative error (fit_gelu.py beside
// this file derives the constants). a is clamped at 6, where Q is 1e-9.
// Relative error below 3e-5 for |u| <= 6 (negative tail included), absolute
// below 2e-8 beyond; 14 VALU operations and no transcendental ones.
__device__ inline float gelu_erf_bf16(float u) {
  constexpr float g[7] = {9.785726666e-01f, -2.440810017e-02f, -9.400018491e-03f, -9.185104282e-04f, 2.617192222e-04f, -1.624105971e-05f, 3.184045454e-07f};
  const float a = fminf(fabsf(u), 6.f);
  float q = g[6];
#pragma unroll
  for (int i = 5; i >= 0; --i) q = fmaf(q, a, g[i]);
#pragma unroll
  for (int i = 0; i < 5; ++i) q *= q;  // p^32
  return fmaf(-fabsf(u), q, fmaxf(u, 0.f));
}

// d GELU(u) / du = Phi(u) + u phi(u). With a = |u| and E = exp(-u^2 / 2),
// Phi(-a) = R(t) E with gelu_erf's R and t, so Phi(u) = 1 - R(t) E for
// u >= 0 and R(t) E below, and phi(u) = E / sqrt(2 pi): one exponential
// serves both terms. Absolute error below 4e-6 (the device library's
// erfcf and expf cost about 60 VALU operations; this, 14 and two
// transcendental ones).
__device__ inline float gelu_grad(float u) {
  const float a = fabsf(u);
  const float t = __builtin_amdgcn_rcpf(fmaf(a, 0.24748737341529164f, 1.f));
  float r = kGeluR[7];
#pragma unroll
  for (int i = 6; i >= 0; --i) r = fmaf(r, t, kGeluR[i]);
  const float e = __builtin_amdgcn_exp2f((u * -0.72134752044448170f) * u);
  const float q = r * e;  // Phi(-|u|)
  return fmaf(u, 0.39894228040143268f * e, u >= 0.f ? 1.f - q : q);
}

}  // namespace moe
