"""Seeded synthetic inputs for the MoE layer.

One module feeds both the HIP path and the CPU oracle, so that both see the
same values. It holds no arithmetic of the method itself: it draws normal
variates, scales them to the stated variance and, for bf16 workloads, rounds
them to bf16 (round to nearest even) so that every value is exactly
representable in the arithmetic type the GPU receives.

Recipe (every stream is its own PCG64 generator keyed by (seed, tag, expert)):

  tag 0  x          [T, d]      N(0, 1)
  tag 1  w_gate     [d, N]      N(0, 1/d)
  tag 2  w_noise    [d, N]      N(0, 1/d)          noisy gate only
  tag 3  noise      [T, N]      N(0, 1), fp32      noisy gate only (the eps tensor)
  tag 4  proj       [d, p]      N(0, 1/d)          cosine gate only
  tag 5  expert_emb [N, p]      N(0, 1), fp32      cosine gate only
  tag 6  W1[e]      [d, h]      N(0, 1/d)
  tag 7  W2[e]      [h, d]      N(0, 1/h)
  tag 8  b1[e]      [h]         N(0, 0.01)         only when spec.expert_bias
  tag 9  b2[e]      [d]         N(0, 0.01)         only when spec.expert_bias
  tag 10 dy         [T, d]      N(0, 1)            the upstream gradient of y (make_output_grad)
  logit_bias [N] fp32: 2 * log(Zipf(s) weight of rank e+1), when spec.zipf_s > 0

The second parameter of N(., .) is the variance.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional

import numpy as np

from .workloads import MoESpec

TAG_X, TAG_WG, TAG_WN, TAG_EPS, TAG_P, TAG_E, TAG_W1, TAG_W2, TAG_B1, TAG_B2, TAG_DY = range(11)


def _rng(seed: int, tag: int, expert: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), tag, expert])))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even), in place; returns a."""
    assert a.dtype == np.float32 and a.flags.c_contiguous
    flat = a.reshape(-1)
    step = 1 << 22
    for s in range(0, flat.size, step):
        bits = flat[s:s + step].view(np.uint32)
        lsb = (bits >> 16) & 1
        bits += np.uint32(0x7FFF) + lsb
        bits &= np.uint32(0xFFFF0000)
    return a


def _normal(shape, std: float, seed: int, tag: int, expert: int = 0, bf16: bool = False,
            out: Optional[np.ndarray] = None) -> np.ndarray:
    a = out if out is not None else np.empty(shape, np.float32)
    _rng(seed, tag, expert).standard_normal(dtype=np.float32, out=a)
    if std != 1.0:
        a *= np.float32(std)
    if bf16:
        round_to_bf16(a)
    return a


def zipf_logit_bias(N: int, s: float) -> np.ndarray:
    """b_e = 2 log(w_{e+1}), w_r = r^-s / sum_r' r'^-s (computed in double, stored fp32)."""
    r = np.arange(1, N + 1, dtype=np.float64)
    w = r ** (-s)
    w /= w.sum()
    return (2.0 * np.log(w)).astype(np.float32)


@dataclass
class MoEInputs:
    """Host copies of every layer input. Arrays are float32; for bf16 workloads the
    values of x, w_gate, w_noise, proj, W1, W2, b1, b2 are exactly bf16-representable."""
    spec: MoESpec
    seed: int
    x: np.ndarray
    w_gate: Optional[np.ndarray]
    w_noise: Optional[np.ndarray]
    noise: Optional[np.ndarray]
    proj: Optional[np.ndarray]
    expert_emb: Optional[np.ndarray]
    logit_bias: Optional[np.ndarray]
    W1: np.ndarray
    W2: np.ndarray
    b1: Optional[np.ndarray]
    b2: Optional[np.ndarray]


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def make_inputs(spec: MoESpec, seed: int, with_experts: bool = True) -> MoEInputs:
    T, d, h, N = spec.T, spec.d, spec.h, spec.N
    bf = spec.dtype == "bf16"
    x = _normal((T, d), 1.0, seed, TAG_X, bf16=bf)
    w_gate = w_noise = noise = proj = emb = bias = None
    if spec.gate in ("softmax", "noisy"):
        w_gate = _normal((d, N), d ** -0.5, seed, TAG_WG, bf16=bf)
    if spec.gate == "noisy":
        w_noise = _normal((d, N), d ** -0.5, seed, TAG_WN, bf16=bf)
        noise = _normal((T, N), 1.0, seed, TAG_EPS)
    if spec.gate == "cosine":
        proj = _normal((d, spec.proj_dim), d ** -0.5, seed, TAG_P, bf16=bf)
        emb = _normal((N, spec.proj_dim), 1.0, seed, TAG_E)
    if spec.zipf_s > 0:
        bias = zipf_logit_bias(N, spec.zipf_s)

    if with_experts:
        W1 = np.empty((N, d, h), np.float32)
        W2 = np.empty((N, h, d), np.float32)

        def fill(e):
            _normal((d, h), d ** -0.5, seed, TAG_W1, e, bf16=bf, out=W1[e])
            _normal((h, d), h ** -0.5, seed, TAG_W2, e, bf16=bf, out=W2[e])

        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(N)))
    else:
        W1 = np.empty((0, d, h), np.float32)
        W2 = np.empty((0, h, d), np.float32)
    b1 = b2 = None
    if spec.expert_bias:
        b1 = _normal((N, h), 0.1, seed, TAG_B1, bf16=bf)
        b2 = _normal((N, d), 0.1, seed, TAG_B2, bf16=bf)
    return MoEInputs(spec, seed, x, w_gate, w_noise, noise, proj, emb, bias, W1, W2, b1, b2)


def make_output_grad(spec: MoESpec, seed: int) -> np.ndarray:
    """dy [T, d]: the gradient a following layer hands back for y (float32;
    bf16-exact for bf16 workloads)."""
    return _normal((spec.T, spec.d), 1.0, seed, TAG_DY, bf16=spec.dtype == "bf16")
