"""CPU oracle for the backward pass of the sparse-gated MoE layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests and bench.py's
CPU-baseline leg may import or run it; it shares no code with the HIP path.

The gradients are those of

    L = sum(dy * y) + aux_coef[0] * load_balance_loss(importance)
                    + aux_coef[1] * importance_loss(importance)

with respect to x, W1, b1, W2, b2, w_gate, w_noise and logit_bias, where y
is the layer output of moe_oracle.forward and importance the per-expert sum
of the gate weights (moe_oracle.expert_importance). The routing (each
token's top-k experts and the capacity slots) is a selection, constant
almost everywhere: gradients flow only through the selected experts' gate
weights and expert outputs (sparse gating keeps only the Top-K experts'
gradient, "MoE稀疏计算加速技术解析与应用实践" §2.1; the auxiliary losses are
added to the total loss on the same page's §4.1 and on
"MoE架构：突破单卡算力瓶颈的密钥" §3.1). A choice dropped by the capacity
limit contributes nothing to y, so its weight receives no gradient from y;
it still counts in the importance and so in the auxiliary losses. The noise
tensor eps is an input, not a parameter. Everything is float64, by the
chain rule through the forward definition:

    y_t = sum over kept j of w_tj E_e(x_t),  E_e(x) = GELU(x W1_e + b1_e) W2_e + b2_e
    g_tj = dL/dw_tj = dy_t . E_e(x_t) (kept j) + dL_aux/dimportance_e
    renorm = 1: w_t = softmax(selected logits)      -> dl = w (g - sum w g) on the selected
    renorm = 0: w_tj = softmax(all logits)_e        -> dl = p (G - sum p G), G = g scattered
    plain: l = x W_g + b;  noisy: l = x W_g + eps * softplus(x W_n) + b

Only the plain and noisy gates are covered (the cosine gate's backward is not
built).
"""
from __future__ import annotations

import math
from typing import Dict, Optional, Sequence

import numpy as np
import torch

from . import moe_oracle as O


def gelu_grad(u: np.ndarray) -> np.ndarray:
    """d GELU(u) / du = Phi(u) + u phi(u) (erf form)."""
    u = O.f64(u)
    cdf = 0.5 * (1.0 + torch.special.erf(torch.from_numpy(u / math.sqrt(2.0))).numpy())
    pdf = np.exp(-0.5 * u * u) / math.sqrt(2.0 * math.pi)
    return cdf + u * pdf


def sigmoid(z: np.ndarray) -> np.ndarray:
    """d softplus(z) / dz, written without overflow for either sign."""
    z = O.f64(z)
    e = np.exp(-np.abs(z))
    return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def importance_grad(importance: np.ndarray, aux_coef: Sequence[float]) -> np.ndarray:
    """d(aux_coef[0] * load_balance_loss + aux_coef[1] * importance_loss) / d importance.
    load_balance_loss = sum_e (mean - imp_e)^2 gives 2 (imp_e - mean) (the mean's own
    derivative cancels, as the deviations sum to zero); importance_loss = 0.1 std (N - 1
    denominator) gives 0.1 (imp_e - mean) / ((N - 1) std), taken as 0 where std = 0 (no
    derivative there; zero is the subgradient of minimal norm)."""
    imp = O.f64(importance)
    N = imp.shape[0]
    dev = imp - imp.mean()
    g = aux_coef[0] * 2.0 * dev
    if aux_coef[1] != 0.0 and N > 1:
        std = math.sqrt((dev ** 2).sum() / (N - 1))
        if std > 0:
            g = g + aux_coef[1] * 0.1 * dev / ((N - 1) * std)
    return g


def backward(spec, inp, r: Dict[str, np.ndarray], dy: np.ndarray,
             aux_coef: Sequence[float] = (0.0, 0.0)) -> Dict[str, Optional[np.ndarray]]:
    """Gradients of L (module docstring) given a routing r from moe_oracle.route
    (its logits are the ones the weights were computed from)."""
    if spec.gate == "cosine":
        raise NotImplementedError("the cosine gate's backward is not built")
    T, k, N = spec.T, spec.k, spec.N
    x = O.f64(inp.x)
    dy = O.f64(dy)
    idx, w, row_of, tor, off = r["topk_idx"], O.f64(r["topk_w"]), r["row_of"], r["token_of_row"], r["off"]
    A = int(off[-1])
    d, h = spec.d, spec.h
    # forward quantities of the expert rows
    x_perm = x[tor // k]
    U = np.zeros((A, h))
    H = np.zeros((A, h))
    Y = np.zeros((A, d))
    for e in range(N):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            U[lo:hi] = x_perm[lo:hi] @ O.f64(inp.W1[e]) + (0.0 if inp.b1 is None else O.f64(inp.b1[e]))
            H[lo:hi] = O.gelu(U[lo:hi])
            Y[lo:hi] = H[lo:hi] @ O.f64(inp.W2[e]) + (0.0 if inp.b2 is None else O.f64(inp.b2[e]))
    # gradient of each gate weight
    g = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            rr = int(row_of[t * k + j])
            if rr >= 0:
                g[t, j] = dy[t] @ Y[rr]
    if aux_coef[0] != 0.0 or aux_coef[1] != 0.0:
        dimp = importance_grad(O.expert_importance(N, idx, w), aux_coef)
        g = g + dimp[idx]
    # through the softmax to the logits
    logits = O.f64(r["logits"])
    dl = np.zeros((T, N))
    if spec.renorm:
        s = (w * g).sum(axis=1, keepdims=True)
        np.put_along_axis(dl, idx, w * (g - s), axis=1)
    else:
        p = O.softmax(logits)
        G = np.zeros((T, N))
        np.put_along_axis(G, idx, g, axis=1)
        dl = p * (G - (p * G).sum(axis=1, keepdims=True))
    # expert rows
    dY = np.zeros((A, d))
    for t in range(T):
        for j in range(k):
            rr = int(row_of[t * k + j])
            if rr >= 0:
                dY[rr] = w[t, j] * dy[t]
    dW1 = np.zeros((N, d, h))
    dW2 = np.zeros((N, h, d))
    db1 = np.zeros((N, h))
    db2 = np.zeros((N, d))
    dx_perm = np.zeros((A, d))
    dU_all = np.zeros((A, h))
    for e in range(N):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi == lo:
            continue
        dW2[e] = H[lo:hi].T @ dY[lo:hi]
        db2[e] = dY[lo:hi].sum(axis=0)
        dH = dY[lo:hi] @ O.f64(inp.W2[e]).T
        dU = dH * gelu_grad(U[lo:hi])
        dU_all[lo:hi] = dU
        dW1[e] = x_perm[lo:hi].T @ dU
        db1[e] = dU.sum(axis=0)
        dx_perm[lo:hi] = dU @ O.f64(inp.W1[e]).T
    dx = np.zeros((T, d))
    for t in range(T):
        for j in range(k):
            rr = int(row_of[t * k + j])
            if rr >= 0:
                dx[t] += dx_perm[rr]
    # the gate
    dw_gate = x.T @ dl
    dx = dx + dl @ O.f64(inp.w_gate).T
    dw_noise = None
    if spec.gate == "noisy":
        dz = dl * O.f64(inp.noise) * sigmoid(x @ O.f64(inp.w_noise))
        dw_noise = x.T @ dz
        dx = dx + dz @ O.f64(inp.w_noise).T
    return dict(dx=dx, dW1=dW1, dW2=dW2, db1=None if inp.b1 is None else db1,
                db2=None if inp.b2 is None else db2, dw_gate=dw_gate, dw_noise=dw_noise,
                dlogit_bias=None if inp.logit_bias is None else dl.sum(axis=0),
                dlogits=dl, dweights=g, dU=dU_all, dY=dY, U=U, H=H, Y=Y, dx_perm=dx_perm)
