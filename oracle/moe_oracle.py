"""CPU oracle for the sparse-gated MoE layer forward pass.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the package smoke check
(``__graft_entry__.smoke``) and the CPU-baseline leg of ``bench.py`` may
import or run anything in this directory. It shares no code with the HIP
path and imports nothing from it: it receives plain NumPy arrays.

Everything is computed in float64 from the exact values the GPU receives
(bf16 or fp32 inputs widen exactly to float64). Each step follows the pages
in their order and notation:

  gate logits      clean_logits = x W_g; noisy_logits = clean_logits +
                   eps * softplus(x W_n)        [noisy top-k gating code on
                   "MoE稀疏计算加速技术解析与应用实践" §2.1 and on
                   "MoE架构：稀疏激活机制如何提升模型计算效率" §2.1]
                   cosine: cos(x P, e_j) / tau  [cosine_top gate named on
                   "4大技术模块掌握Tutel MoE…" (dynamic routing section); the
                   formula is the cosine workload's own definition]
  top-k            top_k_logits, top_k_indices = topk(logits)   [same §2.1 pages]
  gate weights     softmax over the k selected logits (renormalised), or the
                   full softmax probability of each selected expert (the
                   top-1 MOELayer example on "PyTorch-CUDA-v2.6镜像是否支持MoE
                   稀疏激活架构", section "PyTorch v2.6：为动态计算而生")
  capacity         C = ceil(capacity_factor * T * k / N), tokens dropped in
                   token order once an expert is full (capacity_factor on
                   "MoE稀疏计算加速技术解析与应用实践" §3.2 and on the Tutel page)
  grouping         group the tokens by chosen expert, then one batched matmul
                   per group ["MoE架构：稀疏激活机制如何提升模型计算效率" §3.1]
  expert           E_i(x) = Linear(d->h) -> GELU -> Linear(h->d)
                   ["MoE稀疏计算加速技术解析与应用实践" §3.2]
  combine          y = sum_i g_i(x) E_i(x) over the kept experts
                   ["MoE架构：突破单卡算力瓶颈的密钥" §1.2]
  load balance     importance_e = sum_t gates[t, e] (before drops);
                   load_balance_loss = sum_e (mean - importance_e)^2
                   ["MoE架构：突破单卡算力瓶颈的密钥" §3.1];
                   importance loss = 0.1 std(importance)
                   ["MoE稀疏计算加速技术解析与应用实践" §4.1]

Readings where the pages are silent (each is listed with its reason in the
design notes): ties in top-k go to the lower expert index; selection compares
logits, not probabilities; a dropped assignment contributes nothing and the
surviving weights are not renormalised; a token with every choice dropped
outputs zeros; GELU is the erf form; softplus(z) = max(z, 0) + log1p(exp(-|z|));
the cosine norms are clamped below at 1e-12; the per-expert logit bias is
added after the 1/tau scaling.
"""
from __future__ import annotations

import math
from typing import Dict, Optional

import numpy as np
import torch


def f64(a: Optional[np.ndarray]) -> Optional[np.ndarray]:
    return None if a is None else np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# Gate logits
# ----------------------------------------------------------------------------

def softplus(z: np.ndarray) -> np.ndarray:
    """softplus(z) = log(1 + e^z), written so that it neither overflows nor
    loses the small tail: max(z, 0) + log1p(e^-|z|)."""
    z = f64(z)
    return np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))


def clean_logits(x: np.ndarray, w_gate: np.ndarray) -> np.ndarray:
    """The gate's linear map without bias: x W_g, [T, d] x [d, N] -> [T, N]."""
    return f64(x) @ f64(w_gate)


def noisy_logits(x: np.ndarray, w_gate: np.ndarray, w_noise: np.ndarray,
                 noise: np.ndarray) -> np.ndarray:
    """Noisy top-k gating logits: clean_logits + eps * softplus(noise_logits),
    with noise_logits = x W_n and eps the caller's standard-normal tensor
    (the pages draw it with randn_like; here it is an input)."""
    noise_logits = f64(x) @ f64(w_noise)
    return clean_logits(x, w_gate) + f64(noise) * softplus(noise_logits)


def cosine_logits(x: np.ndarray, proj: np.ndarray, expert_emb: np.ndarray,
                  inv_temperature: float) -> np.ndarray:
    """Cosine gate: z = x P; logit_j = cos(z, e_j) / tau, norms clamped at 1e-12."""
    z = f64(x) @ f64(proj)
    e = f64(expert_emb)
    zn = np.maximum(np.sqrt((z * z).sum(axis=1)), 1e-12)
    en = np.maximum(np.sqrt((e * e).sum(axis=1)), 1e-12)
    cos = (z @ e.T) / zn[:, None] / en[None, :]
    return cos * float(np.float32(inv_temperature))


def gate_logits(gate: str, x, w_gate=None, w_noise=None, noise=None, proj=None,
                expert_emb=None, inv_temperature: float = 0.0,
                logit_bias=None) -> np.ndarray:
    if gate == "softmax":
        l = clean_logits(x, w_gate)
    elif gate == "noisy":
        l = noisy_logits(x, w_gate, w_noise, noise)
    elif gate == "cosine":
        l = cosine_logits(x, proj, expert_emb, inv_temperature)
    else:
        raise ValueError(gate)
    if logit_bias is not None:
        l = l + f64(logit_bias)[None, :]
    return l


# ----------------------------------------------------------------------------
# Top-k selection and gate weights
# ----------------------------------------------------------------------------

def top_k(logits: np.ndarray, k: int):
    """top_k_indices[t] = the k experts with the largest logits, ordered by
    logit descending; equal logits keep ascending expert index (a stable sort
    of -logits). Returns (top_k_logits, top_k_indices)."""
    l = f64(logits)
    idx = np.argsort(-l, axis=1, kind="stable")[:, :k]
    return np.take_along_axis(l, idx, axis=1), idx.astype(np.int64)


def softmax(v: np.ndarray) -> np.ndarray:
    v = f64(v)
    m = v.max(axis=1, keepdims=True)
    e = np.exp(v - m)
    return e / e.sum(axis=1, keepdims=True)


def gate_weights(logits: np.ndarray, top_k_logits: np.ndarray, top_k_indices: np.ndarray,
                 renorm: bool) -> np.ndarray:
    """g_i(x) of each selected expert: softmax(top_k_logits) when renormalised,
    otherwise softmax over all N logits, read at the selected experts."""
    if renorm:
        return softmax(top_k_logits)
    return np.take_along_axis(softmax(logits), top_k_indices, axis=1)


def sparse_gates(N: int, top_k_indices: np.ndarray, w: np.ndarray) -> np.ndarray:
    """Dense [T, N] gate matrix: zeros with the selected weights scattered in."""
    g = np.zeros((top_k_indices.shape[0], N), np.float64)
    np.put_along_axis(g, top_k_indices, w, axis=1)
    return g


# ----------------------------------------------------------------------------
# Load-balance terms of the gate
# ----------------------------------------------------------------------------

def expert_importance(N: int, top_k_indices: np.ndarray, w: np.ndarray) -> np.ndarray:
    """The load each expert receives from the gate: the column sums of the
    sparse gate matrix, before any capacity drop (gate_output.sum(dim=0) on
    "MoE架构：突破单卡算力瓶颈的密钥" §3.1, gates.sum(dim=0) on
    "MoE稀疏计算加速技术解析与应用实践" §4.1)."""
    return sparse_gates(N, top_k_indices, w).sum(axis=0)


def load_balance_loss(importance: np.ndarray) -> float:
    """The sum over experts of (mean load - load)^2
    ["MoE架构：突破单卡算力瓶颈的密钥" §3.1, load_balance_loss]."""
    mean = importance.mean()
    return float(((mean - importance) ** 2).sum())


def importance_loss(importance: np.ndarray) -> float:
    """0.1 times the standard deviation of the loads, with torch.std's default
    N - 1 denominator ["MoE稀疏计算加速技术解析与应用实践" §4.1,
    expert_importance_loss]; NaN for a single expert, as that estimate is."""
    N = importance.shape[0]
    if N < 2:
        return float("nan")
    return 0.1 * float(np.sqrt(((importance - importance.mean()) ** 2).sum() / (N - 1)))


# ----------------------------------------------------------------------------
# Capacity and token-order slots
# ----------------------------------------------------------------------------

def capacity(T: int, k: int, N: int, capacity_factor: float) -> int:
    """C = ceil(capacity_factor * T * k / N), evaluated in IEEE double as
    (cf * (T*k)) / N, then clamped to T (an expert never holds more than T rows)."""
    return int(min(T, math.ceil((capacity_factor * (T * k)) / N)))


def assign_slots(top_k_indices: np.ndarray, N: int, C: int):
    """Walk the tokens in order; each (t, j) takes the next free slot of its
    expert, and is dropped once the expert already holds C tokens.

    Returns count[N] (demand), kept[N], off[N+1] (exclusive scan of kept in
    expert order), row_of[T*k] (row in the expert-grouped buffer, -1 when
    dropped), token_of_row[A] (t*k + j of each row)."""
    T, k = top_k_indices.shape
    fill = [0] * N
    slot = [[0] * k for _ in range(T)]
    for t in range(T):
        for j in range(k):
            e = int(top_k_indices[t, j])
            slot[t][j] = fill[e]
            fill[e] += 1
    count = np.array(fill, np.int64)
    kept = np.minimum(count, C)
    off = np.zeros(N + 1, np.int64)
    off[1:] = np.cumsum(kept)
    row_of = np.full(T * k, -1, np.int64)
    token_of_row = np.full(int(off[N]), -1, np.int64)
    for t in range(T):
        for j in range(k):
            e = int(top_k_indices[t, j])
            s = slot[t][j]
            if s < C:
                r = int(off[e]) + s
                row_of[t * k + j] = r
                token_of_row[r] = t * k + j
    return count, kept, off, row_of, token_of_row


# ----------------------------------------------------------------------------
# Experts and combine
# ----------------------------------------------------------------------------

def gelu(u: np.ndarray) -> np.ndarray:
    """GELU(u) = u * Phi(u) = u/2 * (1 + erf(u / sqrt 2))."""
    u = f64(u)
    return 0.5 * u * (1.0 + torch.special.erf(torch.from_numpy(u / math.sqrt(2.0))).numpy())


def expert_ffn(xe: np.ndarray, W1e: np.ndarray, W2e: np.ndarray,
               b1e: Optional[np.ndarray] = None, b2e: Optional[np.ndarray] = None):
    """E_i(x) = GELU(x W1 + b1) W2 + b2 for one expert, on a group of rows.
    Returns (hidden, out)."""
    hid = f64(xe) @ f64(W1e)
    if b1e is not None:
        hid = hid + f64(b1e)[None, :]
    hid = gelu(hid)
    out = hid @ f64(W2e)
    if b2e is not None:
        out = out + f64(b2e)[None, :]
    return hid, out


def grouped_experts(x_perm: np.ndarray, off: np.ndarray, W1, W2, b1=None, b2=None):
    """Run each expert once on its contiguous group of rows [off[e], off[e+1])."""
    N = len(off) - 1
    A = int(off[N])
    h = W1.shape[2]
    H = np.zeros((A, h), np.float64)
    Y = np.zeros((A, W2.shape[2]), np.float64)
    for e in range(N):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            H[lo:hi], Y[lo:hi] = expert_ffn(x_perm[lo:hi], W1[e], W2[e],
                                            None if b1 is None else b1[e],
                                            None if b2 is None else b2[e])
    return H, Y


def combine(y_perm: np.ndarray, row_of: np.ndarray, w: np.ndarray, T: int, k: int) -> np.ndarray:
    """y[t] = sum over kept j of g_j(x_t) * E_j(x_t); zeros if all k were dropped."""
    d = y_perm.shape[1]
    y = np.zeros((T, d), np.float64)
    for t in range(T):
        for j in range(k):
            r = int(row_of[t * k + j])
            if r >= 0:
                y[t] += w[t, j] * y_perm[r]
    return y


# ----------------------------------------------------------------------------
# The whole layer
# ----------------------------------------------------------------------------

def route(spec, inp, logits_override: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """Gate, select, weigh, and assign capacity slots.

    ``logits_override`` replaces the oracle's own fp64 logits (used to check
    routing given the GPU's fp32 logits)."""
    if logits_override is None:
        logits = gate_logits(spec.gate, inp.x, inp.w_gate, inp.w_noise, inp.noise, inp.proj,
                             inp.expert_emb, spec.inv_temperature, inp.logit_bias)
    else:
        logits = f64(logits_override)
    tkl, idx = top_k(logits, spec.k)
    w = gate_weights(logits, tkl, idx, spec.renorm)
    C = capacity(spec.T, spec.k, spec.N, spec.capacity_factor)
    count, kept, off, row_of, token_of_row = assign_slots(idx, spec.N, C)
    return dict(logits=logits, topk_idx=idx, topk_w=w, capacity=C, count=count, kept=kept,
                off=off, row_of=row_of, token_of_row=token_of_row)


def forward(spec, inp, logits_override: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The full layer: route, permute, grouped experts, combine."""
    r = route(spec, inp, logits_override)
    x = f64(inp.x)
    k = spec.k
    x_perm = x[r["token_of_row"] // k]
    H, Y = grouped_experts(x_perm, r["off"], inp.W1, inp.W2, inp.b1, inp.b2)
    y = combine(Y, r["row_of"], r["topk_w"], spec.T, k)
    r.update(x_perm=x_perm, H=H, y_perm=Y, y=y)
    return r
