"""Comparison helpers for the GPU parity tests (HIP path vs the CPU oracle).

Tolerances (derivations in the design notes):
  logits   |l_gpu - l_ref| <= 2e-4 * (1 + |l_ref|): identical inputs, fp32
           accumulation in a different order than the fp64 oracle
  weights  relative 5e-6 against the oracle's fp64 softmax of the GPU's own
           fp32 logits (fp32 exp and sum; the exponent's argument l - max is
           rounded once in fp32)
  rows     per row max|y - y_ref| / max|y_ref| <= 2e-2 for bf16 (fp32
           accumulation, H and outputs rounded to bf16) and <= 1e-5 for fp32;
           a row whose reference is all zeros must be exactly zero
  routing, slots, offsets, row maps: bit-exact given the GPU's fp32 logits
"""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_oracle as O

ROW_TOL = {"bf16": 2e-2, "f32": 1e-5}
LOGIT_TOL = 2e-4
WEIGHT_RTOL = 5e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def host(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()


def row_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max|got - ref| / max|ref|; zero reference rows must be exactly zero."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    den = np.abs(ref).max(axis=1)
    num = np.abs(got - ref).max(axis=1)
    zero = den == 0
    assert np.all(num[zero] == 0), "rows with an all-zero reference must be exactly zero"
    return float((num[~zero] / den[~zero]).max()) if np.any(~zero) else 0.0


def check_logits(spec, inp, logits_gpu: np.ndarray):
    ref = O.gate_logits(spec.gate, inp.x, inp.w_gate, inp.w_noise, inp.noise, inp.proj, inp.expert_emb,
                        spec.inv_temperature, inp.logit_bias)
    err = np.abs(logits_gpu.astype(np.float64) - ref)
    bound = LOGIT_TOL * (1 + np.abs(ref))
    worst = float((err / bound).max())
    assert worst <= 1.0, f"logits off by {worst:.3g} x tolerance (max abs err {err.max():.3g})"
    return ref


def check_routing(spec, inp, dev, logits_gpu: np.ndarray):
    """Oracle routing on the GPU's fp32 logits must equal the GPU's, bit for bit."""
    r = O.route(spec, inp, logits_override=logits_gpu)
    idx = host(dev.topk_idx)
    np.testing.assert_array_equal(idx, r["topk_idx"], err_msg="top-k indices")
    w = host(dev.topk_w).astype(np.float64)
    np.testing.assert_allclose(w, r["topk_w"], rtol=WEIGHT_RTOL, atol=0, err_msg="gate weights")
    A = int(r["off"][-1])
    np.testing.assert_array_equal(host(dev.expert_count), r["count"], err_msg="expert_count")
    np.testing.assert_array_equal(host(dev.expert_off), r["off"], err_msg="expert_off")
    np.testing.assert_array_equal(host(dev.row_of), r["row_of"], err_msg="row_of")
    np.testing.assert_array_equal(host(dev.token_of_row)[:A], r["token_of_row"], err_msg="token_of_row")
    assert A + int((r["row_of"] < 0).sum()) == spec.T * spec.k
    assert np.all(r["kept"] <= r["capacity"])
    return r


def check_x_perm(spec, inp, dev, r, rows=None):
    """x_perm rows are the tokens' rows of x, bitwise."""
    A = int(r["off"][-1])
    rows = np.arange(A) if rows is None else np.asarray(rows)
    if rows.size == 0:
        return
    got = dev.x_perm[torch.as_tensor(rows, device=dev.x_perm.device)]
    want = dev.x[torch.as_tensor(r["token_of_row"][rows] // spec.k, device=dev.x.device)]
    assert torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                       want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32))


def check_ffn(spec, inp, dev, r):
    A = int(r["off"][-1])
    x_perm = O.f64(inp.x)[r["token_of_row"] // spec.k]
    H, Y = O.grouped_experts(x_perm, r["off"], inp.W1, inp.W2, inp.b1, inp.b2)
    eh = row_rel_err(host(dev.H)[:A], H)
    ey = row_rel_err(host(dev.y_perm)[:A], Y)
    tol = ROW_TOL[spec.dtype]
    assert eh <= tol, f"H row error {eh:.3g} > {tol}"
    assert ey <= tol, f"y_perm row error {ey:.3g} > {tol}"
    return H, Y, eh, ey


def check_output(spec, inp, dev, r, Y):
    y_ref = O.combine(Y, r["row_of"], r["topk_w"], spec.T, spec.k)
    e = row_rel_err(host(dev.y), y_ref)
    tol = ROW_TOL[spec.dtype]
    assert e <= tol, f"y row error {e:.3g} > {tol}"
    return e
