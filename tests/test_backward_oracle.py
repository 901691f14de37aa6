"""Pins of the backward oracle (oracle/moe_backward_oracle.py) to facts that
do not come from it: central finite differences of the forward oracle's loss
in float64 (the routing held fixed, and checked unchanged at each probe), an
independent PyTorch autograd re-expression of the layer written from its
definition, and the closed form of a single expert. CPU only."""
import copy

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from mixture_experts_sparse_gate_amd import workloads
from mixture_experts_sparse_gate_amd.inputs import make_inputs, make_output_grad
from oracle import moe_backward_oracle as B
from oracle import moe_oracle as O


def _spec(gate="noisy", renorm=True, **kw):
    base = dict(name="bwd", T=9, d=6, h=5, N=4, k=2, capacity_factor=0.8, gate=gate, renorm=renorm,
                dtype="f32", expert_bias=True, zipf_s=0.5)
    base.update(kw)
    return workloads.MoESpec(**base)


def _f64_inputs(spec, seed):
    inp = make_inputs(spec, seed)
    out = copy.copy(inp)
    for name in ("x", "w_gate", "w_noise", "noise", "logit_bias", "W1", "W2", "b1", "b2"):
        v = getattr(inp, name)
        if v is not None:
            setattr(out, name, np.array(v, np.float64))
    return out


def _loss(spec, inp, dy, aux, ref_route):
    """The forward oracle's loss; asserts the routing equals ref_route's."""
    out = O.forward(spec, inp)
    assert np.array_equal(out["topk_idx"], ref_route["topk_idx"]) and np.array_equal(out["row_of"], ref_route["row_of"]), \
        "a probe changed the routing"
    imp = O.expert_importance(spec.N, out["topk_idx"], out["topk_w"])
    L = float((np.asarray(dy, np.float64) * out["y"]).sum())
    L += aux[0] * O.load_balance_loss(imp)
    if aux[1]:
        L += aux[1] * O.importance_loss(imp)
    return L


PARAMS = ["x", "W1", "W2", "b1", "b2", "w_gate", "w_noise", "logit_bias"]


@pytest.mark.parametrize("gate,renorm,aux", [("noisy", True, (0.0, 0.0)), ("noisy", False, (0.3, 0.7)),
                                             ("softmax", True, (0.5, 0.0)), ("softmax", False, (0.0, 2.0))])
def test_gradients_match_central_differences(gate, renorm, aux):
    spec = _spec(gate, renorm)
    inp = _f64_inputs(spec, 3)
    dy = np.array(make_output_grad(spec, 3), np.float64)
    r = O.route(spec, inp)
    assert (r["row_of"] < 0).any(), "the case must drop some choices"
    g = B.backward(spec, inp, r, dy, aux)
    rng = np.random.default_rng(0)
    eps = 1e-6
    checked = 0
    for name in PARAMS:
        arr = getattr(inp, name)
        if arr is None:
            continue
        key = {"x": "dx", "W1": "dW1", "W2": "dW2", "b1": "db1", "b2": "db2", "w_gate": "dw_gate",
               "w_noise": "dw_noise", "logit_bias": "dlogit_bias"}[name]
        for _ in range(6):
            pos = tuple(int(rng.integers(0, n)) for n in arr.shape)
            keep = arr[pos]
            arr[pos] = keep + eps
            lp = _loss(spec, inp, dy, aux, r)
            arr[pos] = keep - eps
            lm = _loss(spec, inp, dy, aux, r)
            arr[pos] = keep
            fd = (lp - lm) / (2 * eps)
            an = g[key][pos]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), f"{key}{pos}: analytic {an} vs central difference {fd}"
            checked += 1
    assert checked >= 40


def _torch_layer_loss(spec, inp, dy, r, aux):
    """The layer written from its definition in torch float64 (the routing r
    held fixed), returning L and the leaf tensors."""
    t = lambda a: torch.tensor(np.asarray(a, np.float64), requires_grad=True)
    x, Wg, W1, W2 = t(inp.x), t(inp.w_gate), t(inp.W1), t(inp.W2)
    b1, b2 = t(inp.b1), t(inp.b2)
    bias = t(inp.logit_bias)
    leaves = dict(x=x, w_gate=Wg, W1=W1, W2=W2, b1=b1, b2=b2, logit_bias=bias)
    l = x @ Wg
    if spec.gate == "noisy":
        Wn = t(inp.w_noise)
        leaves["w_noise"] = Wn
        l = l + torch.tensor(np.asarray(inp.noise, np.float64)) * F.softplus(x @ Wn)
    l = l + bias
    idx = torch.tensor(r["topk_idx"])
    if spec.renorm:
        w = torch.softmax(torch.gather(l, 1, idx), dim=1)
    else:
        w = torch.gather(torch.softmax(l, dim=1), 1, idx)
    kept = torch.tensor(r["row_of"].reshape(spec.T, spec.k) >= 0)
    ys = []
    for ti in range(spec.T):
        acc = torch.zeros(spec.d, dtype=torch.float64)
        for j in range(spec.k):
            if kept[ti, j]:
                e = int(idx[ti, j])
                acc = acc + w[ti, j] * (F.gelu(x[ti] @ W1[e] + b1[e]) @ W2[e] + b2[e])
        ys.append(acc)
    y = torch.stack(ys)
    imp = torch.zeros(spec.N, dtype=torch.float64).scatter_add(0, idx.reshape(-1), w.reshape(-1))
    L = (torch.tensor(np.asarray(dy, np.float64)) * y).sum()
    L = L + aux[0] * ((imp.mean() - imp) ** 2).sum() + aux[1] * 0.1 * imp.std()
    return L, leaves


@pytest.mark.parametrize("gate,renorm", [("noisy", True), ("noisy", False), ("softmax", True), ("softmax", False)])
def test_gradients_match_torch_autograd(gate, renorm):
    spec = _spec(gate, renorm, T=20, d=8, h=12, N=5, k=3, capacity_factor=0.9)
    inp = _f64_inputs(spec, 5)
    dy = make_output_grad(spec, 5)
    r = O.route(spec, inp)
    aux = (0.25, 1.5)
    g = B.backward(spec, inp, r, dy, aux)
    L, leaves = _torch_layer_loss(spec, inp, dy, r, aux)
    L.backward()
    key = {"x": "dx", "W1": "dW1", "W2": "dW2", "b1": "db1", "b2": "db2", "w_gate": "dw_gate",
           "w_noise": "dw_noise", "logit_bias": "dlogit_bias"}
    for name, leaf in leaves.items():
        np.testing.assert_allclose(g[key[name]], leaf.grad.numpy(), rtol=1e-10, atol=1e-12, err_msg=name)


def test_single_expert_backward_is_the_ffn_backward():
    """N = 1, k = 1: every weight is exactly 1, so the gate gets no gradient
    and dx, dW1, dW2 are those of one Linear-GELU-Linear block."""
    spec = _spec("softmax", False, T=11, N=1, k=1, capacity_factor=1.0, zipf_s=0.0)
    inp = _f64_inputs(spec, 8)
    dy = make_output_grad(spec, 8)
    g = B.backward(spec, inp, O.route(spec, inp), dy)
    x = torch.tensor(inp.x, requires_grad=True)
    W1 = torch.tensor(inp.W1[0], requires_grad=True)
    W2 = torch.tensor(inp.W2[0], requires_grad=True)
    b1 = torch.tensor(inp.b1[0], requires_grad=True)
    b2 = torch.tensor(inp.b2[0], requires_grad=True)
    y = F.gelu(x @ W1 + b1) @ W2 + b2
    (torch.tensor(np.asarray(dy, np.float64)) * y).sum().backward()
    for got, want in ((g["dx"], x.grad), (g["dW1"][0], W1.grad), (g["dW2"][0], W2.grad), (g["db1"][0], b1.grad),
                      (g["db2"][0], b2.grad)):
        np.testing.assert_allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)
    assert not g["dw_gate"].any()


def test_gelu_grad_and_sigmoid():
    u = np.linspace(-9, 9, 181)
    ut = torch.tensor(u, requires_grad=True)
    F.gelu(ut).sum().backward()
    np.testing.assert_allclose(B.gelu_grad(u), ut.grad.numpy(), rtol=1e-12, atol=1e-15)
    z = np.array([-800.0, -30.0, -1.0, 0.0, 2.0, 40.0, 800.0])
    zt = torch.tensor(z, requires_grad=True)
    F.softplus(zt).sum().backward()
    np.testing.assert_allclose(B.sigmoid(z), zt.grad.numpy(), rtol=1e-12, atol=0)


def test_importance_loss_gradient_at_uniform_load_is_zero():
    imp = np.full(6, 3.0)
    assert not B.importance_grad(imp, (1.0, 1.0)).any()
