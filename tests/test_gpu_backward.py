"""moe_backward on the GPU against the backward oracle, through the C ABI.

The forward call's routing (moe_forward's inspection outputs) is handed to
both: the oracle recomputes everything else in float64 from the layer's
inputs and the GPU's fp32 logits. Every row of every gradient is compared
(dx per token; dW1 and dW2 per row of each expert's matrix; w_gate and
w_noise per row; the biases per expert): max |got - ref| / max |ref| per row
<= 2e-2 (bf16 operands with fp32 accumulation; U, H, dU and w dy are
rounded to bf16 once each), rows whose reference is zero exactly zero."""
import numpy as np
import pytest
import torch

from mixture_experts_sparse_gate_amd import _lib, api, workloads
from mixture_experts_sparse_gate_amd.inputs import make_inputs, make_output_grad
from oracle import moe_backward_oracle as B
from oracle import moe_oracle as O

from _parity import ROW_TOL, check_routing, host, row_rel_err, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()


W = workloads.WORKLOADS
CASES = {
    # name: (spec, aux_coef)
    "noisy_scaled_bias_aux": (workloads.MoESpec("noisy_scaled_bias_aux", T=1500, d=256, h=512, N=8, k=2,
                                                capacity_factor=1.0, gate="noisy", renorm=True, dtype="bf16",
                                                expert_bias=True, zipf_s=0.8), (0.01, 0.5)),
    "large_scaled_drops": (workloads.scaled(W["large_expert_top2_bf16"], T=700, d=512, h=1024).with_(
        capacity_factor=0.9), (0.0, 0.0)),
    "decode_scaled": (workloads.scaled(W["decode_top8_bf16"], T=64, d=512, h=256), (0.0, 0.0)),
    "ragged_tails": (workloads.MoESpec("ragged_tails", T=333, d=200, h=136, N=5, k=3, capacity_factor=0.8,
                                       gate="softmax", renorm=False, dtype="bf16", expert_bias=True),
                     (0.2, 0.0)),
    # large enough for the 256 x 256 tiles, with d and h not multiples of
    # the tile: partial row, column and contraction tiles on that path
    "ragged_big_tiles": (workloads.MoESpec("ragged_big_tiles", T=4096, d=1000, h=1960, N=8, k=2,
                                           capacity_factor=1.0, gate="noisy", renorm=True, dtype="bf16",
                                           expert_bias=True, zipf_s=0.5), (0.01, 0.1)),
    "noisy_top2_bf16": (W["noisy_top2_bf16"], (0.0, 0.0)),
    "large_expert_top2_bf16": (W["large_expert_top2_bf16"], (0.0, 0.0)),
    "decode_top8_bf16": (W["decode_top8_bf16"], (0.0, 0.0)),
}


def _forward_and_backward(spec, seed, aux):
    inp = make_inputs(spec, seed)
    dev = api.DeviceLayer(inp)
    say(f"[case] backward {spec.name} T={spec.T} d={spec.d} h={spec.h} N={spec.N} k={spec.k} aux={aux}")
    dev.run_forward(inspect=True)
    dy_h = make_output_grad(spec, seed)
    dy = torch.from_numpy(dy_h).cuda().to(torch.bfloat16)
    dev.backward_buffers()
    dev.run_backward(dy, aux)
    torch.cuda.synchronize()
    return inp, dev, dy_h, dy


def _rows(a):
    a = np.asarray(a)
    return a.reshape(-1, a.shape[-1]) if a.ndim > 1 else a.reshape(1, -1)


@pytest.mark.parametrize("name", list(CASES))
def test_backward_matches_oracle(name):
    spec, aux = CASES[name]
    inp, dev, dy_h, dy = _forward_and_backward(spec, workloads.WORKLOAD_SEED.get(name, 17), aux)
    lg = host(dev.logits)
    r = check_routing(spec, inp, dev, lg)
    say("   oracle backward")
    ref = B.backward(spec, inp, r, dy_h, aux)
    tol = ROW_TOL["bf16"]
    errs = {}
    for key, got in dev.grads.items():
        if got is None:
            assert ref[key] is None
            continue
        errs[key] = row_rel_err(_rows(host(got)), _rows(ref[key]))
    say("   " + " ".join(f"{k} {v:.2e}" for k, v in errs.items()))
    for key, e in errs.items():
        assert e <= tol, f"{key}: row error {e:.3g} > {tol}"
    # the same bits on a second call
    first = {k: v.clone() for k, v in dev.grads.items() if v is not None}
    dev.run_backward(dy, aux)
    torch.cuda.synchronize()
    for k, v in first.items():
        assert torch.equal(dev.grads[k], v), f"{k} differs on a second call"


def test_backward_rejects_unsupported_layers():
    for spec in (W["cosine_zipf_top4_bf16"], W["tiny_top1_f32"]):
        desc = api.desc_from_spec(spec)
        with pytest.raises(RuntimeError, match="MOE_ERR_UNSUPPORTED"):
            api.backward(desc, {}, torch.empty(1, dtype=torch.uint8, device="cuda"))
