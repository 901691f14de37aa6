"""moe_forward_noalloc (the layer on the library's fixed scratch array)
against moe_forward with a caller's workspace: the same bits, on two calls
in a row, the second with a smaller layer than the first (the scratch keeps
the first call's contents)."""
import pytest
import torch

from mixture_experts_sparse_gate_amd import _lib, api, workloads
from mixture_experts_sparse_gate_amd.inputs import make_inputs

from _parity import say

pytestmark = pytest.mark.gpu

OUTPUTS = ("y", "logits", "topk_idx", "topk_w", "expert_count", "expert_off", "row_of")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()


def _both(spec, seed):
    dev = api.DeviceLayer(make_inputs(spec, seed))
    say(f"[case] no-alloc forward {spec.name} T={spec.T} d={spec.d} h={spec.h} N={spec.N} k={spec.k}")
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    ref = {n: getattr(dev, n).clone() for n in OUTPUTS}
    ref["token_of_row"] = dev.token_of_row[:int(dev.expert_off[-1].item())].clone()
    for n in OUTPUTS:
        getattr(dev, n).fill_(-5)
    dev.token_of_row.fill_(-5)
    api.forward_noalloc(dev.desc, dev.layer_tensors(inspect=True))
    torch.cuda.synchronize()
    for n in OUTPUTS:
        assert torch.equal(getattr(dev, n), ref[n]), f"{spec.name}: {n} differs from moe_forward"
    A = ref["token_of_row"].numel()
    assert torch.equal(dev.token_of_row[:A], ref["token_of_row"])
    # without inspection outputs (routing kept in the scratch array only)
    dev.y.fill_(-5)
    api.forward_noalloc(dev.desc, dev.layer_tensors(inspect=False))
    torch.cuda.synchronize()
    assert torch.equal(dev.y, ref["y"])


def test_noalloc_matches_forward_two_calls_second_smaller():
    # the noisy top-2 layer at full size (49 MiB of scratch, the single-launch
    # FFN), then a smaller decode-shaped layer on the same scratch
    big = workloads.get("noisy_top2_bf16")
    small = workloads.scaled(workloads.get("decode_top8_bf16"), T=64, d=512, h=256)
    assert api.workspace_size(api.desc_from_spec(small)) < api.workspace_size(api.desc_from_spec(big))
    _both(big, 3)
    _both(small, 4)


def test_noalloc_rejects_a_layer_above_the_scratch_size():
    spec = workloads.get("large_expert_top2_bf16")
    desc = api.desc_from_spec(spec)
    assert api.workspace_size(desc) > _lib.load().moe_noalloc_scratch_bytes()
    with pytest.raises(RuntimeError, match="MOE_ERR_UNSUPPORTED.*scratch array"):
        api.forward_noalloc(desc, {})
