"""moe_forward captured in a HIP graph: every replay, with the program's own
eager work and synchronisations between replays, gives what the eager call
gives (bitwise), and the eager result itself passes the oracle checks."""
import pytest
import torch

from mixture_experts_sparse_gate_amd import _lib, api, workloads
from mixture_experts_sparse_gate_amd.inputs import make_inputs

from _parity import say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()


W = workloads.WORKLOADS
CASES = {
    "noisy_top2_bf16": workloads.scaled(W["noisy_top2_bf16"], T=1500, d=256, h=512),
    "cosine_zipf_top4_bf16": workloads.scaled(W["cosine_zipf_top4_bf16"], T=3000, d=256, h=128),
    "decode_top8_bf16": workloads.scaled(W["decode_top8_bf16"], T=64, d=512, h=256),
    "tiny_top1_f32": W["tiny_top1_f32"],
    # full size: the expert FFN is the single persistent launch, whose work
    # counters the captured dispatch clears on every replay
    "noisy_top2_bf16_full": W["noisy_top2_bf16"],
    # the same with the combine folded into that launch: its arrival counts
    # are cleared by the captured dispatch too
    "noisy_top2_bf16_full_combine_in_ffn": W["noisy_top2_bf16"],
}
FLAGS = {"noisy_top2_bf16_full_combine_in_ffn": _lib.MOE_FLAG_COMBINE_IN_FFN}
OUTPUTS = ("y", "topk_idx", "topk_w", "row_of", "expert_off")


@pytest.mark.parametrize("name", sorted(CASES))
def test_graph_replays_match_eager(name):
    spec = CASES[name]
    dev = api.DeviceLayer(make_inputs(spec, 11), flags=FLAGS.get(name, 0))
    say(f"[case] graph {spec.name} T={spec.T} d={spec.d} h={spec.h} N={spec.N} k={spec.k}")
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    eager = {n: getattr(dev, n).clone() for n in OUTPUTS}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.run_forward(inspect=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dev.run_forward(inspect=True)

    for rep in range(4):
        for n in OUTPUTS:
            getattr(dev, n).fill_(-3)  # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in OUTPUTS:
            assert torch.equal(getattr(dev, n), eager[n]), f"replay {rep}: {n} differs from the eager call"
        dev.run_forward(inspect=True)  # an eager call between replays
        torch.cuda.synchronize()
        for n in OUTPUTS:
            assert torch.equal(getattr(dev, n), eager[n]), f"eager call after replay {rep}: {n} differs"


FP8_CASES = {
    "decode_top8_bf16": CASES["decode_top8_bf16"],           # 32-row tiles
    "noisy_top2_bf16": CASES["noisy_top2_bf16"],             # 128 x 128 tiles
}


@pytest.mark.parametrize("name", sorted(FP8_CASES))
def test_fp8_graph_replays_match_eager(name):
    """moe_forward_fp8 under a HIP graph: the same replay discipline."""
    spec = FP8_CASES[name]
    dev = api.DeviceLayer(make_inputs(spec, 12))
    dev.quantize_weights_fp8()
    say(f"[case] fp8 graph {spec.name} T={spec.T} d={spec.d} h={spec.h} N={spec.N} k={spec.k}")
    dev.run_forward_fp8(inspect=True)
    torch.cuda.synchronize()
    eager = {n: getattr(dev, n).clone() for n in OUTPUTS}

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dev.run_forward_fp8(inspect=True)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dev.run_forward_fp8(inspect=True)

    for rep in range(4):
        for n in OUTPUTS:
            getattr(dev, n).fill_(-3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n in OUTPUTS:
            assert torch.equal(getattr(dev, n), eager[n]), f"replay {rep}: {n} differs from the eager call"
        dev.run_forward_fp8(inspect=True)
        torch.cuda.synchronize()
        for n in OUTPUTS:
            assert torch.equal(getattr(dev, n), eager[n]), f"eager call after replay {rep}: {n} differs"
