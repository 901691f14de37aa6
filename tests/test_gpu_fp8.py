"""Block-FP8 expert weights on the GPU, through the C ABI.

moe_quantize_fp8 must give the oracle's codes and scales bit for bit (both
take each decision in fp32). The FFN and the whole layer on FP8 weights are
compared with the oracle's FFN on the oracle's own dequantised weights
(decode(code) * scale, exact in float64), to the bf16 row tolerance.
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from mixture_experts_sparse_gate_amd import api, workloads
from mixture_experts_sparse_gate_amd.inputs import make_inputs
from oracle import fp8_oracle as F
from oracle import moe_oracle as O

from _parity import ROW_TOL, check_logits, check_routing, host, row_rel_err, say

pytestmark = pytest.mark.gpu


def logical_codes(codes: torch.Tensor) -> np.ndarray:
    """[G, K/8, Ncols, 8] as stored -> [G, K, Ncols]."""
    G, K8, N, _ = codes.shape
    return host(codes.permute(0, 1, 3, 2).reshape(G, K8 * 8, N))


def check_quantised(W: np.ndarray, codes: torch.Tensor, scales: torch.Tensor, experts):
    for e in experts:
        c_ref, s_ref = F.quantize_blocks(W[e:e + 1])
        c = logical_codes(codes[e:e + 1])
        s = host(scales[e:e + 1])
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32)), f"scales of group {e}"
        bad = np.count_nonzero(c != c_ref)
        assert bad == 0, f"group {e}: {bad} codes differ"


def test_quantize_edge_values():
    """Exact ties, subnormal codes, signed zeros, an all-zero block, fp32 and bf16 input."""
    rng = np.random.default_rng(2)
    W = rng.standard_normal((2, 256, 384)).astype(np.float32)
    blk = W[0, 0:128, 0:128]
    blk[0, 0] = 448.0  # scale exactly 1: the other entries are quantised as given
    grid = F.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((grid[:-1] + grid[1:]) / 2).astype(np.float32)  # every tie, both signs
    blk.reshape(-1)[1:1 + mids.size] = mids
    blk.reshape(-1)[200:200 + mids.size] = -mids
    blk[5, :] = np.float32(2.0 ** -12)  # below half the smallest subnormal: signed zeros
    blk[6, :] = -np.float32(2.0 ** -12)
    blk[7, 3] = -0.0
    W[1, 128:256, 128:256] = 0.0  # an all-zero block
    W[1, 0:128, 256:384] = 0.0  # a block of fp32 subnormals: a subnormal scale, saturated codes
    W[1, 0, 256:384] = (np.linspace(1, 667, 128).round() * 2.0 ** -149).astype(np.float32)
    for dtype in (torch.float32, torch.bfloat16):  # (in bf16 those subnormals are zeros: a zero block)
        Wd = torch.from_numpy(W).cuda().to(dtype).contiguous()
        Wh = Wd.float().cpu().numpy()
        say(f"[case] quantise edge values {dtype}")
        codes, scales = api.quantize_fp8(Wd)
        torch.cuda.synchronize()
        check_quantised(Wh, codes, scales, range(2))
        assert host(scales)[1, 1, 1] == 0 and not logical_codes(codes)[1, 128:256, 128:256].any()


def test_quantize_decode_weights_sampled():
    spec = workloads.get("decode_top8_bf16")
    inp = make_inputs(spec, workloads.WORKLOAD_SEED[spec.name])
    dev = api.DeviceLayer(inp)
    say("[case] quantise decode_top8_bf16 W1, W2")
    w8 = dev.quantize_weights_fp8()
    torch.cuda.synchronize()
    assert w8["W1q"].shape == (spec.N, spec.d // 8, spec.h, 8) and w8["S2"].shape == (spec.N, spec.h // 128, spec.d // 128)
    experts = [0, 57, spec.N - 1]
    check_quantised(inp.W1, w8["W1q"], w8["S1"], experts)
    check_quantised(inp.W2, w8["W2q"], w8["S2"], experts)


class Dequantised:
    """W[e] -> the oracle's block-FP8 quantise-then-dequantise of expert e (float64)."""

    def __init__(self, W):
        self.W = W
        self.cache = {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.cache:
            c, s = F.quantize_blocks(self.W[e:e + 1])
            self.cache[e] = F.dequantize_blocks(c, s)[0]
        return self.cache[e]


SCALED = {
    "decode_scaled": workloads.scaled(workloads.get("decode_top8_bf16"), T=64, d=512, h=256),
    # more rows per expert than a tile, ragged groups, drops (128 x 128 tiles; d = 384: GEMM2's last
    # column tile has waves wholly past Ncols)
    "rows_ragged": workloads.MoESpec("rows_ragged", T=700, d=384, h=256, N=6, k=2, capacity_factor=1.1,
                                     gate="softmax", renorm=True, dtype="bf16"),
    # the noisy gate scaled down: tail tiles, 2 and 4 scale blocks along K
    "noisy_scaled": workloads.scaled(workloads.get("noisy_top2_bf16"), T=1500, d=256, h=512),
}


@pytest.mark.parametrize("name", list(SCALED))
def test_expert_ffn_fp8_matches_oracle(name):
    spec = SCALED[name]
    inp = make_inputs(spec, 21)
    dev = api.DeviceLayer(inp)
    say(f"[case] fp8 FFN {name} T={spec.T} d={spec.d} h={spec.h} N={spec.N} k={spec.k}")
    dev.run_stages()
    dev.quantize_weights_fp8()
    dev.H.zero_()
    dev.y_perm.zero_()
    api.expert_ffn_fp8(dev.desc, dev.x_perm, dev.expert_off, dev.w8["W1q"], dev.w8["S1"], dev.b1,
                       dev.w8["W2q"], dev.w8["S2"], dev.b2, dev.H, dev.y_perm)
    torch.cuda.synchronize()
    off = host(dev.expert_off).astype(np.int64)
    A = int(off[-1])
    tor = host(dev.token_of_row)[:A]
    x_perm = O.f64(inp.x)[tor // spec.k]
    W1d = np.stack([Dequantised(inp.W1)[e] for e in range(spec.N)])
    W2d = np.stack([Dequantised(inp.W2)[e] for e in range(spec.N)])
    H, Y = O.grouped_experts(x_perm, off, W1d, W2d, inp.b1, inp.b2)
    eh = row_rel_err(host(dev.H)[:A], H)
    ey = row_rel_err(host(dev.y_perm)[:A], Y)
    say(f"   A={A} H err {eh:.2e} y_perm err {ey:.2e}")
    assert eh <= ROW_TOL["bf16"] and ey <= ROW_TOL["bf16"]
    # rows past A are not written
    assert not dev.H[A:].any() and not dev.y_perm[A:].any()


@pytest.mark.parametrize("name", ["decode_top8_bf16", "noisy_top2_bf16"])
def test_forward_fp8_full_size(name):
    """The workload at its own size through moe_forward_fp8, as bench.py --weights fp8 runs it
    (decode: 32-row tiles; noisy: 128 x 128 tiles)."""
    spec = workloads.get(name)
    inp = make_inputs(spec, workloads.WORKLOAD_SEED[spec.name])
    dev = api.DeviceLayer(inp)
    dev.quantize_weights_fp8()
    say(f"[case] full-size fp8 forward {name}")
    dev.run_forward_fp8(inspect=True)
    torch.cuda.synchronize()
    lg = host(dev.logits)
    check_logits(spec, inp, lg)
    r = check_routing(spec, inp, dev, lg)
    # every token: each touched expert's weights quantised and dequantised by
    # the oracle (threads over experts, one expert's float64 weights at a
    # time), its rows through the oracle's FFN, then the oracle's combine
    off = r["off"]
    A = int(off[-1])
    x_perm = O.f64(inp.x)[r["token_of_row"] // spec.k]
    Y = np.zeros((A, spec.d), np.float64)

    def expert(e):
        lo, hi = int(off[e]), int(off[e + 1])
        if hi > lo:
            W1e, W2e = Dequantised(inp.W1)[e], Dequantised(inp.W2)[e]
            _, Y[lo:hi] = O.expert_ffn(x_perm[lo:hi], W1e, W2e, None if inp.b1 is None else inp.b1[e],
                                       None if inp.b2 is None else inp.b2[e])

    with ThreadPoolExecutor(16) as ex:
        list(ex.map(expert, range(spec.N)))
    y_ref = O.combine(Y, r["row_of"], r["topk_w"], spec.T, spec.k)
    e = row_rel_err(host(dev.y), y_ref)
    say(f"   all {spec.T} tokens, y err {e:.2e}")
    assert e <= ROW_TOL["bf16"]
    # the same layer with bf16 weights differs by the quantisation only
    y8 = dev.y.clone()
    dev.run_forward(inspect=False)
    torch.cuda.synchronize()
    d = row_rel_err(host(y8), host(dev.y))
    say(f"   fp8 against bf16 weights: row difference {d:.2e}")
    assert d <= 0.1


def test_forward_fp8_repeats_bit_for_bit():
    spec = SCALED["decode_scaled"]
    inp = make_inputs(spec, 4)
    dev = api.DeviceLayer(inp)
    dev.quantize_weights_fp8()
    outs = []
    for rep in range(3):
        dev.y.zero_()
        dev.run_forward_fp8(inspect=False)
        torch.cuda.synchronize()
        outs.append(dev.y.clone())
    assert all(torch.equal(outs[0], o) for o in outs[1:])
