"""HIP path vs the CPU oracle on the GPU, through the C ABI.

Scaled workloads (same routing parameters as the five named workloads, at
shapes the oracle finishes in seconds, with several tiles and ragged tails)
check every stage; the full-size workloads run moe_forward in the same
launch configuration bench.py times, and the stage calls on the same
routing, and every row of y, H and y_perm is compared with the oracle's
whole fp64 layer (seconds on the host even for the large-expert layer)."""
import math

import numpy as np
import pytest
import torch

from mixture_experts_sparse_gate_amd import _lib, api, workloads
from mixture_experts_sparse_gate_amd.inputs import make_inputs
from oracle import moe_oracle as O

from _parity import (check_ffn, check_logits, check_output, check_routing, check_x_perm, host,
                     row_rel_err, say, ROW_TOL)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    _lib.load()


W = workloads.WORKLOADS
SCALED = {
    "tiny_top1_f32": W["tiny_top1_f32"],
    "noisy_top2_bf16": workloads.scaled(W["noisy_top2_bf16"], T=1500, d=256, h=512),
    "large_expert_top2_bf16": workloads.scaled(W["large_expert_top2_bf16"], T=700, d=512, h=1024),
    "cosine_zipf_top4_bf16": workloads.scaled(W["cosine_zipf_top4_bf16"], T=3000, d=256, h=128),
    "decode_top8_bf16": workloads.scaled(W["decode_top8_bf16"], T=64, d=512, h=256),
}


def run_staged(spec, seed):
    inp = make_inputs(spec, seed)
    dev = api.DeviceLayer(inp)
    say(f"[case] staged {spec.name} T={spec.T} d={spec.d} h={spec.h} N={spec.N} k={spec.k} seed={seed}")
    dev.run_stages()
    torch.cuda.synchronize()
    return inp, dev


def full_check(spec, inp, dev):
    lg = host(dev.logits)
    check_logits(spec, inp, lg)
    r = check_routing(spec, inp, dev, lg)
    check_x_perm(spec, inp, dev, r)
    H, Y, eh, ey = check_ffn(spec, inp, dev, r)
    ey_out = check_output(spec, inp, dev, r, Y)
    say(f"   ok: A={int(r['off'][-1])} C={r['capacity']} H err {eh:.2e} y_perm err {ey:.2e} y err {ey_out:.2e}")
    return r


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_scaled_workload_stages(name):
    spec = SCALED[name]
    inp, dev = run_staged(spec, workloads.WORKLOAD_SEED[name] + 100)
    full_check(spec, inp, dev)


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_forward_equals_stages(name):
    spec = SCALED[name]
    inp, dev = run_staged(spec, 7)
    y_st = dev.y.clone()
    idx_st = dev.topk_idx.clone()
    rows_st = dev.row_of.clone()
    dev.y.zero_()
    dev.topk_idx.fill_(-7)
    dev.row_of.fill_(-7)
    say(f"[case] forward {spec.name}")
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    assert torch.equal(dev.topk_idx, idx_st)
    assert torch.equal(dev.row_of, rows_st)
    assert torch.equal(dev.y, y_st)
    # without inspection outputs the result is the same
    dev.y.zero_()
    dev.run_forward(inspect=False)
    torch.cuda.synchronize()
    assert torch.equal(dev.y, y_st)


def assert_ffn_status_clear(dev, kind=_lib.MOE_WS_FORWARD, ws=None):
    """The single-launch FFN's status word: no GEMM2 tile's wait for H expired."""
    st = api.ffn_status(dev.desc, dev.ws if ws is None else ws, kind)
    torch.cuda.synchronize()
    assert int(st.item()) == 0, f"fused FFN status word {int(st.item())}"


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER)
def test_full_size_forward(name):
    """The workload at its own size: one moe_forward call as bench.py makes
    it, then the stage calls on the same routing; every row of y, H and
    y_perm against the oracle's fp64 layer on the GPU's fp32 logits."""
    spec = W[name]
    inp = make_inputs(spec, workloads.WORKLOAD_SEED[name])
    dev = api.DeviceLayer(inp)
    say(f"[case] full-size forward {name}")
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    assert_ffn_status_clear(dev)
    lg = host(dev.logits)
    ref_l = check_logits(spec, inp, lg)
    say("   oracle forward on the GPU's logits")
    ref = O.forward(spec, inp, logits_override=lg)
    r = check_routing(spec, inp, dev, lg)
    # routing from the oracle's own fp64 logits agrees except at near-ties
    _, idx_ref = O.top_k(ref_l, spec.k)
    differ = int((idx_ref != r["topk_idx"]).any(axis=1).sum())
    say(f"   tokens routed differently from fp64 logits: {differ} of {spec.T}")
    assert differ <= max(1, spec.T // 1000)
    A = int(r["off"][-1])
    e = row_rel_err(host(dev.y), ref["y"])
    say(f"   A={A}: all {spec.T} rows of y, error {e:.2e}")
    assert e <= ROW_TOL[spec.dtype]
    y_fwd = dev.y.clone()
    # the stage calls on the same routing: moe_dispatch must reproduce
    # forward's row maps exactly; then every row of x_perm (bitwise), H and
    # y_perm (the expert FFN as moe_expert_ffn runs it with a workspace: the
    # single persistent launch where the shapes allow it)
    row_of_fwd, tor_fwd = dev.row_of.clone(), dev.token_of_row.clone()
    api.dispatch(dev.desc, dev.x, dev.topk_idx, dev.expert_count, dev.expert_off, dev.row_of,
                 dev.token_of_row, dev.x_perm, ws=dev.ws)
    ffn_ws = api.workspace(dev.desc, _lib.MOE_WS_FFN)
    api.expert_ffn(dev.desc, dev.x_perm, dev.expert_off, dev.W1, dev.b1, dev.W2, dev.b2, dev.H, dev.y_perm,
                   ws=ffn_ws)
    api.combine(dev.desc, dev.y_perm, dev.row_of, dev.topk_w, dev.y)
    torch.cuda.synchronize()
    assert_ffn_status_clear(dev, _lib.MOE_WS_FFN, ffn_ws)
    assert torch.equal(dev.row_of, row_of_fwd) and torch.equal(dev.token_of_row[:A], tor_fwd[:A])
    check_x_perm(spec, inp, dev, r)
    eh = row_rel_err(host(dev.H[:A]), ref["H"])
    ey = row_rel_err(host(dev.y_perm[:A]), ref["y_perm"])
    say(f"   all {A} rows: H error {eh:.2e}, y_perm error {ey:.2e}")
    assert eh <= ROW_TOL[spec.dtype] and ey <= ROW_TOL[spec.dtype]
    # the stage calls give moe_forward's bits
    assert torch.equal(dev.y, y_fwd)
    # every token with all choices dropped has an exactly zero row
    dropped = np.nonzero((r["row_of"].reshape(spec.T, spec.k) < 0).all(axis=1))[0]
    if dropped.size:
        assert torch.count_nonzero(dev.y[torch.as_tensor(dropped, device=dev.y.device)]) == 0


# Shapes whose two expert GEMMs both take 256x256 tiles: there moe_forward
# runs the expert FFN as one persistent launch (GEMM2 tiles waiting on the
# GEMM1 tiles of their rows) while moe_expert_ffn makes two launches; the
# tiles and their arithmetic are the same, so the results must agree bit for
# bit, call after call (the launch consumes counters the dispatch clears).
FUSED = {
    "noisy_top2_bf16": W["noisy_top2_bf16"],
    "cosine_zipf_top4_bf16": W["cosine_zipf_top4_bf16"],
    "large_expert_top2_bf16": W["large_expert_top2_bf16"],
    # skewed demand over 16 experts: empty, small and capped groups, tails
    "zipf16_top2": workloads.MoESpec("zipf16_top2", T=8192, d=1024, h=1024, N=16, k=2, capacity_factor=2.0,
                                     gate="softmax", renorm=True, dtype="bf16", zipf_s=1.5),
    # the same skew with fewer GEMM2 tiles than CUs: empty groups, tails
    "skew16_few_tiles": workloads.MoESpec("skew16_few_tiles", T=3000, d=1024, h=2048, N=16, k=2,
                                          capacity_factor=2.0, gate="softmax", renorm=True, dtype="bf16",
                                          zipf_s=1.5),
    # skewed demand with contractions long enough for the ping-pong K loop
    # (96 K-steps in both GEMMs): empty and small groups, tail tiles
    "zipf16_pingpong": workloads.MoESpec("zipf16_pingpong", T=4096, d=3072, h=3072, N=16, k=2,
                                         capacity_factor=2.0, gate="softmax", renorm=True, dtype="bf16",
                                         zipf_s=1.5),
    # the ping-pong loop with remainder steps: GEMM1 runs 98 K-steps (3112 =
    # 97 x 32 + 8, a partial last step), GEMM2 100; partial column tiles
    "pingpong_ragged_k": workloads.MoESpec("pingpong_ragged_k", T=2048, d=3112, h=3200, N=8, k=2,
                                           capacity_factor=1.25, gate="noisy", renorm=True, dtype="bf16",
                                           expert_bias=True),
    # eight choices per token (the folded combine's widest batch), with drops
    "k8_drops": workloads.MoESpec("k8_drops", T=2048, d=1024, h=1024, N=16, k=8, capacity_factor=0.9,
                                  gate="softmax", renorm=True, dtype="bf16", zipf_s=0.7),
}

# H rows that are not a whole number of 256-byte lines (h * 2 = 2064 bytes):
# a line would hold the end of one row tile's last row and the start of the
# next, so these shapes take the two launches (no GEMM2 tile can then read a
# line of H before it is complete)
NOT_FUSED = {
    "zipf16_h1032": workloads.MoESpec("zipf16_h1032", T=8192, d=1024, h=1032, N=16, k=2, capacity_factor=2.0,
                                      gate="softmax", renorm=True, dtype="bf16", zipf_s=1.5),
}


@pytest.mark.parametrize("name", list(NOT_FUSED))
def test_partial_line_rows_take_two_launches(name):
    spec = NOT_FUSED[name]
    inp, dev = run_staged(spec, 11)
    assert int(api.workspace_size(dev.desc, _lib.MOE_WS_FFN)) == 0, "the shape takes the two launches"
    full_check(spec, inp, dev)
    y_st = dev.y.clone()
    dev.y.fill_(float("nan"))
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    assert torch.equal(dev.y, y_st)


@pytest.mark.parametrize("name", list(FUSED))
def test_fused_ffn_forward_equals_stages(name):
    spec = FUSED[name]
    inp, dev = run_staged(spec, 11)
    assert int(api.workspace_size(dev.desc, _lib.MOE_WS_FFN)) > 0, "the shape takes the single launch"
    assert_ffn_status_clear(dev, _lib.MOE_WS_FFN)
    y_st = dev.y.clone()
    counts = host(dev.expert_count)
    say(f"   expert demand: min {counts.min()} max {counts.max()} zero {(counts == 0).sum()}")
    # the single launch against the oracle, on every row
    full_check(spec, inp, dev)
    # the stage call ran the single launch (it had a workspace); the two
    # launches (no workspace) give the same H and y_perm bit for bit
    A = int(host(dev.expert_off)[-1])
    H1, Y1 = dev.H[:A].clone(), dev.y_perm[:A].clone()
    dev.H.zero_()
    dev.y_perm.zero_()
    say(f"[case] two-launch FFN {spec.name}")
    api.expert_ffn(dev.desc, dev.x_perm, dev.expert_off, dev.W1, dev.b1, dev.W2, dev.b2, dev.H, dev.y_perm)
    torch.cuda.synchronize()
    assert torch.equal(dev.H[:A], H1) and torch.equal(dev.y_perm[:A], Y1)
    # repeated single launches give the same bits every time: a stage buffer
    # refilled while a wave still reads it shows up as a stray row fragment in
    # some calls only (tiny groups at the end make the rows of such tail tiles)
    for rep in range(6):
        dev.H.zero_()
        dev.y_perm.zero_()
        api.expert_ffn(dev.desc, dev.x_perm, dev.expert_off, dev.W1, dev.b1, dev.W2, dev.b2, dev.H, dev.y_perm,
                       ws=dev.ws)
        torch.cuda.synchronize()
        assert_ffn_status_clear(dev, _lib.MOE_WS_FFN)
        assert torch.equal(dev.H[:A], H1) and torch.equal(dev.y_perm[:A], Y1), f"single launch, call {rep}"
    for rep in range(2):
        dev.y.fill_(float("nan"))
        say(f"[case] fused forward {spec.name} call {rep}")
        dev.run_forward(inspect=True)
        torch.cuda.synchronize()
        assert_ffn_status_clear(dev)
        assert torch.equal(dev.y, y_st)
    # the combine folded into the same launch (MOE_FLAG_COMBINE_IN_FFN): every
    # row of y is written by the launch itself (NaN before the call), bit for
    # bit the separate combine's, fully dropped tokens included
    fold = api.desc_from_spec(spec, _lib.MOE_FLAG_COMBINE_IN_FFN)
    fold_ws = api.workspace(fold, _lib.MOE_WS_FORWARD)
    assert fold_ws.numel() > dev.ws.numel(), "the flag adds the arrival counts"
    for rep in range(3):
        dev.y.fill_(float("nan"))
        say(f"[case] forward with the combine in the FFN launch {spec.name} call {rep}")
        api.forward(fold, dev.layer_tensors(inspect=True), fold_ws)
        torch.cuda.synchronize()
        st = api.ffn_status(fold, fold_ws)
        torch.cuda.synchronize()
        assert int(st.item()) == 0
        assert torch.equal(dev.y, y_st), f"folded combine, call {rep}"


EDGE = {
    # one expert: every weight is 1 and y = FFN_0(x)
    "single_expert": workloads.MoESpec("single_expert", T=300, d=64, h=128, N=1, k=1, capacity_factor=1.0,
                                       gate="softmax", renorm=False, dtype="bf16"),
    # k = N with unlimited capacity: the dense softmax mixture
    "k_equals_n": workloads.MoESpec("k_equals_n", T=257, d=128, h=64, N=6, k=6, capacity_factor=1.0,
                                    gate="noisy", renorm=False, dtype="f32"),
    "one_token": workloads.MoESpec("one_token", T=1, d=256, h=256, N=16, k=3, capacity_factor=1.0,
                                   gate="softmax", renorm=True, dtype="bf16"),
    "capacity_one": workloads.MoESpec("capacity_one", T=333, d=64, h=64, N=8, k=2, capacity_factor=0.01,
                                      gate="softmax", renorm=True, dtype="bf16"),
    "odd_expert_count": workloads.MoESpec("odd_expert_count", T=1029, d=96, h=160, N=5, k=2,
                                          capacity_factor=1.1, gate="noisy", renorm=True, dtype="bf16",
                                          expert_bias=True),
    "many_experts_f32": workloads.MoESpec("many_experts_f32", T=2100, d=64, h=96, N=256, k=8,
                                          capacity_factor=2.0, gate="softmax", renorm=False, dtype="f32",
                                          expert_bias=True),
    "cosine_small_p": workloads.MoESpec("cosine_small_p", T=1111, d=128, h=64, N=100, k=5,
                                        capacity_factor=0.9, gate="cosine", renorm=True, dtype="bf16",
                                        proj_dim=40, temperature=0.1, zipf_s=0.7),
    # k past 8: the combine's one-row-at-a-time path; k = 32, the largest the
    # library takes, also fills the load-balance kernel's staging arrays
    "k12_bf16": workloads.MoESpec("k12_bf16", T=300, d=64, h=96, N=40, k=12, capacity_factor=1.0,
                                  gate="softmax", renorm=False, dtype="bf16"),
    "k32_f32": workloads.MoESpec("k32_f32", T=290, d=32, h=64, N=33, k=32, capacity_factor=2.0,
                                 gate="noisy", renorm=True, dtype="f32", expert_bias=True),
    # N <= 64: the single-pass cosine kernel, with a partly filled expert tile,
    # renormalised weights, a small p and a ragged last block of tokens
    "cosine_n40_renorm": workloads.MoESpec("cosine_n40_renorm", T=777, d=96, h=64, N=40, k=3,
                                           capacity_factor=1.3, gate="cosine", renorm=True, dtype="bf16",
                                           proj_dim=24, temperature=0.2, zipf_s=0.5, expert_bias=True),
}


@pytest.mark.parametrize("case", sorted(EDGE))
def test_edge_shapes(case):
    spec = EDGE[case]
    inp, dev = run_staged(spec, 21)
    full_check(spec, inp, dev)


def test_all_tokens_to_one_expert():
    """Every token prefers expert 3: massive drops, all other experts empty
    unless second choices land there."""
    spec = workloads.MoESpec("hot_expert", T=2000, d=128, h=64, N=8, k=2, capacity_factor=1.0,
                             gate="softmax", renorm=True, dtype="bf16")
    inp = make_inputs(spec, 31)
    inp.logit_bias = np.zeros(spec.N, np.float32)
    inp.logit_bias[3] = 1000.0
    dev = api.DeviceLayer(inp)
    say("[case] hot expert")
    dev.run_stages()
    torch.cuda.synchronize()
    r = full_check(spec, inp, dev)
    assert r["kept"][3] == r["capacity"] and r["count"][3] == spec.T


def test_exact_ties_go_to_the_lower_index():
    """Zero x rows make every logit 0 (plain gate): experts 0..k-1 are chosen.
    Duplicate gate columns make exact ties between two experts on every token."""
    spec = workloads.MoESpec("ties", T=700, d=64, h=64, N=8, k=3, capacity_factor=2.0,
                             gate="softmax", renorm=False, dtype="bf16")
    inp = make_inputs(spec, 41)
    inp.x[::5] = 0.0
    inp.w_gate[:, 6] = inp.w_gate[:, 1]
    inp.x[1::5, :] *= -1.0  # -0.0 and +0.0 both appear in zero products
    dev = api.DeviceLayer(inp)
    say("[case] exact ties")
    dev.run_stages()
    torch.cuda.synchronize()
    r = full_check(spec, inp, dev)
    assert (r["topk_idx"][::5] == [0, 1, 2]).all()
    both = (r["topk_idx"] == 1).any(axis=1) & (r["topk_idx"] == 6).any(axis=1)
    pos1 = np.argmax(r["topk_idx"] == 1, axis=1)
    pos6 = np.argmax(r["topk_idx"] == 6, axis=1)
    assert np.all(pos1[both] < pos6[both])


def test_deterministic():
    spec = SCALED["cosine_zipf_top4_bf16"]
    inp = make_inputs(spec, 5)
    dev = api.DeviceLayer(inp)
    say("[case] determinism")
    outs = []
    for _ in range(3):
        dev.y.zero_()
        dev.run_forward(inspect=True)
        torch.cuda.synchronize()
        outs.append((dev.y.clone(), dev.topk_w.clone(), dev.row_of.clone()))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert torch.equal(a, b)


def test_dispatch_with_caller_routing():
    """moe_dispatch on a routing the caller supplies (not from moe_route)."""
    spec = workloads.MoESpec("caller_routing", T=4099, d=64, h=64, N=37, k=4, capacity_factor=0.7,
                             gate="softmax", renorm=False, dtype="bf16")
    inp = make_inputs(spec, 51, with_experts=False)
    rng = np.random.default_rng(0)
    # skewed: experts with small ids are much more popular
    p = 1.0 / np.arange(1, spec.N + 1)
    p /= p.sum()
    idx = np.stack([rng.choice(spec.N, size=spec.k, replace=False, p=p) for _ in range(spec.T)])
    desc = api.desc_from_spec(spec)
    R = api.rows_bound(desc)
    dv = dict(dtype=torch.int32, device="cuda")
    x = torch.from_numpy(inp.x).cuda().to(torch.bfloat16)
    t_idx = torch.from_numpy(idx.astype(np.int32)).cuda()
    count, off = torch.empty(spec.N, **dv), torch.empty(spec.N + 1, **dv)
    row_of, tor = torch.empty(spec.T * spec.k, **dv), torch.full((R,), -1, **dv)
    x_perm = torch.zeros(R, spec.d, dtype=torch.bfloat16, device="cuda")
    ws = api.workspace(desc, _lib.MOE_WS_DISPATCH)
    say("[case] caller routing")
    api.dispatch(desc, x, t_idx, count, off, row_of, tor, x_perm, ws=ws)
    torch.cuda.synchronize()
    C = O.capacity(spec.T, spec.k, spec.N, spec.capacity_factor)
    cnt, kept, o, ro, t_o_r = O.assign_slots(idx, spec.N, C)
    assert np.array_equal(host(count), cnt) and np.array_equal(host(off), o)
    assert np.array_equal(host(row_of), ro)
    A = int(o[-1])
    assert np.array_equal(host(tor)[:A], t_o_r)
    assert torch.equal(x_perm[:A].view(torch.int16), x[torch.from_numpy(t_o_r // spec.k).cuda()].view(torch.int16))


def expected_slots_with_invalid(idx, N, C):
    """Slots by the counting definition for a caller's routing in which an
    entry outside [0, N), or a repeat of an earlier expert of the same token,
    occupies no slot (moe_dispatch's documented treatment)."""
    T, k = idx.shape
    valid = np.zeros((T, k), bool)
    for t in range(T):
        seen = set()
        for j in range(k):
            e = int(idx[t, j])
            valid[t, j] = 0 <= e < N and e not in seen
            seen.add(e)
    fill = np.zeros(N, np.int64)
    slot = np.full((T, k), -1, np.int64)
    for t in range(T):
        for j in range(k):
            if valid[t, j]:
                e = int(idx[t, j])
                slot[t, j] = fill[e]
                fill[e] += 1
    kept = np.minimum(fill, C)
    off = np.concatenate([[0], np.cumsum(kept)])
    row_of = np.full(T * k, -1, np.int64)
    for t in range(T):
        for j in range(k):
            if valid[t, j] and slot[t, j] < C:
                row_of[t * k + j] = off[int(idx[t, j])] + slot[t, j]
    return fill, off, row_of


def _dispatch_caller(spec, idx, lib_path=_lib.LIB_PATH):
    desc = api.desc_from_spec(spec)
    R = api.rows_bound(desc)
    dv = dict(dtype=torch.int32, device="cuda")
    x = torch.randn(spec.T, spec.d, device="cuda").to(torch.bfloat16)
    count, off = torch.empty(spec.N, **dv), torch.empty(spec.N + 1, **dv)
    row_of, tor = torch.empty(spec.T * spec.k, **dv), torch.full((R,), -1, **dv)
    x_perm = torch.zeros(R, spec.d, dtype=torch.bfloat16, device="cuda")
    ws = api.workspace(desc, _lib.MOE_WS_DISPATCH)
    api.dispatch(desc, x, torch.from_numpy(idx.astype(np.int32)).cuda(), count, off, row_of, tor, x_perm, ws=ws,
                 lib_path=lib_path)
    torch.cuda.synchronize()
    return host(count), host(off), host(row_of), host(tor)


def test_dispatch_caller_routing_with_invalid_entries():
    """A caller's routing with out-of-range entries and repeated experts: the
    release build drops exactly those choices; the debug build rejects the
    call with a message naming the entry."""
    spec = workloads.MoESpec("caller_invalid", T=1500, d=64, h=64, N=12, k=4, capacity_factor=0.8,
                             gate="softmax", renorm=False, dtype="bf16")
    rng = np.random.default_rng(3)
    idx = np.stack([rng.choice(spec.N, size=spec.k, replace=False) for _ in range(spec.T)])
    idx[5, 2] = idx[5, 0]        # a repeat
    idx[17, 3] = spec.N          # out of range
    idx[40, 1] = -1
    idx[99, 1:] = idx[99, 0]     # three repeats
    idx[rng.choice(spec.T, 50, replace=False), 3] = idx[rng.choice(spec.T, 50, replace=False), 0]
    C = O.capacity(spec.T, spec.k, spec.N, spec.capacity_factor)
    say("[case] caller routing with invalid entries (release build)")
    count, off, row_of, tor = _dispatch_caller(spec, idx)
    want_count, want_off, want_row = expected_slots_with_invalid(idx, spec.N, C)
    assert np.array_equal(count, want_count) and np.array_equal(off, want_off)
    assert np.array_equal(row_of, want_row)
    A = int(want_off[-1])
    kept = np.nonzero(want_row >= 0)[0]
    assert np.array_equal(np.sort(tor[:A]), np.sort(kept)) and np.array_equal(tor[want_row[kept]], kept)
    say("[case] caller routing with a repeated expert (debug build)")
    with pytest.raises(RuntimeError, match="token 5 names expert"):
        _dispatch_caller(spec, idx, _lib.DEBUG_LIB_PATH)
    ok = np.stack([rng.choice(spec.N, size=spec.k, replace=False) for _ in range(spec.T)])
    c2, o2, r2, _ = _dispatch_caller(spec, ok, _lib.DEBUG_LIB_PATH)
    wc, wo, wr = expected_slots_with_invalid(ok, spec.N, C)
    assert np.array_equal(c2, wc) and np.array_equal(o2, wo) and np.array_equal(r2, wr)


def test_dispatch_scan_path_large_T():
    """Large count tables go through the scan kernel (one block per expert)
    instead of every rows block summing the table: caller routing over 70,000
    tokens (274 tiles x 64 experts), then moe_forward with the bf16 noisy gate
    on 262,144 tokens (8,192 groups of 32 tokens x 8 experts); both against
    the oracle's slots."""
    spec = workloads.MoESpec("scan_caller", T=70000, d=64, h=64, N=64, k=2, capacity_factor=1.1,
                             gate="softmax", renorm=False, dtype="bf16")
    rng = np.random.default_rng(9)
    p = 1.0 / np.arange(1, spec.N + 1) ** 0.8
    p /= p.sum()
    idx = np.stack([rng.choice(spec.N, size=spec.k, replace=False, p=p) for _ in range(spec.T)])
    C = O.capacity(spec.T, spec.k, spec.N, spec.capacity_factor)
    say("[case] dispatch scan path, caller routing T=70000 N=64")
    count, off, row_of, tor = _dispatch_caller(spec, idx)
    cnt, kept, o, ro, t_o_r = O.assign_slots(idx, spec.N, C)
    assert np.array_equal(count, cnt) and np.array_equal(off, o) and np.array_equal(row_of, ro)
    assert np.array_equal(tor[:int(o[-1])], t_o_r)
    spec2 = workloads.MoESpec("scan_gate", T=262144, d=64, h=64, N=8, k=2, capacity_factor=1.0,
                              gate="noisy", renorm=True, dtype="bf16")
    inp = make_inputs(spec2, 19)
    dev = api.DeviceLayer(inp)
    say("[case] dispatch scan path, moe_forward with the noisy gate's counts, T=262144")
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    lg = host(dev.logits)
    r = check_routing(spec2, inp, dev, lg)
    assert int(r["off"][-1]) < spec2.T * spec2.k  # drops


@pytest.mark.parametrize("name", ["noisy_top2_bf16", "decode_top8_bf16"])
def test_ffn_launch_events(name):
    """moe_time_ffn_launches: the FFN's launches (one persistent kernel for
    noisy top-2, two grouped GEMMs for decode) record the events around their
    execution, inside the span of the whole step, and change no result."""
    spec = W[name]
    inp = make_inputs(spec, workloads.WORKLOAD_SEED[name])
    dev = api.DeviceLayer(inp)
    dev.run_forward(inspect=False)
    torch.cuda.synchronize()
    y_ref = dev.y.clone()
    s = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(s)
    e1.record(s)
    torch.cuda.synchronize()
    say(f"[case] FFN launch events {name}")
    api.time_ffn_launches(e0._as_parameter_, e1._as_parameter_)
    try:
        dev.y.zero_()
        a.record(s)
        dev.run_forward(inspect=False)
        b.record(s)
        torch.cuda.synchronize()
    finally:
        api.time_ffn_launches(None, None)
    ffn_ms, step_ms = e0.elapsed_time(e1), a.elapsed_time(b)
    say(f"   FFN {ffn_ms * 1e3:.1f} us of a {step_ms * 1e3:.1f} us step")
    assert 0 < ffn_ms < step_ms
    assert torch.equal(dev.y, y_ref)


@pytest.mark.parametrize("name", ["noisy_top2_bf16", "zipf16_pingpong"])
def test_ffn_trace_build(name):
    """The trace build (libmoe_gfx950_trace.so) gives the release build's y
    bit for bit and records every item of the single launch once: as many
    GEMM1 and GEMM2 items as full and tail row tiles times column tiles, each
    ending after it starts, on XCDs 0-7."""
    spec = W[name] if name in W else FUSED[name]
    inp = make_inputs(spec, workloads.WORKLOAD_SEED.get(name, 11))
    dev = api.DeviceLayer(inp)
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    y_ref = dev.y.clone()
    lib = _lib.load(_lib.TRACE_LIB_PATH)
    nbytes = int(lib.moe_ffn_trace_bytes())
    assert nbytes > 0 and int(_lib.load().moe_ffn_trace_bytes()) == 0
    say(f"[case] FFN trace build {name}")
    for _ in range(2):
        dev.y.fill_(float("nan"))
        api.forward(dev.desc, dev.layer_tensors(inspect=True), dev.ws, lib_path=_lib.TRACE_LIB_PATH)
        torch.cuda.synchronize()
        assert torch.equal(dev.y, y_ref)
    buf = np.zeros(nbytes // 8, dtype=np.uint64)
    assert lib.moe_ffn_trace_read(buf.ctypes.data) == _lib.MOE_OK
    rec = buf.reshape(-1, 8).astype(np.int64)
    rec = rec[rec[:, 2] != 0]
    rec = rec[(rec[:, 5] >> 32) == (rec[:, 5] >> 32).max()]
    kept = np.diff(host(dev.expert_off))
    rem = kept % 256
    small = (rem > 0) & (rem <= 128)
    row_tiles = int((kept // 256 + ((rem > 0) & ~small)).sum() + np.where(small, (rem + 63) // 64, 0).sum())
    nt1, nt2 = (spec.h + 255) // 256, (spec.d + 255) // 256
    kind = (rec[:, 5] >> 4) & 15
    assert (kind == 1).sum() == row_tiles * nt1 and (kind == 2).sum() == row_tiles * nt2
    assert ((rec[:, 5] & 15) < 8).all() and (rec[:, 2] >= rec[:, 1]).all() and (rec[:, 1] >= rec[:, 0]).all()
    assert (rec[:, 4] > rec[:, 3]).all()


def _aux(dev, spec, importance=True, losses=True):
    imp = torch.full((spec.N,), -1.0, dtype=torch.float32, device="cuda") if importance else None
    los = torch.full((2,), -1.0, dtype=torch.float32, device="cuda") if losses else None
    api.aux_loss(dev.desc, dev.topk_idx, dev.topk_w, imp, los, api.workspace(dev.desc, _lib.MOE_WS_AUX))
    torch.cuda.synchronize()
    return imp, los


@pytest.mark.parametrize("name", workloads.WORKLOAD_ORDER + ["single_expert", "k32_f32"])
def test_aux_loss_matches_oracle(name):
    """moe_aux_loss on the GPU's own routing: the importance against the
    oracle's column sums of the sparse gate matrix, the losses against the
    oracle's formulas on that importance; the same bits on a second call, and
    either output alone."""
    spec = W[name] if name in W else EDGE[name]
    inp = make_inputs(spec, workloads.WORKLOAD_SEED.get(name, 5))
    dev = api.DeviceLayer(inp)
    dev.run_forward(inspect=True)
    torch.cuda.synchronize()
    say(f"[case] aux loss {name}")
    imp, los = _aux(dev, spec)
    ref = O.expert_importance(spec.N, host(dev.topk_idx), host(dev.topk_w).astype(np.float64))
    got = host(imp).astype(np.float64)
    np.testing.assert_allclose(got, ref, rtol=2e-5, atol=1e-6)
    l0, l1 = (float(v) for v in host(los))
    say(f"   importance {got.min():.4g}..{got.max():.4g}, losses {l0:.6g} {l1:.6g}")
    assert math.isclose(l0, O.load_balance_loss(got), rel_tol=1e-4, abs_tol=1e-6 * max(1.0, ref.max()) ** 2)
    if spec.N == 1:
        assert l0 == 0.0 and math.isnan(l1)
    else:
        assert math.isclose(l1, O.importance_loss(got), rel_tol=1e-4, abs_tol=1e-7 * max(1.0, ref.max()))
    imp2, los2 = _aux(dev, spec)
    assert torch.equal(imp2, imp) and torch.equal(los2[:1], los[:1])
    only_imp, none_l = _aux(dev, spec, losses=False)
    none_i, only_l = _aux(dev, spec, importance=False)
    assert torch.equal(only_imp, imp) and torch.equal(only_l[:1], los[:1])
