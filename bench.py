"""Throughput of the sparse-gated MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole layer (gate, dispatch, expert FFN,
combine) over one batch of seeded synthetic tokens, through the single
moe_forward entry point, with every input already resident in HBM. W warmup
steps, then exactly K timed steps bracketed by torch.cuda.synchronize(); the
headline value is T tokens over the mean step time. The default workload is
the largest of the five that fits one GPU: the large-expert top-2 layer
(T = 8192, d = 4096, h = 14336, N = 8 experts), whose expert GEMMs are
compute bound; --workload names any of the others.

Besides the headline:
  - stages: the same layer through the four stage entry points, with HIP
    events recorded on the launch stream between them; their averages give
    each stage's duration; aux_loss: moe_aux_loss (per-expert importance and
    the two load-balance losses) on the step's routing, timed the same way;
  - graph_ms_per_step: moe_forward captured once in a HIP graph and replayed
    (no host launch cost per kernel); graph4_ms_per_step: four calls per
    captured graph (each replay boundary costs a fixed ~8 us of device idle
    time, which four calls share);
  - cold: each step timed alone by events after writing a 512 MiB buffer
    (twice the last-level cache), median / p10 / p90;
  - measured_peaks: the chip's own ceilings in the same run, a 1 GiB device
    copy with 16-byte loads and stores (HBM, read + write bytes) and a loop
    of bf16 MFMAs on registers over every CU (moe_probe_copy, moe_probe_mfma).
    The MFMA loop multiplies hashed operands that change from one MFMA to the
    next, as a GEMM's do; it is timed in short launches (burst) and over
    about 2 s of back-to-back launches (sustained: the rate once the board's
    power management has settled its clock). The roofline object gives the
    FFN's fraction of the sustained MFMA rate (or of the copy's bandwidth)
    beside its fraction of the published peak.
The roofline object describes the expert FFN kernel of moe_forward (the
single persistent launch of GEMM1+GELU and GEMM2 where the shapes allow it,
else the two grouped-GEMM launches), against the bf16 MFMA peak, or against
HBM bandwidth when few rows per expert make it weight-streaming bound. Its
duration comes from HIP events that the FFN's own launches record when its
kernels start and end executing (moe_time_ffn_launches), averaged over
moe_forward steps like the timed ones.

Prints one JSON line. The CPU oracle is timed afterwards on the host cores
on a bounded sample of the same workload (kind "oracle").

The measured HBM traffic of the expert FFN comes from two rocprofv3 --pmc
runs of this script (FETCH_SIZE, then WRITE_SIZE, with --calib-copy-mib so
that a device copy of known size calibrates both counters), condensed by

    python bench.py --summarize <results.db> --kind traffic --workload W --out profiles/...

into profiles/expert_ffn_<workload>_traffic.txt. That figure is used only
while the file's hash of the GEMM source matches the current source.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sqlite3
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}  # dense MFMA, MI355X published figures


GEMM_SRCS = [os.path.join(ROOT, "mixture_experts_sparse_gate_amd", "csrc", f) for f in ("gemm.hip", "gelu.hpp")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    """Hash of the expert FFN kernel's sources (the tile code and its GELU)."""
    h = hashlib.sha256()
    for path in GEMM_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_path(workload: str) -> str:
    return os.path.join(ROOT, "profiles", f"expert_ffn_{workload}_traffic.txt")


def read_traffic(workload: str):
    """HBM bytes per FFN step from the committed PMC summary, if it was taken
    on the current GEMM source."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None, "no summary"
    fields = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"^(\w+):\s*(\S+)", line)
            if m:
                fields[m.group(1)] = m.group(2)
    if fields.get("gemm_source_sha256_16") != gemm_source_hash():
        return None, "GEMM source changed since the counters were taken"
    return float(fields["ffn_hbm_bytes_per_step"]), path


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="large_expert_top2_bf16")
    ap.add_argument("--weights", choices=["layer", "fp8"], default="layer",
                    help="expert weights in the layer's dtype, or block-FP8 (moe_forward_fp8; bf16 layers)")
    ap.add_argument("--combine-in-ffn", action="store_true",
                    help="moe_forward with the gate-weighted combine folded into the single-launch expert FFN "
                         "(MOE_FLAG_COMBINE_IN_FFN; applies where that launch runs)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--skip-extras", action="store_true",
                    help="time only the warm steps (no graph replay, no cold-cache steps): counter runs")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    ap.add_argument("--graph-ab", action="store_true",
                    help="only interleave 3 rounds of 20 eager moe_forward steps and 20 graph replays "
                         "(for a kernel trace; --summarize --kind gaps condenses it)")
    ap.add_argument("--dispatch-scaling", action="store_true",
                    help="only time moe_dispatch on caller routing at T = 16k .. 256k tokens (N = 64, k = 2) "
                         "and moe_forward's dispatch at the same T (noisy gate, N = 8)")
    ap.add_argument("--ffn-trace", action="store_true",
                    help="only run --warmup then --steps moe_forward calls back to back on the trace build "
                         "(libmoe_gfx950_trace.so) and summarise the single-launch FFN's per-item trace of "
                         "the last call (per-XCD work and end times, tile times, shader clock)")
    ap.add_argument("--summarize", default=None, help="rocprofv3 results.db to condense (no GPU)")
    ap.add_argument("--kind", choices=["stats", "traffic", "pmc", "gaps", "dispatch"], default="stats")
    ap.add_argument("--pmc-dbs", nargs="*", default=[], help="with --kind pmc: results.db files of counter passes")
    ap.add_argument("--fetch-db", default=None, help="with --kind traffic: the FETCH_SIZE results.db")
    ap.add_argument("--write-db", default=None, help="with --kind traffic: the WRITE_SIZE results.db")
    ap.add_argument("--command", default="", help="command line recorded in the summary")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    if args.summarize or args.kind == "traffic" and args.fetch_db or args.kind == "pmc" and args.pmc_dbs:
        return summarize(args)

    if args.dispatch_scaling:
        return dispatch_scaling()

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}): the library has no "
              f"multi-GPU path; across GPUs the layer would shard by experts, each GPU running this "
              f"path on its experts' share after an all-to-all of the dispatched rows", file=sys.stderr)
        return 2

    import torch

    from mixture_experts_sparse_gate_amd import _lib, api, workloads
    from mixture_experts_sparse_gate_amd.inputs import make_inputs

    spec = workloads.get(args.workload)
    seed = workloads.WORKLOAD_SEED[args.workload]
    torch.cuda.set_device(0)
    t_gen = time.perf_counter()
    inp = make_inputs(spec, seed)
    dev = api.DeviceLayer(inp, flags=_lib.MOE_FLAG_COMBINE_IN_FFN if args.combine_in_ffn else 0)
    fp8 = args.weights == "fp8"
    # the flag takes effect where the single-launch FFN runs (its arrival
    # counts then enlarge the workspace)
    folded = (args.combine_in_ffn and not fp8 and
              api.workspace_size(dev.desc) > api.workspace_size(api.desc_from_spec(spec)))
    if fp8:
        if spec.dtype != "bf16":
            print("--weights fp8 needs a bf16 workload", file=sys.stderr)
            return 2
        dev.quantize_weights_fp8()  # model preparation, outside every timed region
    torch.cuda.synchronize()
    log(f"[bench] {spec.name}: inputs ready in {time.perf_counter() - t_gen:.1f}s")

    stream = torch.cuda.current_stream()
    if args.graph_ab:
        return graph_ab(dev, torch)
    if args.ffn_trace:
        return ffn_trace(args, dev, torch)
    if args.calib_copy_mib > 0:
        # a plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read
        # for it calibrates the counters (the only 1-byte-element copy here)
        src = torch.empty(args.calib_copy_mib << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def forward():
        if fp8:
            dev.run_forward_fp8(inspect=False)
        else:
            dev.run_forward(inspect=False)

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        api.route(dev.desc, **dev.gate_inputs(), logits=None, topk_idx=dev.topk_idx,
                  topk_w=dev.topk_w, ws=dev.ws)
        if ev:
            ev[1].record(stream)
        api.dispatch(dev.desc, dev.x, dev.topk_idx, dev.expert_count, dev.expert_off, dev.row_of,
                     dev.token_of_row, dev.x_perm, ws=dev.ws)
        if ev:
            ev[2].record(stream)
        if fp8:
            api.expert_ffn_fp8(dev.desc, dev.x_perm, dev.expert_off, dev.w8["W1q"], dev.w8["S1"], dev.b1,
                               dev.w8["W2q"], dev.w8["S2"], dev.b2, dev.H, dev.y_perm)
        else:
            api.expert_ffn(dev.desc, dev.x_perm, dev.expert_off, dev.W1, dev.b1, dev.W2, dev.b2, dev.H,
                           dev.y_perm, ws=dev.ws)
        if ev:
            ev[3].record(stream)
        api.combine(dev.desc, dev.y_perm, dev.row_of, dev.topk_w, dev.y)
        if ev:
            ev[4].record(stream)

    K = args.steps
    # The headline (K moe_forward steps after W warm-up steps) is timed last,
    # after the breakdowns below, so that the GPU has left its idle clocks
    # behind while the inputs were being generated on the host.

    # ---- stage breakdown through the four stage entry points
    for _ in range(3):
        step()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        step(events[i])
    torch.cuda.synchronize()
    staged_ms = (time.perf_counter() - t0) * 1e3 / K
    names = ["gate", "dispatch", "expert_ffn", "combine"]
    stage_ms = {n: float(np.mean([events[i][j].elapsed_time(events[i][j + 1]) for i in range(K)]))
                for j, n in enumerate(names)}

    # ---- moe_forward replayed from a HIP graph
    graph_ms = graph4_ms = None
    try:
        if args.skip_extras:
            raise RuntimeError("skipped (--skip-extras)")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            forward()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            forward()
        for _ in range(3):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(K):
            graph.replay()
        torch.cuda.synchronize()
        graph_ms = (time.perf_counter() - t0) * 1e3 / K
        del graph
        # four layer calls per graph: the replay boundary's fixed cost is paid
        # once per four steps
        graph4 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph4):
            for _ in range(4):
                forward()
        for _ in range(2):
            graph4.replay()
        torch.cuda.synchronize()
        reps4 = max(1, K // 4)
        t0 = time.perf_counter()
        for _ in range(reps4):
            graph4.replay()
        torch.cuda.synchronize()
        graph4_ms = (time.perf_counter() - t0) * 1e3 / (4 * reps4)
        del graph4
    except RuntimeError as e:  # capture unavailable: report the eager figures only
        log(f"[bench] graph capture skipped: {e}")

    # ---- cold caches: each step alone after a 512 MiB write
    flush = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
    cold = []
    for _ in range(0 if args.skip_extras else min(K, 20)):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        forward()
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    cold.sort()
    cold_ms = None
    if cold:
        cold_ms = {"median_ms": cold[len(cold) // 2], "p10_ms": cold[len(cold) // 10],
                   "p90_ms": cold[(9 * len(cold)) // 10], "reps": len(cold)}
        cold_ms["tokens_per_s"] = spec.T / (cold_ms["median_ms"] * 1e-3)

    # ---- the expert FFN's kernels alone: events that its launches record at
    # the start and end of execution, in moe_forward steps like the timed ones
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    ev1.record(stream)  # both exist from here on
    torch.cuda.synchronize()
    ffn_kernel_ms = []
    api.time_ffn_launches(ev0._as_parameter_, ev1._as_parameter_)
    try:
        for _ in range(max(K, 10)):
            forward()
            ev1.synchronize()
            ffn_kernel_ms.append(ev0.elapsed_time(ev1))
    finally:
        api.time_ffn_launches(None, None)
    ffn_kernel_ms = float(np.mean(ffn_kernel_ms))

    # ---- the backward pass (bf16 layers with the plain or noisy gate) on
    # the routing of a forward call with inspection outputs
    backward = None
    if not args.skip_extras and spec.dtype == "bf16" and spec.gate != "cosine" and not fp8:
        from mixture_experts_sparse_gate_amd.inputs import make_output_grad
        dy = torch.from_numpy(make_output_grad(spec, seed)).cuda().to(torch.bfloat16)
        dev.run_forward(inspect=True)
        dev.backward_buffers()
        for _ in range(2):
            dev.run_backward(dy)
        reps = max(3, min(K, 20))
        b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        b0.record(stream)
        for _ in range(reps):
            dev.run_backward(dy)
        b1.record(stream)
        torch.cuda.synchronize()
        bwd_ms = b0.elapsed_time(b1) / reps
        A_b = int(dev.expert_off[-1].item())
        # five grouped GEMMs of 2 A d h flops each: U (recomputed), dU,
        # dx rows, dW1, dW2
        bwd_flops = 10.0 * A_b * spec.d * spec.h
        backward = {"ms": bwd_ms, "tokens_per_s": spec.T / (bwd_ms * 1e-3), "flops": bwd_flops,
                    "TFLOP/s": bwd_flops / (bwd_ms * 1e-3) / 1e12,
                    "frac_of_bf16_peak": bwd_flops / (bwd_ms * 1e-3) / 1e12 / MFMA_PEAK_TFLOPS["bf16"],
                    "reps": reps}
        del dev.grads, dev.ws_bwd
        dev.grads = None

    # ---- the chip's measured ceilings, in this run
    peaks = None if args.skip_extras else measured_peaks(api, torch, stream)

    # ---- headline: W warm-up steps, then exactly K timed steps of moe_forward
    for _ in range(args.warmup):
        forward()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K):
        forward()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / K

    # algorithmic work of one step, from this step's routing
    off = dev.expert_off.cpu().numpy().astype(np.int64)
    kept = np.diff(off)
    A = int(off[-1])
    U = int((kept > 0).sum())
    s = 2 if spec.dtype == "bf16" else 4
    T, d, h, N, k = spec.T, spec.d, spec.h, spec.N, spec.k
    ffn_flops = 4.0 * A * d * h
    if fp8:  # one byte per weight plus one fp32 scale per 128 x 128 block, both matrices
        touched_weight_bytes = float(U) * 2 * (d * h + (d // 128) * (h // 128) * 4)
    else:
        touched_weight_bytes = float(U) * 2 * d * h * s
    ffn_s = ffn_kernel_ms * 1e-3
    avg_rows = (T * k) / N
    if avg_rows < 64:  # weight streaming: bound by HBM
        roof = {"bound": "hbm", "achieved": touched_weight_bytes / ffn_s / 1e9, "peak": HBM_PEAK_GBS,
                "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": ffn_flops / ffn_s / 1e12, "peak": MFMA_PEAK_TFLOPS[spec.dtype],
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    if fp8:
        roof["kernel"] = ("grouped_gemm_kernel with block-FP8 weights (32-row tiles streaming E4M3 codes), "
                          "launched twice per step (GEMM1+GELU, GEMM2); duration from the HIP events the "
                          "launches record (GEMM1's start to GEMM2's end), mean over moe_forward_fp8 steps")
    elif api.workspace_size(dev.desc, _lib.MOE_WS_FFN) > 0:
        roof["kernel"] = ("fused_ffn_kernel: GEMM1+GELU and GEMM2 in one persistent launch; duration from the "
                          "HIP events its launch records at the start and end of execution, mean over "
                          "moe_forward steps")
    else:
        roof["kernel"] = ("grouped_gemm_kernel, launched twice per step (GEMM1+GELU, GEMM2); duration from the "
                          "HIP events the launches record (GEMM1's start to GEMM2's end), mean over "
                          "moe_forward steps")
    roof["kernel_ms"] = ffn_kernel_ms
    if peaks:
        mp = peaks["hbm_copy_GB/s"] if roof["bound"] == "hbm" else peaks["mfma_bf16_sustained_TFLOP/s"]
        roof["measured_peak"] = mp
        roof["frac_of_measured_peak"] = roof["achieved"] / mp
    roof["algorithmic"] = {"flops": ffn_flops, "touched_weight_bytes": touched_weight_bytes}
    traffic, tsrc = read_traffic(spec.name + ("_fp8w" if fp8 else ""))
    roof["traffic"] = traffic
    roof["traffic_source"] = tsrc

    gate_bytes = T * d * s + (2 if spec.gate == "noisy" else 1) * d * N * s * (spec.gate != "cosine") \
        + (d * spec.proj_dim * s if spec.gate == "cosine" else 0) + T * k * 8
    disp_bytes = T * d * s + A * d * s + T * k * 8
    comb_bytes = A * d * s + T * d * s + T * k * 8
    stages = {
        "gate": {"ms": stage_ms["gate"], "GB/s": gate_bytes / (stage_ms["gate"] * 1e-3) / 1e9},
        "dispatch": {"ms": stage_ms["dispatch"], "GB/s": disp_bytes / (stage_ms["dispatch"] * 1e-3) / 1e9},
        "expert_ffn": {"ms": stage_ms["expert_ffn"], "TFLOP/s": ffn_flops / stage_ms["expert_ffn"] / 1e9,
                       "touched_weight_GB/s": touched_weight_bytes / stage_ms["expert_ffn"] / 1e6},
        "combine": {"ms": stage_ms["combine"], "GB/s": comb_bytes / (stage_ms["combine"] * 1e-3) / 1e9},
    }
    # load-balance terms on this step's routing (optional output; not in the step)
    aux_ws = api.workspace(dev.desc, _lib.MOE_WS_AUX)
    aux_imp = torch.empty(N, dtype=torch.float32, device="cuda")
    aux_loss = torch.empty(2, dtype=torch.float32, device="cuda")
    for _ in range(3):
        api.aux_loss(dev.desc, dev.topk_idx, dev.topk_w, aux_imp, aux_loss, aux_ws)
    a0, a1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(K):
        api.aux_loss(dev.desc, dev.topk_idx, dev.topk_w, aux_imp, aux_loss, aux_ws)
    a1.record(stream)
    torch.cuda.synchronize()
    stages["aux_loss"] = {"ms": a0.elapsed_time(a1) / K, "T*k": T * k}

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(spec, inp, args.cpu_seconds)
        if fp8:
            cpu["sample"] += ("; the oracle's FFN on the layer's own weights, whose cost does not depend on "
                              "the weights' storage format")

    out = {
        "metric": "MoE layer fwd tokens/s; expert GEMM % bf16 MFMA peak; dispatch/combine GB/s",
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": spec.dtype,
        "data": "synthetic (seeded normal inputs and random-init expert weights)",
        "config": {"workload": spec.name, "T": T, "d": d, "h": h, "N": N, "k": k, "gate": spec.gate,
                   "capacity_factor": spec.capacity_factor, "renorm": spec.renorm,
                   "capacity": int(dev.C), "kept_rows": A, "experts_touched": U,
                   "weights": "fp8_e4m3_block128" if fp8 else spec.dtype,
                   "combine": "in_ffn_launch" if folded else "separate"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages": stages,
        "staged_ms_per_step": staged_ms,
        "graph_ms_per_step": graph_ms,
        "graph4_ms_per_step": graph4_ms,
        "cold": cold_ms,
        "measured_peaks": peaks,
        "backward": backward,
    }
    print(json.dumps(out), flush=True)
    return 0


def dispatch_scaling():
    """moe_dispatch (count, scan where the count table is large, rows and
    permute kernels) on a seeded caller routing of T tokens over 64 experts
    (k = 2, Zipf-skewed choices), T from 16k to 256k: mean of 20 calls by
    events. Under a kernel trace the per-kernel times show that every
    kernel's time grows linearly with T (one JSON line per T)."""
    import torch

    from mixture_experts_sparse_gate_amd import _lib, api, workloads

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    rng = np.random.default_rng(0)
    for T in (16384, 32768, 65536, 131072, 262144):
        spec = workloads.MoESpec("dispatch_scaling", T=T, d=256, h=256, N=64, k=2, capacity_factor=1.25,
                                 gate="softmax", renorm=False, dtype="bf16")
        p = 1.0 / np.arange(1, spec.N + 1) ** 0.8
        p /= p.sum()
        first = rng.choice(spec.N, size=T, p=p)
        second = (first + 1 + rng.choice(spec.N - 1, size=T)) % spec.N
        idx = torch.from_numpy(np.stack([first, second], 1).astype(np.int32)).cuda()
        desc = api.desc_from_spec(spec)
        R = api.rows_bound(desc)
        dv = dict(dtype=torch.int32, device="cuda")
        x = torch.zeros(T, spec.d, dtype=torch.bfloat16, device="cuda")
        count, off = torch.empty(spec.N, **dv), torch.empty(spec.N + 1, **dv)
        row_of, tor = torch.empty(T * spec.k, **dv), torch.empty(R, **dv)
        x_perm = torch.empty(R, spec.d, dtype=torch.bfloat16, device="cuda")
        ws = api.workspace(desc, _lib.MOE_WS_DISPATCH)
        call = lambda: api.dispatch(desc, x, idx, count, off, row_of, tor, x_perm, ws=ws)
        for _ in range(3):
            call()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(20):
            call()
        b.record(stream)
        torch.cuda.synchronize()
        print(json.dumps({"T": T, "N": spec.N, "k": spec.k, "moe_dispatch_us": a.elapsed_time(b) / 20 * 1e3}),
              flush=True)
    return 0


def _dispatch_kernels(db):
    """Mean duration per dispatch kernel for each T of a --dispatch-scaling
    trace (the 23 calls per T follow each other in T order)."""
    import statistics
    c = sqlite3.connect(db)
    rows = [(_short(n), (b - a) / 1e3) for n, a, b in c.execute("select name, start, end from kernels order by start")]
    names = ("count_kernel", "scan_kernel", "rows_kernel", "permute_kernel")
    calls = []
    cur = {}
    for k, dur in rows:
        if k not in names:
            continue
        if k == "count_kernel" and cur:
            calls.append(cur)
            cur = {}
        cur[k] = dur
    calls.append(cur)
    out = []
    Ts = (16384, 32768, 65536, 131072, 262144)
    for i, T in enumerate(Ts):
        blk = calls[i * 23 + 3:(i + 1) * 23]
        kd = ", ".join(f"{k} {statistics.mean(c[k] for c in blk if k in c):.1f}" for k in names
                       if any(k in c for c in blk))
        out.append(f"T={T}: mean over {len(blk)} calls (us): {kd}")
    return out


def ffn_trace(args, dev, torch):
    """Per-item trace of the single-launch FFN on the trace build: the last of
    --steps back-to-back moe_forward calls (after --warmup), summarised per XCD
    and over time. Wall clock: a 100 MHz counter; clock = shader cycles over
    wall time of each item."""
    import numpy as np
    from mixture_experts_sparse_gate_amd import _lib, api

    lib = _lib.load(_lib.TRACE_LIB_PATH)
    nbytes = int(lib.moe_ffn_trace_bytes())
    if nbytes == 0:
        print("the trace build records no trace", file=sys.stderr)
        return 2
    spec = dev.spec
    tensors = dev.layer_tensors(inspect=True)
    for _ in range(args.warmup + args.steps):
        api.forward(dev.desc, tensors, dev.ws, lib_path=_lib.TRACE_LIB_PATH)
    torch.cuda.synchronize()
    buf = np.zeros(nbytes // 8, dtype=np.uint64)
    api._check(lib.moe_ffn_trace_read(buf.ctypes.data), "moe_ffn_trace_read", _lib.TRACE_LIB_PATH)
    rec = buf.reshape(-1, 8).astype(np.int64)
    if not (rec[:, 2] != 0).any():
        print("no single-launch FFN ran (the layer takes the two grouped-GEMM launches)", file=sys.stderr)
        return 2
    header = [f"command: {args.command}" if args.command else
              f"command: python3 <repo>/bench.py --workload {spec.name} --ffn-trace --warmup {args.warmup} --steps {args.steps}",
              "source: moe_ffn_trace_read on libmoe_gfx950_trace.so (MOE_FFN_TRACE), records of the last of "
              f"{args.warmup + args.steps} back-to-back moe_forward calls"]
    lines = summarize_ffn_trace(rec, spec, header)
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


def summarize_ffn_trace(rec, spec, header=()):
    """Summary lines of the single-launch FFN's per-item trace records
    (moe_ffn_trace_read layout, int64 [n, 8]; zero records unwritten): the
    records of the highest launch number only, per XCD (items, mean duration
    after the wait, mean clock, end of the last item), shader cycles per
    K-step of full tiles, and the clock over the launch in 8 bins. Wall
    clock: a 100 MHz counter; clock = shader cycles over wall time."""
    import numpy as np

    rec = rec[rec[:, 2] != 0]
    launch = rec[:, 5] >> 32
    rec = rec[launch == launch.max()]
    t0 = rec[:, 0].min()
    start, wait_end, end = (rec[:, 0] - t0) / 100.0, (rec[:, 1] - t0) / 100.0, (rec[:, 2] - t0) / 100.0  # us
    cyc = (rec[:, 4] - rec[:, 3]).astype(np.float64)
    mhz = cyc / np.maximum(rec[:, 2] - rec[:, 0], 1) * 100.0
    xcd, kind, tail = rec[:, 5] & 15, (rec[:, 5] >> 4) & 15, (rec[:, 5] >> 8) & 1
    span = end.max()
    busy = (end - wait_end).sum()
    nk = {1: (spec.d + 31) // 32, 2: (spec.h + 31) // 32}
    lines = list(header) + [
             f"workload: {spec.name}",
             f"items: {len(rec)}; span {span:.1f} us; tile time / (256 CUs x span): {busy / (256 * span):.3f}",
             "per XCD: end of its last item (us); per kind: items x mean duration after the wait (us) @ mean clock (MHz)"]
    names = {(1, 0): "GEMM1", (1, 1): "GEMM1 tail", (2, 0): "GEMM2", (2, 1): "GEMM2 tail"}
    for x in range(8):
        m = xcd == x
        if not m.any():
            continue
        parts = []
        for (k_, t_), nm in names.items():
            q = m & (kind == k_) & (tail == t_)
            if q.any():
                parts.append(f"{nm} {q.sum()}x{(end[q] - wait_end[q]).mean():.1f}@{mhz[q].mean():.0f}")
        lines.append(f"  XCD {x}: end {end[m].max():8.1f} | " + ", ".join(parts))
    for k_ in (1, 2):
        q = (kind == k_) & (tail == 0)
        if q.any():
            lines.append(f"GEMM{k_} full tiles: {cyc[q].mean():.0f} shader cycles per tile, "
                         f"{cyc[q].mean() / nk[k_]:.0f} per 32-deep K-step ({nk[k_]} steps, epilogue included; "
                         f"1024 cycles of MFMA work per step)")
    lines.append("clock over the launch (items by midpoint):")
    edges = np.linspace(0, span, 9)
    mid = (start + end) / 2
    for a, b in zip(edges[:-1], edges[1:]):
        q = (mid >= a) & (mid < b) if b < span else (mid >= a)
        if q.any():
            lines.append(f"  {a:7.0f}-{b:7.0f} us: {q.sum():4d} items, {mhz[q].mean():.0f} MHz, "
                         f"GEMM1 {(q & (kind == 1)).sum()}, GEMM2 {(q & (kind == 2)).sum()}")
    return lines


def graph_ab(dev, torch):
    """Three rounds of 20 eager moe_forward steps then 20 replays of one
    captured call, timed on the host; run under a kernel trace, the trace
    shows where the time goes (bench.py --summarize <db> --kind gaps)."""
    fwd = lambda: dev.run_forward(inspect=False)
    for _ in range(30):
        fwd()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fwd()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for rnd in range(3):
        for mode in ("eager", "graph"):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(20):
                g.replay() if mode == "graph" else fwd()
            torch.cuda.synchronize()
            print(f"round {rnd} {mode}: {(time.perf_counter() - t0) * 1e3 / 20:.4f} ms/step", flush=True)
    return 0


def _gaps(db):
    """Kernel durations and device gaps of the last 3 x (20 eager + 20 graph)
    steps of a --graph-ab trace."""
    import statistics
    c = sqlite3.connect(db)
    rows = list(c.execute("select name, start, end from kernels order by start"))
    steps, cur = [], []
    for n, a, b in rows:
        k = _short(n)
        if k in ("gate_fused_kernel", "gate_partial_kernel", "gate_logits_kernel", "cosine_gate_kernel") and cur:
            steps.append(cur)
            cur = []
        cur.append((k, a, b))
    steps.append(cur)
    steps = [st for st in steps if any("ffn" in k or "grouped_gemm" in k for k, _, _ in st)][-120:]
    out = []
    for i in range(6):
        blk = steps[i * 20:(i + 1) * 20]
        mode = "eager" if i % 2 == 0 else "graph"
        per = {}
        for st in blk:
            for k, a, b in st:
                per.setdefault(k, []).append((b - a) / 1e3)
        inner = statistics.mean(sum(max(0, st[j + 1][1] - st[j][2]) for j in range(len(st) - 1)) / 1e3 for st in blk)
        between = statistics.mean((blk[j + 1][0][1] - blk[j][-1][2]) / 1e3 for j in range(len(blk) - 1))
        span = (blk[-1][-1][2] - blk[0][0][1]) / 1e3 / len(blk)
        kd = ", ".join(f"{k} {statistics.mean(v):.1f}" for k, v in per.items())
        out.append(f"round {i // 2} {mode}: per-step span {span:.1f} us; gaps inside a step {inner:.1f} us; "
                   f"gap before the next step {between:.1f} us; kernels (us): {kd}")
    return out


def measured_peaks(api, torch, stream):
    """HBM copy bandwidth (read + write bytes over 1 GiB, beyond the 256 MB
    last-level cache) and the bf16 MFMA rate with register operands only,
    each the best of 5 timed launches after 2 untimed ones."""
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)

    def best(fn):
        for _ in range(2):
            fn()
        ts = []
        for _ in range(5):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            fn()
            b.record(stream)
            b.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    t_copy = best(lambda: api.probe_copy(src, dst))
    del src, dst
    iters = 40000
    flops, sink = api.probe_mfma(iters)
    t_mfma = best(lambda: api.probe_mfma(iters, sink))
    # sustained: launches back to back for about 2 s; the rate of the last
    # 0.5 s (groups of 20 launches timed by events)
    t0, rates = time.perf_counter(), []
    while time.perf_counter() - t0 < 2.0:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(20):
            api.probe_mfma(iters, sink)
        b.record(stream)
        b.synchronize()
        rates.append((time.perf_counter() - t0, 20 * flops / (a.elapsed_time(b) * 1e-3) / 1e12))
    tail = [r for t, r in rates if t >= rates[-1][0] - 0.5]
    return {"hbm_copy_GB/s": 2 * n / t_copy / 1e9, "hbm_copy_bytes": 2 * n,
            "mfma_bf16_TFLOP/s": flops / t_mfma / 1e12, "mfma_flops": flops,
            "mfma_bf16_sustained_TFLOP/s": sum(tail) / len(tail)}


def cpu_baseline(spec, inp, target_s: float):
    """The oracle as it is, on the host cores, repeated over the workload (or a
    token prefix of it when one full pass would take far longer than the target)."""
    from threadpoolctl import threadpool_info

    from oracle import moe_oracle as O

    blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    # estimate: fp64 BLAS at a few tens of GFLOP/s per core
    T = spec.T
    est_flops = 4.0 * T * spec.k * spec.d * spec.h
    sub_T = T
    if est_flops > 50e9 * blas_threads * target_s:
        sub_T = max(1, int(T * 50e9 * blas_threads * target_s / est_flops))
    sub = spec.with_(T=sub_T)
    sub_inp = inp
    if sub_T != T:
        import copy
        sub_inp = copy.copy(inp)
        sub_inp.spec = sub
        sub_inp.x = inp.x[:sub_T]
        if inp.noise is not None:
            sub_inp.noise = inp.noise[:sub_T]
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.forward(sub, sub_inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= target_s or el / reps * (reps + 1) > 3 * target_s:
            break
    what = (f"oracle forward over all {T} tokens" if sub_T == T else
            f"oracle forward over the first {sub_T} of {T} tokens (same capacity factor)")
    return {"value": sub_T * reps / el, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
            "sample": f"{what}, {reps} repetition(s), {el:.1f} s, fp64 NumPy"}


# ---------------------------------------------------------------- summaries

def _kernel_rows(db):
    c = sqlite3.connect(db)
    return list(c.execute("select name, total_calls, total_duration, average, percentage from top_kernels"))


def _short(name: str) -> str:
    m = re.search(r"grouped_gemm_kernel.*?Cfg<([^>]*)>", name)
    if m:
        return "grouped_gemm_kernel<" + m.group(1) + ">"
    m = re.search(r"CfgI(\w+?)EEELb([01])EEEvNS_10GemmParamsE", name)
    if m:
        # the Cfg's last flag: the dual (pre-activation and GELU) output; the
        # kernel's flag: the ping-pong K loop
        return ("grouped_gemm_kernel<" + m.group(1) + (", U and H" if m.group(1).endswith("Lb1") else "") +
                (", ping-pong" if m.group(2) == "1" else "") + ">")
    m = re.search(r"CfgI(\w+?)EEEEEvNS_10GemmParamsE", name)
    if m:
        return "grouped_gemm_kernel<" + m.group(1) + (", U and H" if m.group(1).endswith("Lb1") else "") + ">"
    m = re.search(r"fused_ffn_kernelINS0_3CfgI(\w+?)EEELb([01])ELb([01])EEEvNS0_8FusedFfnE", name)
    if m:
        return ("fused_ffn_kernel<" + m.group(1) + (", combine in launch" if m.group(2) == "1" else "") +
                (", ping-pong" if m.group(3) == "1" else "") + ">")
    m = re.search(r"fused_ffn_kernel<.*?Cfg<([^>]*)>, (true|false), (true|false)>", name)
    if m:
        return ("fused_ffn_kernel<" + m.group(1) + (", combine in launch" if m.group(2) == "true" else "") +
                (", ping-pong" if m.group(3) == "true" else "") + ">")
    # backward GEMMs: tile, operand layouts, epilogue, output type, ragged K
    lay, epi = {"0": "Kc", "1": "Ks"}, {"0": "plain", "1": "dU"}
    m = re.search(r"bwd_gemm_kernelILi(\d+)ELNS_9BwdLayoutE(\d)ELS\d+_(\d)ELNS_6BwdEpiE(\d)E(\w+?)Lb(\d)E", name)
    if m:
        ts, a_, b_, e_, o_, rk = m.groups()
        o_ = "bf16" if "DF16b" in o_ else "f32"
        return f"bwd_gemm_kernel<{ts} A:{lay[a_]} B:{lay[b_]} {epi[e_]} {o_}{' raggedK' if rk == '1' else ''}>"
    m = re.search(r"bwd_gemm_kernel<(\d+), \(moe::BwdLayout\)(\d), \(moe::BwdLayout\)(\d), "
                  r"\(moe::BwdEpi\)(\d), (\w+), (true|false)>", name)
    if m:
        ts, a_, b_, e_, o_, rk = m.groups()
        o_ = "bf16" if "bf16" in o_ or "bfloat" in o_ else "f32"
        return f"bwd_gemm_kernel<{ts} A:{lay[a_]} B:{lay[b_]} {epi[e_]} {o_}{' raggedK' if rk == 'true' else ''}>"
    for key in ("gate_logits_kernel", "gate_select_kernel", "cosine_select_kernel", "count_kernel",
                "scan_kernel", "slots_kernel", "permute_kernel", "combine_kernel", "fill_kernel",
                "gate_fused_kernel", "gate_partial_kernel", "gate_finish_kernel", "rows_kernel",
                "copy_kernel", "mfma_kernel", "ffn_status_kernel", "cosine_gate_kernel", "aux_partial_kernel",
                "aux_final_kernel", "quantize_fp8_kernel", "bwd_token_kernel", "scale_rows_kernel",
                "gate_grad_partial_kernel", "gate_grad_final_kernel", "importance_grad_kernel",
                "column_sum_partial_kernel", "colsum_kernel", "probe"):
        if key in name:
            return key
    return name[:70]


def _pmc_per_kernel(db, counter):
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, kernel_name, grid_size, sum(value) from counters_collection "
                     "where counter_name = ? group by dispatch_id", (counter,))
    return [(d, n, g, v) for d, n, g, v in rows]


def _pmc_all(db):
    """{counter: [(dispatch_id, kernel_name, value summed over the dispatch's instances)]}"""
    c = sqlite3.connect(db)
    rows = c.execute("select counter_name, dispatch_id, kernel_name, sum(value) from counters_collection "
                     "group by counter_name, dispatch_id")
    out = {}
    for name, d, k, v in rows:
        out.setdefault(name, []).append((d, k, v))
    return out


def summarize(args):
    lines = [f"command: {args.command}"] if args.command else []
    if args.kind in ("gaps", "dispatch"):
        if args.kind == "gaps":
            lines.append("source: rocprofv3 --kernel-trace of bench.py --graph-ab (kernels table)")
            lines.append(f"workload: {args.workload}")
            lines.extend(_gaps(args.summarize))
        else:
            lines.append("source: rocprofv3 --kernel-trace of bench.py --dispatch-scaling (kernels table)")
            lines.extend(_dispatch_kernels(args.summarize))
        text = "\n".join(lines) + "\n"
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text)
        return 0
    if args.kind == "pmc":
        # per-dispatch averages of each counter over the expert FFN's launches
        # (the later half of them: warm steps), from one or more passes
        lines.append("source: rocprofv3 --pmc passes (one results.db per pass); values per dispatch, "
                     "mean over the later half of the FFN kernel's dispatches")
        lines.append(f"workload: {args.workload}")
        for db in args.pmc_dbs:
            for name, rows in sorted(_pmc_all(db).items()):
                sel = [v for d, k, v in rows if "fused_ffn_kernel" in k]
                kern = "fused_ffn_kernel"
                if not sel:
                    sel = [v for d, k, v in rows if "grouped_gemm_kernel" in k and "DF16bfLi" not in k]
                    kern = "grouped_gemm_kernel (both GEMMs, per launch)"
                if not sel:
                    continue
                steady = sel[len(sel) // 2:]
                lines.append(f"{name}: {sum(steady) / len(steady):.6g}   [{kern}, {len(steady)} dispatches]")
        lines.append(f"gemm_source_sha256_16: {gemm_source_hash()}")
        text = "\n".join(lines) + "\n"
        if args.out:
            with open(args.out, "w") as f:
                f.write(text)
        print(text)
        return 0
    if args.kind == "stats":
        lines.append(f"source: rocprofv3 --kernel-trace --stats (top_kernels of {os.path.basename(args.summarize)})")
        lines.append(f"{'kernel':70s} {'calls':>6s} {'total_us':>12s} {'avg_us':>10s} {'%':>7s}")
        for n, calls, tot, avg, pct in _kernel_rows(args.summarize):
            lines.append(f"{_short(n):70s} {calls:6d} {tot:12.1f} {avg:10.2f} {pct:7.2f}")
    else:
        out = {}
        for tag, db, counter in (("fetch", args.fetch_db, "FETCH_SIZE"), ("write", args.write_db, "WRITE_SIZE")):
            rows = _pmc_per_kernel(db, counter)
            copies = [v for d, n, g, v in rows if "copy" in n.lower() and "bfloat16" not in n.lower()]
            calib_kib = max(copies) if copies else None
            # expert-FFN launches only: one fused_ffn_kernel per step, or
            # GEMM1 and GEMM2 alternating; the cosine gate's projection (bf16
            # in, fp32 out: "DF16bf" in the name) is not
            fused = [v for d, n, g, v in rows if "fused_ffn_kernel" in n]
            gemm = [v for d, n, g, v in rows if "grouped_gemm_kernel" in n and "DF16bfLi" not in n]
            out[tag] = dict(calib_kib=calib_kib, gemm_kib=gemm, fused_kib=fused)
        mib = None
        if args.command:
            m = re.search(r"--calib-copy-mib\s+(\d+)", args.command)
            mib = int(m.group(1)) if m else None
        known_kib = (mib or 0) * 1024
        lines.append("source: rocprofv3 --pmc FETCH_SIZE, then --pmc WRITE_SIZE (KiB per dispatch)")
        res = {}
        for tag in ("fetch", "write"):
            o = out[tag]
            fac = known_kib / o["calib_kib"] if o["calib_kib"] and known_kib else float("nan")
            g = o["gemm_kib"]
            per_step = list(o["fused_kib"]) if o["fused_kib"] else [g[i] + g[i + 1] for i in range(0, len(g) - 1, 2)]
            steady = per_step[len(per_step) // 2:] or per_step
            kib = sum(steady) / max(len(steady), 1)
            res[tag] = kib * fac * 1024
            lines.append(f"{tag}_calib_copy_kib: {o['calib_kib']}")
            lines.append(f"{tag}_scale_factor: {fac:.4f}")
            lines.append(f"{tag}_ffn_kib_per_step_raw: {kib:.1f}")
        lines.append(f"workload: {args.workload}")
        # a second calibration point for FETCH_SIZE: the gate kernel reads x
        # (T d s bytes) and the small gate matrices once per call
        try:
            from mixture_experts_sparse_gate_amd import workloads as _w
            sp = _w.get(args.workload)
            gate = [v for d_, n, g, v in _pmc_per_kernel(args.fetch_db, "FETCH_SIZE") if "gate_fused_kernel" in n]
            if gate:
                steady = gate[len(gate) // 2:]
                fac = known_kib / out["fetch"]["calib_kib"] if out["fetch"]["calib_kib"] and known_kib else float("nan")
                got = sum(steady) / len(steady) * fac * 1024
                x_bytes = sp.T * sp.d * (2 if sp.dtype == "bf16" else 4)
                lines.append(f"gate_fetch_bytes_per_call: {got:.0f}")
                lines.append(f"gate_x_bytes_per_call: {x_bytes}")
                lines.append(f"gate_fetch_over_x: {got / x_bytes:.4f}")
        except Exception as e:  # the check is informative only
            lines.append(f"gate_fetch_check: unavailable ({e})")
        lines.append(f"ffn_hbm_bytes_per_step: {res['fetch'] + res['write']:.0f}")
        lines.append(f"ffn_hbm_read_bytes_per_step: {res['fetch']:.0f}")
        lines.append(f"ffn_hbm_write_bytes_per_step: {res['write']:.0f}")
        lines.append(f"gemm_source_sha256_16: {gemm_source_hash()}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)
    return 0


if __name__ == "__main__":
    sys.exit(main())
