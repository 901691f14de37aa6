"""Throughput of the sparse-gated MoE layer forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is one pass of the whole layer (gate, dispatch, expert FFN,
combine) over one batch of seeded synthetic tokens, through the single
moe_forward entry point, with every input already resident in HBM. W warmup
steps, then exactly K timed steps bracketed by torch.cuda.synchronize(); the
headline value is T tokens over the mean step time.

Besides the headline:
  - stages: the same layer through the four stage entry points, with HIP
    events recorded on the launch stream between them; their averages give
    each stage's duration; aux_loss: moe_aux_loss (per-expert importance and
    the two load-balance losses) on the step's routing, timed the same way;
  - graph_ms_per_step: moe_forward captured once in a HIP graph and replayed
    (no host launch cost per kernel);
  - cold: each step timed alone by events after writing a 512 MiB buffer
    (twice the last-level cache), median / p10 / p90.
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


GEMM_SRC = os.path.join(ROOT, "mixture_experts_sparse_gate_amd", "csrc", "gemm.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_hash() -> str:
    with open(GEMM_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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
    ap.add_argument("--workload", default="noisy_top2_bf16")
    ap.add_argument("--weights", choices=["layer", "fp8"], default="layer",
                    help="expert weights in the layer's dtype, or block-FP8 (moe_forward_fp8; bf16 layers)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target CPU time of the oracle baseline (0 disables it)")
    ap.add_argument("--skip-extras", action="store_true",
                    help="time only the warm steps (no graph replay, no cold-cache steps): counter runs")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="run one device copy of this many MiB first (counter calibration)")
    ap.add_argument("--summarize", default=None, help="rocprofv3 results.db to condense (no GPU)")
    ap.add_argument("--kind", choices=["stats", "traffic"], default="stats")
    ap.add_argument("--fetch-db", default=None, help="with --kind traffic: the FETCH_SIZE results.db")
    ap.add_argument("--write-db", default=None, help="with --kind traffic: the WRITE_SIZE results.db")
    ap.add_argument("--command", default="", help="command line recorded in the summary")
    ap.add_argument("--out", default=None)
    args = ap.parse_args()

    if args.summarize or args.kind == "traffic" and args.fetch_db:
        return summarize(args)

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
    dev = api.DeviceLayer(inp)
    fp8 = args.weights == "fp8"
    if fp8:
        if spec.dtype != "bf16":
            print("--weights fp8 needs a bf16 workload", file=sys.stderr)
            return 2
        dev.quantize_weights_fp8()  # model preparation, outside every timed region
    torch.cuda.synchronize()
    log(f"[bench] {spec.name}: inputs ready in {time.perf_counter() - t_gen:.1f}s")

    stream = torch.cuda.current_stream()
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
    graph_ms = None
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
                   "weights": "fp8_e4m3_block128" if fp8 else spec.dtype},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stages": stages,
        "staged_ms_per_step": staged_ms,
        "graph_ms_per_step": graph_ms,
        "cold": cold_ms,
    }
    print(json.dumps(out), flush=True)
    return 0


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
    m = re.search(r"CfgI(\w+?)EEEEEvNS_10GemmParamsE", name)
    if m:
        return "grouped_gemm_kernel<" + m.group(1) + ">"
    m = re.search(r"fused_ffn_kernelINS0_3CfgI(\w+?)EEEEEvNS0_8FusedFfnE", name)
    if m:
        return "fused_ffn_kernel<" + m.group(1) + ">"
    for key in ("gate_logits_kernel", "gate_select_kernel", "cosine_select_kernel", "count_kernel",
                "scan_kernel", "slots_kernel", "permute_kernel", "combine_kernel", "fill_kernel",
                "gate_fused_kernel", "gate_partial_kernel", "gate_finish_kernel", "rows_kernel"):
        if key in name:
            return key
    return name[:70]


def _pmc_per_kernel(db, counter):
    c = sqlite3.connect(db)
    rows = c.execute("select dispatch_id, kernel_name, grid_size, sum(value) from counters_collection "
                     "where counter_name = ? group by dispatch_id", (counter,))
    return [(d, n, g, v) for d, n, g, v in rows]


def summarize(args):
    lines = [f"command: {args.command}"] if args.command else []
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
