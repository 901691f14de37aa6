"""The FFN trace summary (bench.py --ffn-trace) on synthetic records: host
logic only, no GPU. Records follow moe_ffn_trace_read's layout: wall clock at
start / after the wait / at the end (100 MHz), shader cycles at start / end,
XCD | kind << 4 | tail << 8 | launch << 32, row tile, first column."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import bench  # noqa: E402
from mixture_experts_sparse_gate_amd import workloads  # noqa: E402


def _rec(t0, tw, t1, c0, c1, xcd, kind, tail, launch):
    return [t0, tw, t1, c0, c1, xcd | (kind << 4) | (tail << 8) | (launch << 32), 0, 0]


def test_summary_uses_the_last_launch_and_derives_clock_and_cycles():
    spec = workloads.get("noisy_top2_bf16")  # d = 1024: 32 K-steps for GEMM1; h = 2048: 64 for GEMM2
    recs = []
    # an earlier launch that must be ignored (older timestamps, launch 1)
    recs.append(_rec(10, 10, 500, 0, 10_000_000, 3, 1, 0, 1))
    # launch 2: XCD 0 runs a GEMM1 tile from 1000 to 4000 (30 us) at 2 GHz
    # (60000 cycles over 3000 ticks of 10 ns); XCD 1 a GEMM2 tile that waits
    # 5 us then runs 40 us at 1.5 GHz (67500 cycles over 4500 ticks)
    recs.append(_rec(1000, 1000, 4000, 5_000, 65_000, 0, 1, 0, 2))
    recs.append(_rec(1500, 2000, 6000, 0, 67_500, 1, 2, 0, 2))
    # a GEMM1 tail tile on XCD 1, 10 us at 1 GHz
    recs.append(_rec(1000, 1000, 2000, 0, 10_000, 1, 1, 1, 2))
    rec = np.array(recs + [[0] * 8] * 3, dtype=np.int64)  # unwritten records stay zero
    lines = bench.summarize_ffn_trace(rec, spec, ["command: test"])
    text = "\n".join(lines)
    assert lines[0] == "command: test"
    # three items of launch 2; span from the earliest start (1000) to the last end (6000): 50 us
    assert "items: 3; span 50.0 us" in text
    # busy = 30 + 40 + 10 us of tile time over 256 CUs x 50 us
    assert f"{80 / (256 * 50):.3f}" in text
    xcd0 = next(l for l in lines if l.startswith("  XCD 0:"))
    xcd1 = next(l for l in lines if l.startswith("  XCD 1:"))
    assert "end     30.0" in xcd0 and "GEMM1 1x30.0@2000" in xcd0
    assert "end     50.0" in xcd1 and "GEMM2 1x40.0@1500" in xcd1 and "GEMM1 tail 1x10.0@1000" in xcd1
    assert not any(l.startswith("  XCD 3:") for l in lines)  # the older launch's record
    # cycles per K-step of full tiles: 60000 / 32 and 67500 / 64
    assert "GEMM1 full tiles: 60000 shader cycles per tile, 1875 per 32-deep K-step (32 steps" in text
    assert "GEMM2 full tiles: 67500 shader cycles per tile, 1055 per 32-deep K-step (64 steps" in text
