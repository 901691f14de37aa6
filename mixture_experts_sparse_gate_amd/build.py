"""Builds libmoe_gfx950.so from csrc/*.hip with hipcc for gfx950.

    python -m mixture_experts_sparse_gate_amd.build [-j JOBS]

Objects go to <repo>/_build/ and the libraries next to this file:
libmoe_gfx950.so; libmoe_gfx950_debug.so, the same library with the
debug checks of caller-supplied routing (-DMOE_DEBUG_CHECKS: moe_dispatch
copies topk_idx to the host and rejects indices outside [0, N) or repeated
within a token); and libmoe_gfx950_trace.so, the same library whose
single-launch FFN records a per-item trace (-DMOE_FFN_TRACE, read with
moe_ffn_trace_read). Every call recompiles, so a call always checks that the
current sources compile.
"""
from __future__ import annotations

import argparse
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_NAME = "libmoe_gfx950.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
ARCH = "gfx950"

SOURCES = ["gate.hip", "dispatch.hip", "gemm.hip", "combine.hip", "aux.hip", "quant.hip", "probe.hip", "backward.hip",
           "capi.hip"]
HOST_SOURCES = ["routing_check.cpp"]
DEBUG_LIB_NAME = "libmoe_gfx950_debug.so"
DEBUG_LIB_PATH = os.path.join(HERE, DEBUG_LIB_NAME)
TRACE_LIB_NAME = "libmoe_gfx950_trace.so"
TRACE_LIB_PATH = os.path.join(HERE, TRACE_LIB_NAME)
# sources compiled again for the trace build (MOE_FFN_TRACE)
TRACE_SOURCES = ["gemm.hip", "capi.hip"]

HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-fvisibility=hidden", f"-I{INCLUDE}",
    # packed fp32 instructions stay off: the compiler emits plain v_fma/v_add
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP kernels)")


HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-fvisibility=hidden"]


def _compile(job) -> str:
    src, variant = job if isinstance(job, tuple) else (job, "")
    stem = os.path.splitext(src)[0] + (f"_{variant}" if variant else "")
    obj = os.path.join(BUILD_DIR, stem + ".o")
    defines = {"": [], "debug": ["-DMOE_DEBUG_CHECKS"], "trace": ["-DMOE_FFN_TRACE"]}[variant]
    if src.endswith(".cpp"):
        cmd = ["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    else:
        cmd = [hipcc(), *HIP_FLAGS, *defines, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msg = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{msg}")
    if msg.strip():
        print(msg, file=sys.stderr)
    return obj


def _link(objs, path: str) -> None:
    tmp = path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}{r.stderr}")
    os.replace(tmp, path)


def build(jobs: int = 0, verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs_list = SOURCES + HOST_SOURCES + [("capi.hip", "debug")] + [(src, "trace") for src in TRACE_SOURCES]
    jobs = jobs or min(len(jobs_list), max(1, os.cpu_count() or 1), 16)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, jobs_list))
    nrel = len(SOURCES) + len(HOST_SOURCES)
    release = objs[:nrel]
    debug_capi, trace_objs = objs[nrel], objs[nrel + 1:]

    def without(names):
        return [o for o in release if os.path.basename(o) not in names]

    _link(without({"capi.o"}) + [debug_capi], DEBUG_LIB_PATH)
    _link(without({os.path.splitext(s)[0] + ".o" for s in TRACE_SOURCES}) + trace_objs, TRACE_LIB_PATH)
    _link(release, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}, {DEBUG_LIB_NAME} and {TRACE_LIB_NAME}")
    return LIB_PATH


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("-j", "--jobs", type=int, default=0)
    build(ap.parse_args().jobs)
