"""The debug build's check of a caller's routing (csrc/routing_check.cpp),
compiled on its own with g++ and run on the CPU: every index in [0, N),
no expert named twice by one token, the first offending (t, j) reported."""
import ctypes
import os
import subprocess

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "mixture_experts_sparse_gate_amd", "csrc", "routing_check.cpp")


@pytest.fixture(scope="module")
def check(tmp_path_factory):
    out = str(tmp_path_factory.mktemp("routing_check") / "librouting_check.so")
    subprocess.run(["g++", "-O1", "-std=c++17", "-shared", "-fPIC", "-Wall", SRC, "-o", out], check=True)
    lib = ctypes.CDLL(out)
    fn = lib.moe_check_routing_host
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, ctypes.c_char_p,
                   ctypes.c_size_t]

    def run(idx, N):
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        T, k = idx.shape
        msg = ctypes.create_string_buffer(256)
        rc = fn(idx.ctypes.data, T, k, N, msg, len(msg))
        return rc, msg.value.decode()
    return run


def first_problem(idx, N):
    """Brute force: (code, t, j) of the first entry out of range (1) or
    repeating an earlier expert of its token (2), scanning tokens then choices."""
    T, k = idx.shape
    for t in range(T):
        for j in range(k):
            e = int(idx[t, j])
            if not 0 <= e < N:
                return 1, t, j
            if e in [int(v) for v in idx[t, :j]]:
                return 2, t, j
    return 0, -1, -1


def test_valid_routing_passes(check):
    rng = np.random.default_rng(0)
    idx = np.stack([rng.choice(64, 4, replace=False) for _ in range(500)])
    assert check(idx, 64) == (0, "")


def test_out_of_range_and_repeats_are_named(check):
    idx = np.array([[0, 1], [2, 3], [4, 4], [9, 1]], np.int32)
    rc, msg = check(idx, 8)
    assert rc == 2 and "token 2 names expert 4 twice" in msg
    idx[2, 1] = 5
    rc, msg = check(idx, 8)
    assert rc == 1 and "(3, 0) = 9" in msg
    idx[3, 0] = -1
    rc, msg = check(idx, 8)
    assert rc == 1 and "(3, 0) = -1" in msg


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 40), st.integers(1, 6), st.integers(1, 9), st.integers(0, 2**31 - 1))
def test_matches_brute_force(check, T, k, N, seed):
    rng = np.random.default_rng(seed)
    idx = rng.integers(-1, N + 1, size=(T, k)).astype(np.int32)
    if rng.random() < 0.5 and k <= N:  # often a valid routing
        idx = np.stack([rng.choice(N, k, replace=False) for _ in range(T)]).astype(np.int32)
    code, t, j = first_problem(idx, N)
    rc, msg = check(idx, N)
    assert rc == code
    if code == 1:
        assert f"({t}, {j})" in msg
    elif code == 2:
        assert f"token {t} names expert {int(idx[t, j])} twice" in msg


DRIVER = r"""
#include <stdio.h>
#include <string.h>
#include "routing_check.h"
int main() {
  char msg[64];
  const int32_t ok[6] = {0, 1, 2, 3, 4, 5}, rep[6] = {0, 1, 2, 2, 4, 5}, bad[6] = {0, 1, 2, 3, 4, 77};
  if (moe_check_routing_host(ok, 3, 2, 6, msg, sizeof msg) != 0) return 10;
  if (moe_check_routing_host(rep, 3, 2, 6, msg, sizeof msg) != 2) return 11;
  if (moe_check_routing_host(bad, 3, 2, 6, msg, 8) != 1 || strlen(msg) != 7) return 12;  /* message cut to fit */
  if (moe_check_routing_host(bad, 3, 2, 6, NULL, 0) != 1) return 13;
  if (moe_check_routing_host(ok, 0, 2, 6, msg, sizeof msg) != 0) return 14;
  puts("ok");
  return 0;
}
"""


def test_under_address_and_undefined_behaviour_sanitizers(tmp_path):
    """The check compiled with ASan and UBSan into a small driver program
    (its own process: the sanitizer runtimes must load first)."""
    drv = tmp_path / "driver.cpp"
    drv.write_text(DRIVER)
    exe = str(tmp_path / "driver")
    inc = os.path.dirname(SRC)
    subprocess.run(["g++", "-O1", "-g", "-std=c++17", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    f"-I{inc}", str(drv), SRC, "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", (r.returncode, r.stdout, r.stderr)
