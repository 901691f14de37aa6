"""ctypes view of libmoe_gfx950.so and of the structs in include/moe.h."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_gfx950.so")
# the same library with the debug checks of caller routing (MOE_DEBUG_CHECKS)
DEBUG_LIB_PATH = os.path.join(HERE, "libmoe_gfx950_debug.so")
# the same library recording a per-item trace of the single-launch FFN (MOE_FFN_TRACE)
TRACE_LIB_PATH = os.path.join(HERE, "libmoe_gfx950_trace.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(5)
MOE_F32, MOE_BF16 = 0, 1
MOE_GATE_SOFTMAX, MOE_GATE_NOISY, MOE_GATE_COSINE = 0, 1, 2
MOE_WS_ROUTE, MOE_WS_DISPATCH, MOE_WS_FORWARD, MOE_WS_FFN, MOE_WS_AUX, MOE_WS_BACKWARD = 0, 1, 2, 3, 4, 5
MOE_FLAG_COMBINE_IN_FFN = 1


class MoeDesc(ctypes.Structure):
    _fields_ = [
        ("T", c_int64),
        ("d", c_int32),
        ("h", c_int32),
        ("N", c_int32),
        ("k", c_int32),
        ("capacity_factor", c_double),
        ("gate", c_int32),
        ("renorm", c_int32),
        ("dtype", c_int32),
        ("proj_dim", c_int32),
        ("inv_temperature", c_float),
        ("flags", c_int32),
    ]


class MoeLayerTensors(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in (
        "x", "w_gate", "w_noise", "noise", "proj", "expert_emb", "logit_bias",
        "W1", "b1", "W2", "b2", "y",
        "logits", "topk_idx", "topk_w", "expert_count", "expert_off", "row_of", "token_of_row")]


class MoeBackwardTensors(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in (
        "x", "w_gate", "w_noise", "noise", "W1", "b1", "W2", "b2",
        "logits", "topk_idx", "topk_w", "expert_off", "row_of", "token_of_row", "dy",
        "dx", "dW1", "dW2", "db1", "db2", "dw_gate", "dw_noise", "dlogit_bias")]


class MoeFp8Weights(ctypes.Structure):
    _fields_ = [(name, c_void_p) for name in ("W1q", "S1", "W2q", "S2")]


# name -> (restype, argtypes)
SIGNATURES = {
    "moe_capacity": (c_int64, [POINTER(MoeDesc)]),
    "moe_rows_bound": (c_int64, [POINTER(MoeDesc)]),
    "moe_workspace_size": (c_int, [POINTER(MoeDesc), c_int, POINTER(c_size_t)]),
    "moe_route": (c_int, [POINTER(MoeDesc)] + [c_void_p] * 10 + [c_void_p, c_size_t, c_void_p]),
    "moe_dispatch": (c_int, [POINTER(MoeDesc)] + [c_void_p] * 7 + [c_void_p, c_size_t, c_void_p]),
    "moe_expert_ffn": (c_int, [POINTER(MoeDesc)] + [c_void_p] * 8 + [c_void_p, c_size_t, c_void_p]),
    "moe_combine": (c_int, [POINTER(MoeDesc)] + [c_void_p] * 4 + [c_void_p]),
    "moe_forward": (c_int, [POINTER(MoeDesc), POINTER(MoeLayerTensors), c_void_p, c_size_t, c_void_p]),
    "moe_time_ffn_launches": (c_int, [c_void_p, c_void_p]),
    "moe_backward": (c_int, [POINTER(MoeDesc), POINTER(MoeBackwardTensors), c_void_p, c_void_p, c_size_t, c_void_p]),
    "moe_forward_noalloc": (c_int, [POINTER(MoeDesc), POINTER(MoeLayerTensors), c_void_p]),
    "moe_noalloc_scratch_bytes": (c_size_t, []),
    "moe_ffn_status": (c_int, [POINTER(MoeDesc), c_int, c_void_p, c_size_t, c_void_p, c_void_p]),
    "moe_probe_copy": (c_int, [c_void_p, c_void_p, c_int64, c_void_p]),
    "moe_probe_mfma": (c_int, [c_int32, c_void_p, POINTER(c_int64), c_void_p]),
    "moe_probe_mfma_sink_floats": (c_int64, []),
    "moe_quantize_fp8": (c_int, [c_void_p, c_int32, c_int32, c_int32, c_int32, c_void_p, c_void_p, c_void_p]),
    "moe_expert_ffn_fp8": (c_int, [POINTER(MoeDesc)] + [c_void_p] * 10 + [c_void_p]),
    "moe_forward_fp8": (c_int, [POINTER(MoeDesc), POINTER(MoeLayerTensors), POINTER(MoeFp8Weights), c_void_p,
                                c_size_t, c_void_p]),
    "moe_aux_loss": (c_int, [POINTER(MoeDesc), c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                             c_void_p]),
    "moe_ffn_trace_bytes": (c_size_t, []),
    "moe_ffn_trace_read": (c_int, [c_void_p]),
    "moe_status_string": (c_char_p, [c_int]),
    "moe_last_error": (c_char_p, []),
    "moe_version": (c_char_p, []),
}

_libs = {}


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Loads a build of the HIP library once (the release build by default).
    Raises if it has not been built: there is no other implementation to fall
    back to."""
    if path not in _libs:
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is missing: build it with `python -m mixture_experts_sparse_gate_amd.build` "
                "(the MoE layer runs only on the HIP kernels)")
        lib = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _libs[path] = lib
    return _libs[path]
