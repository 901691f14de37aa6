"""Block-FP8 expert weights: the oracle's E4M3 encoder and decoder and its
block quantiser.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the tests, the package smoke check
(``__graft_entry__.smoke``) and the CPU-baseline leg of ``bench.py`` may
import or run anything in this directory. It shares no code with the HIP
path and imports nothing from it: it receives plain NumPy arrays.

What the pages fix: expert weights held in FP8 to shrink the model
("MoE架构：突破单卡算力瓶颈的密钥" §1.3, FP8 mixed precision) with a scale per
block ("Block FP8" serving on MI300 in the table of the CUDA-to-ROCm section
of "4大技术模块掌握Tutel MoE…"; fp8 quantisation halving memory in its vLLM
section). They fix neither the FP8 encoding nor the block shape. Readings
(each listed with its reason in the design notes):

  encoding  OCP E4M3 ("e4m3fn"): sign, 4 exponent bits with bias 7, 3 mantissa
            bits; exponent field 0 holds subnormals m * 2^-9; no infinities;
            0x7F and 0xFF are NaN; the largest finite magnitude is 448
  blocks    128 x 128 blocks of each expert's [K, Ncols] weight matrix
  scale     s = amax / 448 in fp32 (one IEEE division), amax the largest |w|
            of the block (w widened exactly to fp32); an all-zero block has
            s = 0 and zero codes
  codes     q = E4M3(w / s): the fp32 quotient rounded to the nearest E4M3
            value, ties to the even code; the sign bit is w's. A quotient
            above 448 in magnitude (possible only when s is an inexact fp32
            subnormal) saturates to 448
  dequant   w' = decode(q) * s, exact in float64

Both decisions (each scale and each code) are taken in fp32, the precision
the quantisation kernel takes them in, so codes compare bit for bit.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
BLOCK = 128


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each E4M3 code byte, in float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2((e - 7).astype(np.float64)))
    out = sign * mag
    return np.where((e == 15) & ((c & 7) == 7), np.nan, out)


# the 127 finite non-negative magnitudes, in code order (which is increasing)
_MAGS = e4m3_decode(np.arange(127, dtype=np.uint8))


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each fp32 value, ties to the even code.

    Searches the table of finite magnitudes; |v| must not exceed 464, the
    midpoint between 448 and the next (non-finite) step, which rounds to 448.
    """
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    if not np.all(a <= 464.0):
        raise ValueError("value out of the E4M3 range")
    hi = np.clip(np.searchsorted(_MAGS, a, side="left"), 0, 126)  # first magnitude >= a
    lo = np.clip(hi - 1, 0, 126)
    d_hi, d_lo = _MAGS[hi] - a, a - _MAGS[lo]
    pick_lo = (d_lo < d_hi) | ((d_lo == d_hi) & (lo % 2 == 0))
    code = np.where(pick_lo, lo, hi).astype(np.uint8)
    negative = np.signbit(v)
    return np.where(negative, code | np.uint8(0x80), code).astype(np.uint8)


def quantize_blocks(W: np.ndarray, block: int = BLOCK):
    """Block-FP8 form of a stack of weight matrices W [G, K, Ncols] (values
    exactly representable in fp32; K and Ncols multiples of block).

    Returns codes [G, K, Ncols] uint8 (logical layout) and scales
    [G, K/block, Ncols/block] float32.
    """
    W = np.asarray(W)
    G, K, N = W.shape
    if K % block or N % block:
        raise ValueError("K and Ncols must be multiples of the block")
    w32 = W.astype(np.float32)
    if not np.array_equal(w32.astype(np.float64), W.astype(np.float64)):
        raise ValueError("weights must be exact in fp32")
    blocks = w32.reshape(G, K // block, block, N // block, block)
    amax = np.abs(blocks).max(axis=(2, 4))                      # [G, K/b, N/b] fp32
    scales = (amax / np.float32(E4M3_MAX)).astype(np.float32)   # fp32 division
    s = scales[:, :, None, :, None]
    with np.errstate(invalid="ignore", divide="ignore"):
        q = np.where(s > 0, blocks / s, np.float32(0)).astype(np.float32)  # fp32 division
    q = np.clip(q, np.float32(-E4M3_MAX), np.float32(E4M3_MAX))
    codes = e4m3_encode(q).reshape(G, K, N)
    # an all-zero block: zero codes (w / s would be 0 / 0)
    codes = np.where(np.repeat(np.repeat(scales == 0, block, 1), block, 2), np.uint8(0), codes)
    return codes.astype(np.uint8), scales


def dequantize_blocks(codes: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """w' = decode(code) * scale, float64 [G, K, Ncols]."""
    vals = e4m3_decode(codes)
    s = np.repeat(np.repeat(np.asarray(scales, np.float64), block, axis=1), block, axis=2)
    return vals * s
