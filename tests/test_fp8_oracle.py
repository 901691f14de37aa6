"""Pins of the oracle's block-FP8 quantiser (CPU).

The E4M3 decoder is checked against the textbook values of the format and
against torch's float8_e4m3fn view of every code; the encoder against
torch's float32 -> float8_e4m3fn cast (round to nearest, ties to even) on
random values, on every midpoint between neighbouring codes and on signed
zeros; the block quantiser against properties its definition fixes.
"""
import numpy as np
import pytest
import torch

from oracle import fp8_oracle as F


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)


def torch_encode(v):
    return torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_textbook_values():
    got = F.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x3C, 0x7E, 0x80, 0xFE, 0xB8], np.uint8))
    want = [0.0, 2.0 ** -9, 7 * 2.0 ** -9, 2.0 ** -6, 1.0, 1.5, 448.0, -0.0, -448.0, -1.0]
    assert got.tolist() == want
    assert np.signbit(got[7])
    assert np.isnan(F.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    a, b = F.e4m3_decode(codes), torch_decode(codes)
    assert np.array_equal(np.isnan(a), np.isnan(b))
    ok = ~np.isnan(a)
    assert np.array_equal(a[ok], b[ok]) and np.array_equal(np.signbit(a[ok]), np.signbit(b[ok]))


def test_encode_matches_torch_random_and_ties():
    rng = np.random.default_rng(3)
    mags = np.exp2(rng.uniform(-14, np.log2(448.0), 20000)).astype(np.float32)
    v = np.where(rng.random(mags.size) < 0.5, -mags, mags).astype(np.float32)
    # every midpoint between neighbouring finite codes (exact in fp32), both signs
    t = F.e4m3_decode(np.arange(127, dtype=np.uint8))
    mids = ((t[:-1] + t[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (t[:-1] + t[1:]) / 2)
    extra = np.array([0.0, -0.0, 448.0, -448.0, 464.0, 1e-12, -1e-12, 2.0 ** -10, -(2.0 ** -10)], np.float32)
    for vals in (v, mids, -mids, extra):
        assert np.array_equal(F.e4m3_encode(vals), torch_encode(vals))


def test_encode_rejects_out_of_range():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([465.0], np.float32))


def test_block_quantiser_properties():
    rng = np.random.default_rng(5)
    G, K, N = 2, 256, 384
    W = (rng.standard_normal((G, K, N)) * np.exp2(rng.uniform(-8, 4, (G, 1, N)))).astype(np.float32)
    W[1, 128:256, 0:128] = 0.0                   # an all-zero block
    W[0, 5, 7] = -0.0
    codes, scales = F.quantize_blocks(W)
    assert codes.shape == (G, K, N) and scales.shape == (G, 2, 3) and scales.dtype == np.float32
    # the scale is amax / 448 in fp32, and the block's largest element maps to 448 exactly
    for g in range(G):
        for i in range(2):
            for j in range(3):
                blk = W[g, 128 * i:128 * (i + 1), 128 * j:128 * (j + 1)]
                amax = np.float32(np.abs(blk).max())
                assert scales[g, i, j] == np.float32(amax / np.float32(448.0))
                if amax > 0:
                    r, c = np.unravel_index(np.abs(blk).argmax(), blk.shape)
                    assert codes[g, 128 * i + r, 128 * j + c] & 0x7F == 0x7E
    # the zero block: scale 0, codes 0; negative zero keeps its sign
    assert scales[1, 1, 0] == 0 and not codes[1, 128:256, 0:128].any()
    assert codes[0, 5, 7] == 0x80
    # no NaN codes; dequantised values within half a step of the weights
    assert not np.isin(codes & 0x7F, [0x7F]).any()
    Wq = F.dequantize_blocks(codes, scales)
    s = np.repeat(np.repeat(scales.astype(np.float64), 128, 1), 128, 2)
    x = np.abs(W.astype(np.float64))
    normal = x >= 2.0 ** -6 * s
    err = np.abs(Wq - W.astype(np.float64))
    assert np.all(err[normal] <= x[normal] * 2.0 ** -4 * (1 + 1e-6))  # half of 2^-3 relative spacing
    assert np.all(err[~normal] <= s[~normal] * 2.0 ** -10 * (1 + 1e-6))  # half of the subnormal step
    # each block is quantised on its own: one block alone gives the same codes
    c1, s1 = F.quantize_blocks(W[:1, 128:256, 256:384])
    assert np.array_equal(c1[0], codes[0, 128:256, 256:384]) and s1[0, 0, 0] == scales[0, 1, 2]


def test_quantiser_saturates_with_a_subnormal_scale():
    """amax / 448 below fp32's normal range rounds coarsely: w / s may pass 448 and saturates there."""
    W = np.zeros((1, 128, 128), np.float32)
    # multiples of the smallest fp32 subnormal, up to 667: s = 667/448 * 2^-149 rounds to 2^-149
    W[0, 0, :] = (np.linspace(1, 667, 128).round() * 2.0 ** -149).astype(np.float32)
    codes, scales = F.quantize_blocks(W)
    s = scales[0, 0, 0]
    assert 0 < s < np.finfo(np.float32).tiny
    q = (W[0, 0] / s).astype(np.float32)
    assert np.abs(q).max() > 464  # the plain quotient leaves the E4M3 range
    assert (codes[0, 0] & 0x7F).max() == 0x7E and not np.isin(codes, [0x7F, 0xFF]).any()


def test_quantiser_brute_force_tiny():
    """Each code is the nearest finite E4M3 value to w / s (brute force over all codes)."""
    rng = np.random.default_rng(9)
    W = rng.standard_normal((1, 128, 128)).astype(np.float32)
    codes, scales = F.quantize_blocks(W)
    q = (W[0] / scales[0, 0, 0]).astype(np.float32).astype(np.float64).ravel()[:2000]
    table = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    finite = np.nonzero(~np.isnan(table))[0]
    best = np.abs(table[finite][None, :] - q[:, None]).min(axis=1)
    got = F.e4m3_decode(codes[0].ravel()[:2000])
    assert np.array_equal(np.abs(got - q), best)
