"""Pins of the second weight codecs (FP8-E4M3 with fp16 group scales,
NVFP4 = E2M1 codes with E4M3 block scales and an fp32 global scale): code
tables against the format definitions and torch's own float8_e4m3fn,
linear layers against hand-worked fixtures, one-hot inputs and brute force."""
import math

import numpy as np
import pytest

import oracle
import synth

# E4M3FN written out from the definition (sign, 4-bit exponent bias 7, 3-bit mantissa)
E4M3_HAND = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x39: 1.125, 0x40: 2.0, 0x7E: 448.0, 0xB8: -1.0, 0xFE: -448.0, 0x30: 0.5}
E2M1_HAND = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e4m3_hand_table_and_nan():
    for b, v in E4M3_HAND.items():
        assert oracle.e4m3_to_f64(np.array([b], np.uint8))[0] == v, hex(b)
    assert np.isnan(oracle.e4m3_to_f64(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_matches_torch_float8():
    import torch
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_f64(b)
    both_nan = np.isnan(ref) & np.isnan(got)
    assert np.array_equal(got[~both_nan], ref[~both_nan]) and both_nan.sum() == 2


def test_e2m1_table():
    got = oracle.e2m1_to_f64(np.arange(16))
    assert got[:8].tolist() == E2M1_HAND
    assert got[8:].tolist() == [-v for v in E2M1_HAND]


def _fp8_w(codes, scales):
    codes = np.asarray(codes, np.uint8)
    return {"codes": codes, "scales": np.asarray(scales, np.float16), "K": codes.shape[1], "N": codes.shape[0]}


def test_fp8_linear_hand_fixture():
    """K = 128 (two groups), N = 2; x = 1 for k < 64 and 2 for k >= 64.
    Output 0: every code 0x38 (1.0), scales 0.5 and 0.25: 64*0.5 + 128*0.25 = 64.
    Output 1: codes 0xC0 (-2.0) then 0x7E (448), scales 1/64 and 1/448:
    64*(-2/64) + 128*(448/448) = -2 + 128 = 126."""
    codes = np.array([[0x38] * 128, [0xC0] * 64 + [0x7E] * 64], np.uint8)
    scales = [[0.5, 0.25], [1 / 64, 1 / 448]]
    W = _fp8_w(codes, scales)
    x = np.array([1.0] * 64 + [2.0] * 64, np.float16)
    y = oracle.linear_fp8(x, W)[0]
    s448 = float(np.float16(1 / 448))
    assert y[0] == 64.0 and abs(y[1] - (-2.0 + 128 * 448 * s448)) < 1e-12


def test_fp8_one_hot_and_bruteforce():
    rng = np.random.default_rng(2)
    W = synth.fp8_matrix(rng, 128, 9)
    X = synth.activations(rng, 2, 128)
    Y = oracle.linear_fp8(X, W)
    for n in range(9):
        for k in (0, 63, 64, 127):
            e = np.zeros(128, np.float16)
            e[k] = 1.0
            want = E4M3_DEF(W["codes"][n, k]) * float(W["scales"][n, k // 64])
            assert oracle.linear_fp8(e, W)[0][n] == want
        for m in range(2):
            ref = math.fsum(float(X[m, k]) * E4M3_DEF(W["codes"][n, k]) * float(W["scales"][n, k // 64])
                            for k in range(128))
            assert abs(Y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def E4M3_DEF(b):
    # Straight from the definition, one code at a time.
    b = int(b)
    s = -1.0 if b & 0x80 else 1.0
    e, m = (b >> 3) & 15, b & 7
    return s * (m / 8 * 2.0 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def _nvfp4_w(nibbles, block, g):
    nib = np.asarray(nibbles, np.int64)
    N, K = nib.shape
    words = np.zeros((N, K // 8), np.uint32)
    for j in range(8):
        words |= (nib[:, j::8] << (4 * j)).astype(np.uint32)
    return {"qweight": words, "block_scales": np.asarray(block, np.uint8),
            "global_scale": np.float32(g), "K": K, "N": N}


def test_nvfp4_block_scales_and_global():
    """K = 32 (two blocks of 16), N = 1: codes 2 (1.0) everywhere, block
    scales 0x38 (1.0) and 0x40 (2.0), global 0.5; x = 1 for k < 16 and 3
    after: 16*1*1*0.5 + 16*3*1*2*0.5 = 8 + 48 = 56.  A one-hot at k = 15 and
    at k = 16 picks the two different block scales."""
    W = _nvfp4_w([[2] * 32], [[0x38, 0x40]], 0.5)
    x = np.array([1.0] * 16 + [3.0] * 16, np.float16)
    assert oracle.linear_nvfp4(x, W)[0][0] == 56.0
    for k, want in ((15, 0.5), (16, 1.0)):
        e = np.zeros(32, np.float16)
        e[k] = 1.0
        assert oracle.linear_nvfp4(e, W)[0][0] == want
    # the sign bit and the largest magnitude: code 15 = -6
    W2 = _nvfp4_w([[15] * 16], [[0x38]], 1.0)
    assert oracle.linear_nvfp4(np.ones(16, np.float16), W2)[0][0] == -96.0


def test_nvfp4_bruteforce():
    rng = np.random.default_rng(4)
    W = synth.nvfp4_matrix(rng, 64, 5)
    X = synth.activations(rng, 2, 64)
    Y = oracle.linear_nvfp4(X, W)
    g = float(W["global_scale"])
    for m in range(2):
        for n in range(5):
            ref = 0.0
            terms = []
            for k in range(64):
                code = int(format(int(W["qweight"][n][k // 8]), "08x")[::-1][k % 8], 16)
                terms.append(float(X[m, k]) * E2M1_HAND[code & 7] * (-1 if code & 8 else 1)
                             * E4M3_DEF(W["block_scales"][n, k // 16]) * g)
            ref = math.fsum(terms)
            assert abs(Y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_codec_shape_checks():
    with pytest.raises(ValueError):
        oracle.dequantize_fp8(np.zeros((1, 96), np.uint8), np.ones((1, 1), np.float16))
    with pytest.raises(ValueError):
        oracle.dequantize_nvfp4(np.zeros((1, 3), np.uint32), np.zeros((1, 1), np.uint8), 1.0, 24)
