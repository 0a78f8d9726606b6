"""Pins of the oracle's w4 format and linear layer against facts fixed
outside the oracle: hand-worked fixtures, closed forms, exact rational
arithmetic, brute force and integer special cases."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _nibble_via_hex(word: int, j: int) -> int:
    # Independent extraction: the j-th hex digit counted from the right.
    return int(format(int(word), "08x")[::-1][j], 16)


def test_pack_words_hand():
    for case in _load("pack_words.json")["cases"]:
        word = int(case["word"], 16)
        codes = np.array([case["codes"]])
        assert int(oracle.pack_codes(codes)[0, 0]) == word
        assert oracle.unpack_codes(np.array([[word]], dtype=np.uint32), 8)[0].tolist() == case["codes"]


def test_pack_unpack_roundtrip_random():
    rng = np.random.default_rng(7)
    words = rng.integers(0, 2**32, size=(5, 33), dtype=np.uint64).astype(np.uint32)
    codes = oracle.unpack_codes(words, 33 * 8)
    assert codes.min() >= 0 and codes.max() <= 15
    assert np.array_equal(oracle.pack_codes(codes), words)
    # Each code agrees with the hex digit of its word.
    for n in range(5):
        for k in range(0, 33 * 8, 7):
            assert codes[n, k] == _nibble_via_hex(words[n, k // 8], k % 8)


def test_pack_rejects_bad_codes():
    with pytest.raises(ValueError):
        oracle.pack_codes(np.array([[16, 0, 0, 0, 0, 0, 0, 0]]))
    with pytest.raises(ValueError):
        oracle.pack_codes(np.zeros((1, 12), dtype=np.int64))


def test_dequantize_exact_rational():
    rng = np.random.default_rng(3)
    K, N = 192, 5
    W = synth.w4_matrix(rng, K, N)
    Wd = oracle.dequantize(W["qweight"], W["scales"], W["biases"], K)
    for n in range(N):
        for k in range(K):
            q = _nibble_via_hex(W["qweight"][n, k // 8], k % 8)
            s = Fraction(float(W["scales"][n, k // 64]))
            b = Fraction(float(W["biases"][n, k // 64]))
            assert Fraction(float(Wd[n, k])) == s * q + b


def test_dequantize_rejects_ragged_group():
    with pytest.raises(ValueError):
        oracle.dequantize(np.zeros((1, 12), np.uint32), np.zeros((1, 2), np.float16),
                          np.zeros((1, 2), np.float16), 96)


def _hand_matrix(case):
    codes = np.array(case["codes"], dtype=np.int64)  # [N][G]
    N, G = codes.shape
    K = case["K"]
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for n in range(N):
        for g in range(G):
            words[n, g * 8:(g + 1) * 8] = codes[n, g] * 0x11111111
    return {"qweight": words, "scales": np.array(case["scales"], dtype=np.float16),
            "biases": np.array(case["biases"], dtype=np.float16), "K": K, "N": N}


def test_gemv_hand_fixture():
    case = _load("gemv_hand.json")
    W = _hand_matrix(case)
    x = np.array([case["x_low"]] * 64 + [case["x_high"]] * 64, dtype=np.float16)
    y = oracle.linear(x, W)
    assert y.tolist() == [case["y"]]


def test_one_hot_picks_single_weight():
    """x = e_k gives y[n] = W[k][n]: pins orientation (no transposition) and
    the group index k // 64, with K != N."""
    rng = np.random.default_rng(11)
    K, N = 256, 40
    W = synth.w4_matrix(rng, K, N)
    for k in (0, 7, 8, 63, 64, 130, 255):
        x = np.zeros(K, dtype=np.float16)
        x[k] = 1
        y = oracle.linear(x, W)[0]
        for n in (0, 1, 17, 39):
            q = _nibble_via_hex(W["qweight"][n, k // 8], k % 8)
            expect = float(W["scales"][n, k // 64]) * q + float(W["biases"][n, k // 64])
            assert y[n] == expect


def test_affine_identity_all_equal_codes():
    """All codes of group g equal c_g => y[n] = sum_g (s*c + b) * sum_{k in g} x_k."""
    rng = np.random.default_rng(5)
    K, N = 512, 24
    G = K // 64
    c = rng.integers(0, 16, size=(N, G))
    W = synth.w4_matrix(rng, K, N)
    W["qweight"] = np.repeat((c * 0x11111111).astype(np.uint32), 8, axis=1)
    x = synth.activations(rng, 1, K)[0]
    y = oracle.linear(x, W)[0]
    xs = x.astype(np.float64)
    for n in range(N):
        terms = []
        for g in range(G):
            w = float(W["scales"][n, g]) * int(c[n, g]) + float(W["biases"][n, g])
            terms.append(w * math.fsum(xs[g * 64:(g + 1) * 64]))
        ref = math.fsum(terms)
        assert abs(y[n] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_zero_case_code8():
    """Code 8 everywhere, bias = -8 * scale with power-of-two scales: W = 0
    exactly, so y = 0 exactly."""
    rng = np.random.default_rng(1)
    K, N = 256, 16
    scales = (2.0 ** -rng.integers(1, 9, size=(N, K // 64))).astype(np.float16)
    W = {"qweight": np.full((N, K // 8), 0x88888888, dtype=np.uint32), "scales": scales,
         "biases": (-8 * scales.astype(np.float64)).astype(np.float16), "K": K, "N": N}
    x = synth.activations(rng, 3, K)
    assert np.all(oracle.linear(x, W) == 0.0)


def test_integer_special_case_exact():
    """scale = 1, bias = 0, small integer x: y = x @ Q, an integer matmul done
    here with Python integers."""
    rng = np.random.default_rng(2)
    K, N, M = 128, 20, 3
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    W = {"qweight": words, "scales": np.ones((N, K // 64), np.float16),
         "biases": np.zeros((N, K // 64), np.float16), "K": K, "N": N}
    X = rng.integers(-4, 5, size=(M, K))
    y = oracle.linear(X.astype(np.float16), W)
    for m in range(M):
        for n in range(N):
            ref = sum(int(X[m, k]) * _nibble_via_hex(words[n, k // 8], k % 8) for k in range(K))
            assert y[m, n] == ref


def test_bruteforce_fsum_small():
    """K, N <= 128: every product x*w is exact in float64 (an fp16 times a
    value of at most 27 significant bits), so math.fsum gives the correctly
    rounded sum; the oracle's matmul must agree to 1e-15 of sum |x*w|."""
    for seed, (M, K, N) in enumerate([(1, 64, 64), (2, 128, 96), (3, 128, 128)]):
        case = synth.gemm_case(seed, M, K, N)
        X, W = case["X"], case["W"]
        y = oracle.linear(X, W)
        for m in range(M):
            for n in range(N):
                prods = []
                for k in range(K):
                    q = _nibble_via_hex(W["qweight"][n, k // 8], k % 8)
                    w = float(W["scales"][n, k // 64]) * q + float(W["biases"][n, k // 64])
                    prods.append(float(X[m, k]) * w)
                ref = math.fsum(prods)
                bound = 1e-15 * math.fsum(abs(p) for p in prods)
                assert abs(y[m, n] - ref) <= bound


def test_bias_factorisation_identity():
    """sum_k x_k (s q_k + b) = sum_g [ s_g * (x_g . q_g) + b_g * sum(x_g) ]."""
    case = synth.gemv_case(4, 1024, 64)
    x, W = case["x"][0].astype(np.float64), case["W"]
    q = np.zeros((64, 1024))
    for n in range(64):
        for k in range(1024):
            q[n, k] = _nibble_via_hex(W["qweight"][n, k // 8], k % 8)
    y = oracle.linear(case["x"], W)[0]
    for n in range(64):
        acc = 0.0
        for g in range(1024 // 64):
            sl = slice(g * 64, (g + 1) * 64)
            acc += float(W["scales"][n, g]) * float(x[sl] @ q[n, sl]) + float(W["biases"][n, g]) * float(x[sl].sum())
        assert abs(acc - y[n]) <= 1e-12 * max(1.0, abs(y[n]))


def test_linear_chunking_invariant():
    case = synth.gemm_case(9, 4, 256, 300)
    a = oracle.linear(case["X"], case["W"], row_chunk=7)
    b = oracle.linear(case["X"], case["W"], row_chunk=4096)
    assert np.array_equal(a, b)


def test_round_f16_ties_to_even():
    one = 1.0
    assert float(oracle.round_f16(one + 2.0**-11)) == 1.0             # tie -> even
    assert float(oracle.round_f16(one + 3 * 2.0**-11)) == 1.0 + 2.0**-9  # tie -> even
    assert float(oracle.round_f16(one + 2.0**-11 + 2.0**-20)) == 1.0 + 2.0**-10
    assert float(oracle.round_f16(65520.0)) == float("inf")
    assert float(oracle.round_f16(65519.0)) == 65504.0
