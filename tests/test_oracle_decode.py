"""Pins of the oracle's decode steps (RMSNorm in front of a projection, the
token choice after the vocabulary head, the embedding row of a token)
against hand-worked fixtures, closed forms, invariants and brute force."""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _fx():
    with open(os.path.join(GOLDEN, "decode_hand.json")) as f:
        return json.load(f)


def _w4(words_per_output, scales, biases, K):
    """w4 dict from one repeated 32-bit word per output and one scale and
    bias per output (a single group when K = 64)."""
    N = len(words_per_output)
    qw = np.array([[w] * (K // 8) for w in words_per_output], dtype=np.uint32)
    G = K // 64
    sc = np.array([[s] * G for s in scales], dtype=np.float16)
    bi = np.array([[b] * G for b in biases], dtype=np.float16)
    return {"qweight": qw, "scales": sc, "biases": bi, "K": K, "N": N}


def _nibble(word, j):
    # Independent of the oracle's unpacking: the j-th hex digit from the right.
    return int(format(int(word), "08x")[::-1][j], 16)


def _dequant_by_hex(W, n):
    """Row n of the dequantized matrix, decoded digit by digit in Python."""
    K = W["K"]
    out = []
    for k in range(K):
        code = _nibble(W["qweight"][n][k // 8], k % 8)
        s = float(W["scales"][n][k // 64])
        b = float(W["biases"][n][k // 64])
        out.append(s * code + b)
    return out


def test_rms_norm_hand_fixture():
    for c in _fx()["rms_norm"]:
        u = oracle.rms_norm(np.array(c["x"]), np.array(c["gamma"]), c["eps"])
        if "u" in c:
            assert np.allclose(u, c["u"], rtol=0, atol=1e-15), c["why"]
        else:
            assert np.allclose(u / math.sqrt(2.0), c["u_over_sqrt2"], rtol=1e-15), c["why"]


def test_rms_norm_invariants():
    rng = np.random.default_rng(4)
    x = rng.normal(0, 3, 2048)
    ones = np.ones_like(x)
    u = oracle.rms_norm(x, ones, 0.0)
    assert abs(np.mean(u * u) - 1.0) < 1e-12                      # unit RMS
    for a in (1e-3, 7.5):                                          # scale invariance
        assert np.allclose(oracle.rms_norm(a * x, ones, 0.0), u, rtol=1e-12)
    assert np.allclose(oracle.rms_norm(-x, ones, 0.0), -u, rtol=1e-12)
    g1, g2 = rng.normal(size=x.size), rng.normal(size=x.size)     # linear in gamma
    assert np.allclose(oracle.rms_norm(x, g1 + g2, 1e-6),
                       oracle.rms_norm(x, g1, 1e-6) + oracle.rms_norm(x, g2, 1e-6), rtol=1e-10, atol=1e-12)
    # eps sits inside the root next to the mean: for x = c everywhere,
    # u = c / sqrt(c^2 + eps)
    for c, eps in ((2.0, 5.0), (0.5, 0.75)):
        assert np.allclose(oracle.rms_norm(np.full(64, c), np.ones(64), eps), c / math.sqrt(c * c + eps))


def test_gemv_rmsnorm_hand_fixture():
    f = _fx()["gemv_rmsnorm"]
    K = f["K"]
    x = np.array([f["x_even"] if k % 2 == 0 else f["x_odd"] for k in range(K)], dtype=np.float16)
    gamma = np.full(K, f["gamma"], dtype=np.float16)
    W = _w4([int(w, 16) for w in f["words"]], f["scales"], f["biases"], K)
    y, u = oracle.gemv_rmsnorm(x, gamma, f["eps"], W)
    assert u.dtype == np.float16
    assert np.array_equal(u[0::2].astype(np.float64), np.full(K // 2, f["u_even"]))
    assert np.array_equal(u[1::2].astype(np.float64), np.full(K // 2, f["u_odd"]))
    assert np.array_equal(y, np.array(f["y"]))


def test_gemv_rmsnorm_rounds_the_normalized_row_once():
    """The projection reads the fp16-rounded normalized row: with a single
    output whose weights are all 1, y is the exact sum of the fp16 values."""
    rng = np.random.default_rng(9)
    K = 128
    x = rng.normal(0, 1, K).astype(np.float16)
    gamma = rng.uniform(0.5, 1.5, K).astype(np.float16)
    W = _w4([0x11111111], [1.0], [0.0], K)
    y, u = oracle.gemv_rmsnorm(x, gamma, 1e-6, W)
    exact = oracle.rms_norm(x, gamma, 1e-6)
    assert math.fsum(float(v) for v in u) == y[0]
    assert math.fsum(exact) != y[0]                                 # rounding is visible here
    assert np.max(np.abs(u.astype(np.float64) - exact)) <= np.max(np.abs(exact)) * 2.0 ** -11


def _argmax_loop(v):
    best, idx = v[0], 0
    for i in range(1, len(v)):
        if v[i] > best:
            best, idx = v[i], i
    return idx


def test_argmax_hand_and_bruteforce():
    for c in _fx()["argmax"]:
        assert oracle.argmax_first(c["v"]) == c["token"]
    rng = np.random.default_rng(2)
    for _ in range(300):
        n = int(rng.integers(1, 40))
        v = rng.integers(-3, 4, n).astype(np.float64)                 # many ties
        assert oracle.argmax_first(v) == _argmax_loop(list(v))


def test_lm_head_hand_fixture():
    f = _fx()["lm_head"]
    W = _w4([c * 0x11111111 for c in f["codes"]], f["scales"], f["biases"], f["K"])
    tok, logits = oracle.lm_head_token(np.full(f["K"], f["x"], dtype=np.float16), W)
    assert np.array_equal(logits, np.array(f["logits"]))
    assert tok == f["token"]


def test_lm_head_one_hot_selects_a_weight_column():
    """x = e_k turns the logits into weight k of every output; the token is
    the output with the largest such weight (decoded digit by digit)."""
    rng = np.random.default_rng(5)
    K, N = 128, 37
    W = synth.w4_matrix(rng, K, N)
    for k in (0, 63, 64, 127):
        x = np.zeros(K, dtype=np.float16)
        x[k] = 1.0
        tok, logits = oracle.lm_head_token(x, W)
        col = [_dequant_by_hex(W, n)[k] for n in range(N)]
        assert np.array_equal(logits, np.array(col))
        assert tok == _argmax_loop(col)


def test_embed_hand_fixture():
    f = _fx()["embed"]
    W = _w4([0, 0], f["scales"], f["biases"], f["K"])
    W["qweight"][1, 0::2] = 0x76543210
    W["qweight"][1, 1::2] = 0xFEDCBA98
    r0 = oracle.embed_row(W, 0)
    r1 = oracle.embed_row(W, 1)
    assert r0.dtype == np.float16 and r1.dtype == np.float16
    assert np.array_equal(r0.astype(np.float64), np.full(f["K"], f["row0"]))
    assert np.array_equal(r1[:16].astype(np.float64), np.array(f["row1_first16"]))
    assert np.array_equal(r1[16:32], r1[:16])
    with pytest.raises(IndexError):
        oracle.embed_row(W, 2)
    with pytest.raises(IndexError):
        oracle.embed_row(W, -1)


def test_embed_matches_digit_decode():
    rng = np.random.default_rng(6)
    E = synth.w4_matrix(rng, 192, 11)
    for tok in (0, 5, 10):
        ref = np.array(_dequant_by_hex(E, tok)).astype(np.float16)
        assert np.array_equal(oracle.embed_row(E, tok).view(np.uint16), ref.view(np.uint16))
