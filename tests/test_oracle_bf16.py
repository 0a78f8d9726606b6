"""Pins of the bf16 variant of the oracle: exact bf16 decoding, rounding to
bf16 against torch's own conversion and hand-worked ties, and the linear
layer against a hand-worked fixture, one-hot inputs and brute force."""
import json
import math
import os
import struct

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# bf16 patterns written out by hand (sign | 8-bit exponent | 7-bit mantissa)
HAND = {0x3F80: 1.0, 0xC000: -2.0, 0x3F00: 0.5, 0x3E80: 0.25, 0x3E00: 0.125, 0x3D80: 0.0625,
        0x4000: 2.0, 0xBF80: -1.0, 0x0000: 0.0, 0x4049: 3.140625, 0x0001: 2.0 ** -133,
        0x0080: 2.0 ** -126, 0x7F7F: (2 - 2 ** -7) * 2.0 ** 127, 0x7F80: math.inf, 0xFF80: -math.inf}


def _dec(bits):
    # Independent decoding: the pattern as the upper half of a float32.
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def test_decode_hand_patterns():
    for b, v in HAND.items():
        assert oracle.bf16_to_f64(np.array([b], np.uint16))[0] == v, hex(b)
        assert _dec(b) == v


def test_round_trip_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = oracle.bf16_to_f64(bits)
    keep = ~np.isnan(vals)
    assert np.array_equal(oracle.round_bf16(vals[keep]), bits[keep])
    assert np.all(oracle.round_bf16(vals[~keep]) == 0x7FC0)


def test_round_hand_ties():
    # bf16 spacing at 1 is 2**-7: 1 + 2**-8 is a tie (to the even 1.0),
    # 1 + 3 * 2**-8 a tie to the even 1 + 2**-6.
    assert oracle.round_bf16(1 + 2.0 ** -8) == 0x3F80
    assert oracle.round_bf16(1 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.round_bf16(1 + 2.0 ** -8 + 2.0 ** -30) == 0x3F81  # just above the tie
    assert oracle.round_bf16(-(1 + 2.0 ** -8)) == 0xBF80
    assert oracle.round_bf16((2 - 2 ** -8) * 2.0 ** 127) == 0x7F80   # tie above the largest -> inf
    assert oracle.round_bf16(1.5 * 2.0 ** -133) == 0x0002           # subnormal tie to even
    assert oracle.round_bf16(-0.0) == 0x8000


def test_round_matches_torch_conversion():
    import torch
    rng = np.random.default_rng(12)
    with np.errstate(over="ignore"):  # some draws overflow float32 on purpose (-> inf)
        f = (rng.standard_normal(20000) * np.exp2(rng.integers(-140, 128, 20000))).astype(np.float32)
    ties = (rng.integers(0, 2**32, 4000, dtype=np.uint64).astype(np.uint32) & 0xFFFF0000) | 0x8000
    f = np.concatenate([f, ties.view(np.float32)[np.isfinite(ties.view(np.float32))],
                        np.array([3.4e38, -3.4e38, 1e-39, -1e-40, 0.0], np.float32)])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16(f.astype(np.float64)), ref)


def _hand_w(codes, scales_bits, biases_bits, K):
    N, G = len(codes), K // 64
    qw = np.zeros((N, K // 8), np.uint32)
    for n in range(N):
        for g in range(G):
            qw[n, g * 8:(g + 1) * 8] = codes[n][g] * 0x11111111
    return {"qweight": qw, "scales": np.array(scales_bits, np.uint16),
            "biases": np.array(biases_bits, np.uint16), "K": K, "N": N}


def test_linear_hand_fixture():
    """The hand-worked two-group GEMV of gemv_hand.json with its scales,
    biases and activations written as bf16 patterns (all exact in bf16)."""
    f = json.load(open(os.path.join(GOLDEN, "gemv_hand.json")))
    enc = {v: b for b, v in HAND.items() if math.isfinite(v)}
    sb = [[enc[v] for v in row] for row in f["scales"]]
    bb = [[enc[v] for v in row] for row in f["biases"]]
    W = _hand_w(f["codes"], sb, bb, f["K"])
    x = np.array([enc[f["x_low"]]] * 64 + [enc[f["x_high"]]] * 64, np.uint16)
    assert np.array_equal(oracle.linear_bf16(x[None, :], W)[0], np.array(f["y"]))


def test_one_hot_and_bruteforce():
    rng = np.random.default_rng(3)
    K, N = 128, 7
    W = synth.w4_matrix_bf16(rng, K, N)
    X = synth.bf16_bits(rng.standard_normal((3, K)))

    def w_digit(n, k):
        code = int(format(int(W["qweight"][n][k // 8]), "08x")[::-1][k % 8], 16)
        return _dec(W["scales"][n][k // 64]) * code + _dec(W["biases"][n][k // 64])

    for k in (0, 63, 64, 127):
        e = np.zeros((1, K), np.uint16)
        e[0, k] = 0x3F80
        col = oracle.linear_bf16(e, W)[0]
        assert np.array_equal(col, np.array([w_digit(n, k) for n in range(N)]))
    Y = oracle.linear_bf16(X, W)
    for m in range(3):
        for n in range(N):
            ref = math.fsum(_dec(X[m, k]) * w_digit(n, k) for k in range(K))
            assert abs(Y[m, n] - ref) <= 1e-12 * max(1.0, abs(ref))


def _tiny_bf16(seed, T=5, D=64, I=64, E=6):
    w = synth.moe_weights_bf16(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens_bf16(seed + 100, T, D=D, E=E, skewed=True)
    return w, tok


def _ffn_one_token_bf16(h_bits, gu, dn):
    """One expert on one token, written from the definitions with a plain
    loop over outputs (no matrix routine)."""
    h = oracle.bf16_to_f64(h_bits)
    Wgu = oracle.dequantize_bf16(gu["qweight"], gu["scales"], gu["biases"], gu["K"])
    I = gu["N"] // 2
    u = np.array([math.fsum(h * Wgu[n]) for n in range(2 * I)])
    act = oracle.round_bf16(u[:I] / (1.0 + np.exp(-u[:I])) * u[I:])
    Wdn = oracle.dequantize_bf16(dn["qweight"], dn["scales"], dn["biases"], dn["K"])
    a = oracle.bf16_to_f64(act)
    return np.array([math.fsum(a * Wdn[n]) for n in range(dn["N"])])


def test_moe_layer_bf16_matches_per_token_bruteforce():
    """Token by token: logits from the decoded bf16 inputs, the k best by a
    sort, each chosen expert on that token alone, weighted, plus the shared
    expert.  No histogram, scan or permutation."""
    for seed, topk in [(0, 2), (1, 3), (2, 6)]:
        w, tok = _tiny_bf16(seed)
        res = oracle.moe_layer_bf16(tok["H"], w, tok["logit_bias"], topk=topk)
        H = oracle.bf16_to_f64(tok["H"])
        Wr = oracle.bf16_to_f64(w["Wr"])
        for t in range(H.shape[0]):
            L = np.array([math.fsum(H[t] * Wr[:, e]) for e in range(Wr.shape[1])])
            L = L + tok["logit_bias"].astype(np.float64)
            chosen = sorted(range(len(L)), key=lambda e: (-L[e], e))[:topk]
            g = np.exp(L[chosen] - L[chosen].max())
            g = g / g.sum()
            assert res["ids"][t].tolist() == chosen
            assert np.allclose(res["gates"][t], g, rtol=1e-12, atol=1e-15)
            ref = _ffn_one_token_bf16(tok["H"][t], w["shared_gate_up"], w["shared_down"])
            for gj, e in zip(g, chosen):
                one = lambda W: {k: (v[e] if isinstance(v, np.ndarray) else v) for k, v in W.items()}
                ref = ref + gj * _ffn_one_token_bf16(tok["H"][t], one(w["gate_up"]), one(w["down"]))
            assert np.allclose(res["out"][t], ref, rtol=1e-9, atol=1e-9)


def test_moe_layer_bf16_without_shared_and_identical_experts():
    """Every routed expert equal to the shared one: with the shared expert
    the output is twice one FFN, without it once (the gates sum to 1)."""
    E = 5
    w, tok = _tiny_bf16(3, T=4, E=E)
    for key, skey in (("gate_up", "shared_gate_up"), ("down", "shared_down")):
        for f in ("qweight", "scales", "biases"):
            w[key][f] = np.repeat(w[skey][f][None], E, axis=0)
    both = oracle.moe_layer_bf16(tok["H"], w, tok["logit_bias"], topk=3)
    routed = oracle.moe_layer_bf16(tok["H"], w, tok["logit_bias"], topk=3, with_shared=False)
    for t in range(4):
        one = _ffn_one_token_bf16(tok["H"][t], w["shared_gate_up"], w["shared_down"])
        assert np.allclose(both["out"][t], 2 * one, rtol=1e-9, atol=1e-9)
        assert np.allclose(routed["out"][t], one, rtol=1e-9, atol=1e-9)
