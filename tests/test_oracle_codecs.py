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


# E4M3 codes of the integers 0..8 (sign bit 0x80 gives -0..-8).
_E4M3_INT = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50], np.uint8)


def _w4_as_fp8(W):
    """A w4 matrix (stack) whose biases are -8 * scale, rewritten as FP8: the
    weight s*q - 8s is e4m3(q - 8) * s, both exact in float64."""
    q = oracle.unpack_codes(W["qweight"], W["K"]).astype(np.int64) - 8
    codes = _E4M3_INT[np.abs(q)] | np.where(q < 0, 0x80, 0).astype(np.uint8)
    return {"codes": codes.astype(np.uint8), "scales": W["scales"], "K": W["K"], "N": W["N"]}


def _w4_centered(W):
    W = dict(W)
    W["biases"] = (W["scales"].astype(np.float64) * -8.0).astype(np.float16)
    return W


@pytest.mark.parametrize("shared", [True, False])
def test_moe_fp8_equals_w4_layer_on_common_weights(shared):
    """Weights that both formats hold exactly (w4 with bias = -8 * scale, the
    FP8 codes of q - 8 with the same scales): the FP8 layer must reproduce the
    separately pinned w4 layer exactly, routing, every row and the output."""
    import synth
    w = synth.moe_weights(11, D=128, I=64, E=8)
    w4 = {k: (_w4_centered(v) if isinstance(v, dict) else v) for k, v in w.items()}
    f8 = {k: (_w4_as_fp8(v) if isinstance(v, dict) else v) for k, v in w4.items()}
    H = synth.activations(synth.rng_for(12), 37, 128)
    a = oracle.moe_layer(H, w4, None, 3, with_shared=shared)
    b = oracle.moe_layer_fp8(H, f8, None, 3, with_shared=shared)
    for key in ("ids", "counts", "offsets", "sorted_assign", "pos"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["act"].view(np.uint16), b["act"].view(np.uint16))
    assert np.array_equal(a["ydown"], b["ydown"]) and np.array_equal(a["out"], b["out"])


def test_moe_fp8_token_loop_bruteforce():
    """Token by token, in token order (no sorting or permutation): out[t] =
    sum_j gate[t][j] * down_e(fp16(SiLU(gate_e(h)) * up_e(h))) + the shared
    expert's, with e = ids[t][j] and every dot product a math.fsum."""
    import math
    import synth
    T, D, I, E, topk = 4, 64, 64, 6, 2
    w = synth.moe_weights_fp8(13, D=D, I=I, E=E)
    H = synth.activations(synth.rng_for(14), T, D)
    ref = oracle.moe_layer_fp8(H, w, None, topk)

    def ffn(h, gu_codes, gu_scales, dn_codes, dn_scales):
        Wg = oracle.dequantize_fp8(gu_codes, gu_scales)     # [2I][D]
        Wd = oracle.dequantize_fp8(dn_codes, dn_scales)     # [D][I]
        hv = [float(v) for v in h]
        u = [math.fsum(hv[k] * Wg[n][k] for k in range(D)) for n in range(2 * I)]
        act = [float(np.float16(u[i] / (1.0 + math.exp(-u[i])) * u[I + i])) for i in range(I)]
        return [math.fsum(act[i] * Wd[n][i] for i in range(I)) for n in range(D)]

    for tok in range(T):
        acc = [0.0] * D
        for j in range(topk):
            e = int(ref["ids"][tok][j])
            y = ffn(H[tok], w["gate_up"]["codes"][e], w["gate_up"]["scales"][e],
                    w["down"]["codes"][e], w["down"]["scales"][e])
            acc = [a + float(ref["gates"][tok][j]) * v for a, v in zip(acc, y)]
        ys = ffn(H[tok], w["shared_gate_up"]["codes"], w["shared_gate_up"]["scales"],
                 w["shared_down"]["codes"], w["shared_down"]["scales"])
        acc = [a + v for a, v in zip(acc, ys)]
        np.testing.assert_allclose(ref["out"][tok], acc, rtol=1e-9, atol=1e-9)


# E4M3 codes of the eight E2M1 magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
_E4M3_OF_E2M1 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], np.uint8)


def _nvfp4_as_fp8(W, K):
    """An NVFP4 matrix (stack) whose block scales are equal within each 64
    along K and whose e4m3(block) * global is an fp16 value, rewritten as
    FP8: e2m1(code) is an E4M3 value, the scale the same fp16 number."""
    q = oracle.unpack_codes(W["qweight"], K).astype(np.int64)
    codes = _E4M3_OF_E2M1[q & 7] | np.where(q & 8, 0x80, 0).astype(np.uint8)
    g = np.asarray(W["global_scale"], np.float64)[..., None, None]
    s = oracle.e4m3_to_f64(W["block_scales"][..., ::4]) * g
    assert np.array_equal(s, s.astype(np.float16).astype(np.float64))
    return {"codes": codes.astype(np.uint8), "scales": s.astype(np.float16), "K": K, "N": W["N"]}


@pytest.mark.parametrize("shared", [True, False])
def test_moe_nvfp4_equals_fp8_layer_on_common_weights(shared):
    """NVFP4 weights that the FP8 format holds exactly (block scales constant
    over each 64, global scales powers of two): the NVFP4 layer must
    reproduce the FP8 layer, itself pinned to the w4 layer, exactly."""
    import synth
    w = synth.moe_weights_nvfp4(15, D=128, I=64, E=8)
    for key in ("gate_up", "down", "shared_gate_up", "shared_down"):
        W = w[key]
        W["block_scales"] = np.repeat(W["block_scales"][..., ::4], 4, axis=-1)
        W["global_scale"] = (np.float32(2.0 ** -7) if np.ndim(W["global_scale"]) == 0 else
                             np.exp2(-np.arange(W["global_scale"].size) % 3 - 6).astype(np.float32))
    f8 = {k: (_nvfp4_as_fp8(v, v["K"]) if isinstance(v, dict) else v) for k, v in w.items()}
    H = synth.activations(synth.rng_for(16), 29, 128)
    a = oracle.moe_layer_nvfp4(H, w, None, 3, with_shared=shared)
    b = oracle.moe_layer_fp8(H, f8, None, 3, with_shared=shared)
    for key in ("ids", "counts", "offsets", "sorted_assign", "pos"):
        assert np.array_equal(a[key], b[key]), key
    assert np.array_equal(a["act"].view(np.uint16), b["act"].view(np.uint16))
    assert np.array_equal(a["ydown"], b["ydown"]) and np.array_equal(a["out"], b["out"])


def test_moe_nvfp4_per_expert_global_scale():
    """Each expert's global scale multiplies only its own rows: doubling the
    down projection's global scale of one expert doubles exactly the ydown
    rows routed to that expert and leaves every other row unchanged."""
    import synth
    w = synth.moe_weights_nvfp4(17, D=128, I=64, E=8)
    H = synth.activations(synth.rng_for(18), 40, 128)
    a = oracle.moe_layer_nvfp4(H, w, None, 2)
    e = int(np.argmax(a["counts"]))
    w["down"]["global_scale"] = w["down"]["global_scale"].copy()
    w["down"]["global_scale"][e] *= 2
    b = oracle.moe_layer_nvfp4(H, w, None, 2)
    r0, r1 = int(a["offsets"][e]), int(a["offsets"][e + 1])
    assert r1 > r0
    assert np.array_equal(b["ydown"][r0:r1], 2 * a["ydown"][r0:r1])
    mask = np.ones(a["ydown"].shape[0], bool)
    mask[r0:r1] = False
    assert np.array_equal(b["ydown"][mask], a["ydown"][mask])
