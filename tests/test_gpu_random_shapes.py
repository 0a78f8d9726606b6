"""Seeded random shapes across the entry points (a fixed list drawn once
from a seeded generator, so every run checks the same cases): ragged M, N
and K over each path's supported range, against the oracle at the parity
bars.  Complements the hand-picked shapes of the other GPU tests."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, assert_close_bf16, host, say, t, w4_dev

pytestmark = pytest.mark.gpu

_R = np.random.default_rng(20261202)
GEMM_SHAPES = [(int(_R.integers(1, 3000)), int(64 * _R.integers(1, 48)), int(_R.integers(1, 3000)))
               for _ in range(12)]
GEMV_SHAPES = [(int(64 * _R.integers(1, 80)), int(_R.integers(1, 20000))) for _ in range(10)]
MOE_SHAPES = [(int(_R.integers(1, 600)), int(64 * 2 ** _R.integers(1, 5)), int(64 * 2 ** _R.integers(0, 4)),
               int(_R.integers(2, 80)), int(_R.integers(1, 9))) for _ in range(8)]


@pytest.mark.parametrize("i", range(len(GEMM_SHAPES)))
def test_random_gemm(i):
    import torch
    M, K, N = GEMM_SHAPES[i]
    say(f"random gemm M={M} K={K} N={N}")
    c = synth.gemm_case(100 + i, M, K, N)
    ref = oracle.linear(c["X"], c["W"])
    Y = ql.qlinear_gemm(w4_dev(c["W"]), t(c["X"]))
    torch.cuda.synchronize()
    assert_close(host(Y).astype(np.float64), ref, f"gemm M={M} K={K} N={N}")
    if K % 64 == 0 and K <= 8192:
        rng = synth.rng_for(200 + i)
        W8 = synth.fp8_matrix(rng, K, N)
        Y8 = ql.qlinear_gemm_fp8({"codes": t(W8["codes"]), "scales": t(W8["scales"]), "K": K, "N": N}, t(c["X"]))
        torch.cuda.synchronize()
        assert_close(host(Y8).astype(np.float64), oracle.linear_fp8(c["X"], W8), "gemm_fp8")


@pytest.mark.parametrize("i", range(len(GEMV_SHAPES)))
def test_random_gemv(i):
    import torch
    K, N = GEMV_SHAPES[i]
    say(f"random gemv K={K} N={N}")
    c = synth.gemv_case(300 + i, K, N)
    ref = oracle.linear(c["x"], c["W"])[0]
    y = ql.qlinear_gemv(w4_dev(c["W"]), t(c["x"][0]))
    torch.cuda.synchronize()
    assert_close(host(y).astype(np.float64), ref, f"gemv K={K} N={N}")


@pytest.mark.parametrize("i", range(len(MOE_SHAPES)))
def test_random_moe_layer(i):
    """The prefill call sequence (route, gate/up, down, combine) on random
    T, D, I, E, top-k; the routed expert sets must equal the oracle's
    (cases with a near tie at the top-k cut are skipped by construction:
    the seed is advanced until the oracle's gap clears 1e-4)."""
    import torch
    T, D, I, E, topk = MOE_SHAPES[i]
    topk = min(topk, E)
    for seed in range(400 + 100 * i, 400 + 100 * i + 50):
        w = synth.moe_weights(seed, D=D, I=I, E=E)
        tok = synth.moe_tokens(seed + 1, T, D=D, E=E, skewed=True)
        L = oracle.router_logits(tok["H"], w["Wr"], tok["logit_bias"])
        srt = -np.sort(-L, axis=1)
        if topk == E or (srt[:, topk - 1] - srt[:, topk]).min() > 1e-4:
            break
    else:
        pytest.skip("no screened seed in 50 tries")
    say(f"random moe T={T} D={D} I={I} E={E} topk={topk} seed={seed}")
    ref = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk)
    H = t(tok["H"])
    dw = {k: w4_dev(w[k]) for k in ("gate_up", "down", "shared_gate_up", "shared_down")}
    route = ql.moe_route(H, t(w["Wr"]), t(tok["logit_bias"]), topk)
    act = ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk, ql.QL_OP_GATE_UP_SILU, route)
    yd = ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk, ql.QL_OP_DOWN, route)
    out = ql.moe_combine(yd, route["gates"], route["pos"], T, topk, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(route["ids"]), ref["ids"])
    assert np.array_equal(host(route["sorted_assign"]), ref["sorted_assign"])
    assert_close(host(out).astype(np.float64), ref["out"], "moe out")


def _codec_dev(W):
    import torch
    d = {k: (t(v) if isinstance(v, np.ndarray) and v.ndim > 0 else v) for k, v in W.items()}
    if "global_scale" in d and not torch.is_tensor(d["global_scale"]):
        d["global_scale"] = float(d["global_scale"])
    return d


@pytest.mark.parametrize("codec", ["fp8", "nvfp4"])
@pytest.mark.parametrize("i", range(len(MOE_SHAPES)))
def test_random_moe_layer_codecs(i, codec):
    """The same call sequence with FP8 or NVFP4 experts (moe_grouped_gemm_fp8
    / _nvfp4); the router weight equals moe_weights(seed)'s, so the seed
    screening is the w4 layer's."""
    import torch
    T, D, I, E, topk = MOE_SHAPES[i]
    topk = min(topk, E)
    for seed in range(400 + 100 * i, 400 + 100 * i + 50):
        tok = synth.moe_tokens(seed + 1, T, D=D, E=E, skewed=True)
        L = oracle.router_logits(tok["H"], synth.router_weight(synth.rng_for(seed), D, E), tok["logit_bias"])
        srt = -np.sort(-L, axis=1)
        if topk == E or (srt[:, topk - 1] - srt[:, topk]).min() > 1e-4:
            break
    else:
        pytest.skip("no screened seed in 50 tries")
    say(f"random moe {codec} T={T} D={D} I={I} E={E} topk={topk} seed={seed}")
    if codec == "fp8":
        w, layer, gemm = synth.moe_weights_fp8(seed, D=D, I=I, E=E), oracle.moe_layer_fp8, ql.moe_grouped_gemm_fp8
    else:
        w, layer, gemm = synth.moe_weights_nvfp4(seed, D=D, I=I, E=E), oracle.moe_layer_nvfp4, ql.moe_grouped_gemm_nvfp4
    ref = layer(tok["H"], w, tok["logit_bias"], topk)
    H = t(tok["H"])
    dw = {k: _codec_dev(w[k]) for k in ("gate_up", "down", "shared_gate_up", "shared_down")}
    route = ql.moe_route(H, t(w["Wr"]), t(tok["logit_bias"]), topk)
    act = gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk, ql.QL_OP_GATE_UP_SILU, route)
    yd = gemm(dw["down"], dw["shared_down"], act, T, topk, ql.QL_OP_DOWN, route)
    out = ql.moe_combine(yd, route["gates"], route["pos"], T, topk, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(route["ids"]), ref["ids"])
    assert np.array_equal(host(route["sorted_assign"]), ref["sorted_assign"])
    assert_close(host(out).astype(np.float64), ref["out"], f"moe {codec} out")
