"""GPU behaviour on special values, against the oracle.

A NaN activation poisons exactly the outputs that depend on it: every
output of the GEMV, one row of the GEMM (the rows stay independent), one
token's output of the routed-expert layer (its NaN logits rank below every
number, so its experts stay valid ids).
Outputs beyond the fp16 range overflow to infinity exactly where rounding
the oracle's exact result to fp16 does: with scale 512 and bias -4096 on
every other output column (dequantized weights 512 q - 4096, exact in fp16,
so the GEMM's fp16 weights are the oracle's), those columns' sums reach 1e5
and mostly overflow, while the other columns keep the workload's scales.
Rounding to nearest even sends |y| >= 65520 to infinity; outputs within
0.1% of that boundary may fall either way under fp32 accumulation and are
only checked for sign and range.
"""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, host, say, t, w4_dev

pytestmark = pytest.mark.gpu

FP16_OVERFLOW = 65520.0  # smallest magnitude that rounds to infinity
BAND = 1e-3


def overflow_case(seed, M, K, N):
    rng = synth.rng_for(seed)
    X = synth.activations(rng, M, K)
    W = synth.w4_matrix(rng, K, N)
    sc = W["scales"].astype(np.float64)
    bi = W["biases"].astype(np.float64)
    sc[1::2, :] = 512.0   # weights 512 q - 4096: multiples of 512, exact in fp16
    bi[1::2, :] = -4096.0
    return X, dict(W, scales=synth.f16(sc), biases=synth.f16(bi))


def check_overflow(g, ref, what):
    g = np.asarray(g, dtype=np.float64)
    a = np.abs(ref)
    big = a >= FP16_OVERFLOW * (1 + BAND)
    small = a <= FP16_OVERFLOW * (1 - BAND)
    band = ~(big | small)
    assert big.any() and small.any(), what
    assert np.isinf(g[big]).all(), f"{what}: {int((~np.isinf(g[big])).sum())} outputs beyond fp16 are finite"
    assert (np.sign(g[big]) == np.sign(ref[big])).all(), f"{what}: overflow sign"
    assert np.isfinite(g[small]).all(), f"{what}: {int((~np.isfinite(g[small])).sum())} representable outputs overflowed"
    assert (np.isinf(g[band]) | (np.abs(g[band]) <= 65504.0)).all(), f"{what}: boundary outputs"
    assert (np.sign(g[band]) == np.sign(ref[band])).all(), f"{what}: boundary signs"
    # the columns with the workload's scales, and the finite outputs of the others
    assert_close(g[..., 0::2], ref[..., 0::2], f"{what}: ordinary columns")
    odd = np.zeros_like(small)
    odd[..., 1::2] = True
    keep = small & odd
    assert_close(g[keep], ref[keep], f"{what}: finite outputs of the large-scale columns")


@pytest.mark.parametrize("K,N", [(2048, 8192), (2048, 40001), (512, 512)])
def test_gemv_nan_activation_poisons_every_output(K, N):
    import torch
    say(f"gemv NaN activation K={K} N={N}")
    case = synth.gemv_case(50, K, N)
    x = case["x"][0].copy()
    x[K // 3] = np.float16(np.nan)
    y = torch.empty(N, dtype=torch.float16, device="cuda")
    ql.qlinear_gemv(w4_dev(case["W"]), t(x), y=y)
    torch.cuda.synchronize()
    assert np.isnan(host(y).astype(np.float64)).all()


@pytest.mark.parametrize("M,K,N", [(300, 2048, 1000), (4096, 512, 8192)])
def test_gemm_nan_activation_poisons_only_its_row(M, K, N):
    """Small and 256 x 256 tile classes: the row holding the NaN is NaN
    everywhere, every other row matches the oracle."""
    import torch
    say(f"gemm NaN activation M={M} K={K} N={N}")
    case = synth.gemm_case(51, M, K, N)
    X = case["X"].copy()
    r = M // 2 + 1
    X[r, K // 5] = np.float16(np.nan)
    Y = host(ql.qlinear_gemm(w4_dev(case["W"]), t(X))).astype(np.float64)
    torch.cuda.synchronize()
    assert np.isnan(Y[r]).all()
    rest = np.delete(np.arange(M), r)
    assert_close(Y[rest], oracle.linear(X[rest], case["W"]), f"gemm M={M} rows without NaN")


@pytest.mark.parametrize("K,N", [(2048, 8192), (2048, 40001)])
def test_gemv_overflow_to_infinity(K, N):
    """The model-size projection and a ragged head-class launch (eight rows
    per wave)."""
    import torch
    say(f"gemv overflow K={K} N={N}")
    X, W = overflow_case(60, 1, K, N)
    y = torch.empty(N, dtype=torch.float16, device="cuda")
    ql.qlinear_gemv(w4_dev(W), t(X[0]), y=y)
    torch.cuda.synchronize()
    check_overflow(host(y), oracle.linear(X, W)[0], f"gemv K={K} N={N}")


@pytest.mark.parametrize("M,K,N", [(300, 2048, 1000), (4096, 512, 8192)])
def test_gemm_overflow_to_infinity(M, K, N):
    import torch
    say(f"gemm overflow M={M} K={K} N={N}")
    X, W = overflow_case(61, M, K, N)
    Y = ql.qlinear_gemm(w4_dev(W), t(X))
    torch.cuda.synchronize()
    check_overflow(host(Y), oracle.linear(X, W), f"gemm M={M} K={K} N={N}")


def _moe_dev_weights(w):
    return {"Wr": t(w["Wr"]), "gate_up": w4_dev(w["gate_up"]), "down": w4_dev(w["down"]),
            "shared_gate_up": w4_dev(w["shared_gate_up"]), "shared_down": w4_dev(w["shared_down"])}


def _check_nan_token(ids, out, r, E, topk, ref_out, what):
    """The poisoned token still has topk distinct experts in range; its
    output row is NaN; every other row matches the oracle run on the other
    tokens alone."""
    ids = np.asarray(ids)
    assert ids.min() >= 0 and ids.max() < E, f"{what}: expert id out of range"
    assert all(len(set(row)) == topk for row in ids.tolist()), f"{what}: repeated expert"
    o = np.asarray(out, dtype=np.float64)
    assert np.isnan(o[r]).all(), f"{what}: the NaN token's output is not NaN"
    keep = np.delete(np.arange(o.shape[0]), r)
    assert_close(o[keep], ref_out, f"{what}: the other tokens")


@pytest.mark.parametrize("T,D,I,E,topk,seed", [(300, 256, 128, 16, 4, 3), (700, 512, 256, 64, 8, 4)])
def test_moe_nan_token_poisons_only_its_output(T, D, I, E, topk, seed):
    """Prefill path (route, grouped gate/up, down, combine): a token whose
    hidden state holds a NaN has NaN logits, which the top-k ranks below
    every number, so it still takes topk valid experts; its rows share tiles
    with other tokens' rows, which stay independent."""
    import torch
    say(f"moe NaN token T={T} D={D} E={E} topk={topk}")
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 50, T, D=D, E=E, skewed=True)
    H = tok["H"].copy()
    r = T // 3
    H[r, D // 2] = np.float16(np.nan)
    dw = _moe_dev_weights(w)
    Hd = t(H)
    route = ql.moe_route(Hd, dw["Wr"], t(tok["logit_bias"]), topk)
    act = ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], Hd, T, topk, ql.QL_OP_GATE_UP_SILU, route)
    ydown = ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk, ql.QL_OP_DOWN, route)
    out = ql.moe_combine(ydown, route["gates"], route["pos"], T, topk, True)
    torch.cuda.synchronize()
    keep = np.delete(np.arange(T), r)
    ref = oracle.moe_layer(H[keep], w, tok["logit_bias"], topk)
    _check_nan_token(host(route["ids"]), host(out), r, E, topk, ref["out"], f"moe T={T}")


def test_moe_decode_nan_token_poisons_only_its_output():
    """The fused decode layer (moe_decode) on four tokens, one of them with a
    NaN in its hidden state."""
    import torch
    T, D, I, E, topk, seed = 4, 2048, 512, 256, 8, 7
    say("moe_decode NaN token")
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 60, T, D=D, E=E, skewed=True)
    H = tok["H"].copy()
    r = 2
    H[r, 7] = np.float16(np.nan)
    dw = _moe_dev_weights(w)
    res = ql.moe_decode(t(H), dw["Wr"], t(tok["logit_bias"]), topk, gate_up=dw["gate_up"], down=dw["down"],
                        shared_gate_up=dw["shared_gate_up"], shared_down=dw["shared_down"])
    torch.cuda.synchronize()
    keep = np.delete(np.arange(T), r)
    ref = oracle.moe_layer(H[keep], w, tok["logit_bias"], topk)
    _check_nan_token(host(res["ids"]), host(res["out"]), r, E, topk, ref["out"], "moe_decode")
