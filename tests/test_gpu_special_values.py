"""GPU behaviour on special values, against the oracle.

A NaN activation poisons exactly the outputs that depend on it: every
output of the GEMV, one row of the GEMM (the rows stay independent).
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
