"""GPU parity of the bf16 variant (bf16 activations, scales, biases and
outputs) of the GEMV and the GEMM against the oracle, at the derived bf16
tolerance (tests/gpu_util.py)."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close_bf16, guarded, say, t, w4_dev

pytestmark = pytest.mark.gpu


def bits(y):
    import torch
    return y.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("K,N,seed", [
    (2048, 8192, 0), (256, 100, 1), (512, 513, 2), (1024, 1000, 3),
    (4096, 257, 4), (8192, 65, 5), (16384, 33, 6), (2048, 1, 7),
])
def test_gemv_bf16_matches_oracle(K, N, seed):
    import torch
    say(f"gemv_bf16 K={K} N={N} seed={seed}")
    c = synth.gemm_case_bf16(seed, 1, K, N)
    ref = oracle.linear_bf16(c["X"], c["W"])[0]
    y = ql.qlinear_gemv_bf16(w4_dev(c["W"]), t(c["X"][0]))
    torch.cuda.synchronize()
    rel, mx = assert_close_bf16(bits(y), ref, f"gemv_bf16 K={K} N={N}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemv_bf16_vocab_head_full():
    """K = 2048, N = 151552 in the benchmark's launch configuration: every
    output against the oracle, behind guard regions."""
    import torch
    K, N = 2048, synth.VOCAB
    say(f"gemv_bf16 head K={K} N={N}")
    c = synth.gemm_case_bf16(9, 1, K, N)
    y = guarded(N, torch.bfloat16)
    ql.qlinear_gemv_bf16(w4_dev(c["W"]), t(c["X"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv_bf16 head")
    rel, mx = assert_close_bf16(bits(y.t), oracle.linear_bf16(c["X"], c["W"])[0], "gemv_bf16 head")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("K,N,seed", [(2048, 40001, 13), (4096, 33001, 14), (1024, 65601, 15)])
def test_gemv_bf16_eight_rows_ragged(K, N, seed):
    """The 8-rows-per-lane instance with a ragged last block."""
    import torch
    say(f"gemv_bf16 8-row K={K} N={N}")
    c = synth.gemm_case_bf16(seed, 1, K, N)
    y = guarded(N, torch.bfloat16)
    ql.qlinear_gemv_bf16(w4_dev(c["W"]), t(c["X"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv_bf16")
    assert_close_bf16(bits(y.t), oracle.linear_bf16(c["X"], c["W"])[0], f"gemv_bf16 K={K} N={N}")


@pytest.mark.parametrize("M,K,N,seed", [
    (1, 2048, 512, 0), (7, 512, 200, 1), (300, 2048, 1000, 2), (129, 64, 257, 3),
    (700, 1024, 3000, 4), (1500, 512, 4000, 5), (2100, 256, 4100, 6),
])
def test_gemm_bf16_matches_oracle(M, K, N, seed):
    """Ragged M and N in every tile class of the shape table."""
    import torch
    say(f"gemm_bf16 M={M} K={K} N={N} seed={seed}")
    c = synth.gemm_case_bf16(seed, M, K, N)
    ref = oracle.linear_bf16(c["X"], c["W"])
    Y = ql.qlinear_gemm_bf16(w4_dev(c["W"]), t(c["X"]))
    torch.cuda.synchronize()
    rel, mx = assert_close_bf16(bits(Y), ref, f"gemm_bf16 M={M} K={K} N={N}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemm_bf16_prefill_full():
    """The prefill shape (M = 4096, K = 2048, N = 8192) in the benchmark's
    launch configuration (256 x 256 tiles): every output against the oracle,
    behind guard regions."""
    import torch
    M, K, N = 4096, 2048, 8192
    say("gemm_bf16 prefill M=4096")
    c = synth.gemm_case_bf16(0, M, K, N)
    Y = guarded((M, N), torch.bfloat16)
    ql.qlinear_gemm_bf16(w4_dev(c["W"]), t(c["X"]), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm_bf16 prefill")
    rel, mx = assert_close_bf16(bits(Y.t), oracle.linear_bf16(c["X"], c["W"]), "gemm_bf16 M=4096")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemm_bf16_row_invariance():
    import torch
    K, N = 2048, 4096
    c = synth.gemm_case_bf16(5, 4096, K, N)
    W = w4_dev(c["W"])
    X = t(c["X"])
    full = bits(ql.qlinear_gemm_bf16(W, X))
    for M in (1, 1000, 2048):
        part = bits(ql.qlinear_gemm_bf16(W, X[:M].contiguous()))
        assert np.array_equal(part, full[:M]), M
    torch.cuda.synchronize()


def test_bf16_integer_case_bit_exact():
    """scale 1, bias 0 and small integer activations: every weight, product
    and fp32 sum is exact, so both paths give the oracle's bf16 rounding of
    the exact result, bit for bit."""
    import torch
    rng = np.random.default_rng(17)
    K, N, M = 512, 320, 200
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    W = {"qweight": words, "scales": np.full((N, K // 64), 0x3F80, np.uint16),
         "biases": np.zeros((N, K // 64), np.uint16), "K": K, "N": N}
    Xf = rng.integers(-2, 3, size=(M, K)).astype(np.float64)
    X = oracle.round_bf16(Xf)                      # small integers: exact in bf16
    ref = oracle.round_bf16(oracle.linear_bf16(X, W))
    Wd = w4_dev(W)
    Y = bits(ql.qlinear_gemm_bf16(Wd, t(X)))
    y = bits(ql.qlinear_gemv_bf16(Wd, t(X[0])))
    torch.cuda.synchronize()
    assert np.array_equal(Y, ref)
    assert np.array_equal(y, ref[0])
