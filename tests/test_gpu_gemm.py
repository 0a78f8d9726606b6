"""GPU parity of qlinear_gemm against the oracle."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, guarded, host, say, t, w4_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,K,N,seed", [
    (1, 2048, 512, 0), (7, 512, 200, 1), (256, 2048, 8192, 0), (300, 2048, 1000, 2),
    (129, 64, 257, 3), (1024, 1024, 640, 4), (2048, 512, 384, 5), (2500, 192, 300, 6),
    (700, 1024, 3000, 7), (1500, 512, 4000, 8), (2100, 256, 4100, 9),
    (130, 32768, 70, 10),  # the largest K (QL_MAX_K)
])
def test_gemm_matches_oracle(M, K, N, seed):
    """Ragged M and N in every tile class of the shape table (64 x 128,
    128 x 128, 128 x 256 and 256 x 256 tiles), outputs behind guard
    regions."""
    import torch
    say(f"gemm M={M} K={K} N={N} seed={seed}")
    case = synth.gemm_case(seed, M, K, N)
    ref = oracle.linear(case["X"], case["W"])
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm(w4_dev(case["W"]), t(case["X"]), Y.t)
    torch.cuda.synchronize()
    Y.check(f"gemm M={M} K={K} N={N}")
    assert_close(host(Y.t).astype(np.float64), ref, f"gemm M={M} K={K} N={N}")


def test_gemm_prefill_full():
    """The prefill workload (M = 4096, K = 2048, N = 8192) in the benchmark's
    launch configuration (256 x 256 tiles): every output against the
    oracle, behind guard regions."""
    import torch
    M, K, N = 4096, 2048, 8192
    say(f"gemm prefill M={M}")
    case = synth.gemm_case(0, M, K, N)
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm(w4_dev(case["W"]), t(case["X"]), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm prefill")
    rel, mx = assert_close(host(Y.t).astype(np.float64), oracle.linear(case["X"], case["W"]), "gemm prefill")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemm_prefill_16384_full():
    """M = 16384 (the sweep's largest M): every output against the oracle,
    behind guard regions."""
    import torch
    M, K, N = 16384, 2048, 8192
    say(f"gemm prefill M={M}")
    case = synth.gemm_case(0, M, K, N)
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm(w4_dev(case["W"]), t(case["X"]), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm prefill 16384")
    rel, mx = assert_close(host(Y.t).astype(np.float64), oracle.linear(case["X"], case["W"]), f"gemm M={M}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemm_row_invariance():
    """Row m of the output depends only on row m of X: bit-identical across
    M in {1, 1000, 2048, 4096}, which fall in the four tile classes of the
    shape table at N = 4096 (no split over K, same accumulation order)."""
    import torch
    K, N = 2048, 4096
    case = synth.gemm_case(5, 4096, K, N)
    W = w4_dev(case["W"])
    Xd = t(case["X"])
    full = host(ql.qlinear_gemm(W, Xd)).view(np.uint16)
    for M in (1, 1000, 2048):
        part = host(ql.qlinear_gemm(W, Xd[:M].contiguous())).view(np.uint16)
        assert np.array_equal(part, full[:M]), f"M={M}"
    torch.cuda.synchronize()


def test_gemm_integer_case_bit_exact():
    import torch
    rng = np.random.default_rng(13)
    K, N, M = 512, 320, 200
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    W = {"qweight": words, "scales": np.ones((N, K // 64), np.float16),
         "biases": np.zeros((N, K // 64), np.float16), "K": K, "N": N}
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    ref = oracle.round_f16(oracle.linear(X, W))
    Y = host(ql.qlinear_gemm(w4_dev(W), t(X)))
    torch.cuda.synchronize()
    assert np.array_equal(Y.view(np.uint16), ref.view(np.uint16))


def test_gemv_and_gemm_agree_on_one_row():
    import torch
    case = synth.gemm_case(8, 1, 2048, 8192)
    W = w4_dev(case["W"])
    y1 = host(ql.qlinear_gemv(W, t(case["X"][0]))).astype(np.float64)
    y2 = host(ql.qlinear_gemm(W, t(case["X"])))[0].astype(np.float64)
    torch.cuda.synchronize()
    ref = oracle.linear(case["X"], case["W"])[0]
    assert_close(y1, ref, "gemv")
    assert_close(y2, ref, "gemm M=1")


@pytest.mark.parametrize("M,K,N,seed", [
    (1, 2048, 512, 10), (2, 512, 200, 11), (5, 1024, 1000, 12), (31, 2048, 257, 13),
    (32, 2048, 8192, 14), (33, 512, 96, 15), (64, 1024, 640, 16), (100, 2048, 33, 17),
    (256, 2048, 8192, 18), (1024, 512, 384, 19),
])
def test_gemm_few_rows_matches_oracle(M, K, N, seed):
    """Weight-stationary few-row GEMM: full parity over ragged M (chunks of
    32 rows) and N (blocks of 32 columns), every supported K."""
    import torch
    say(f"gemm_few_rows M={M} K={K} N={N} seed={seed}")
    case = synth.gemm_case(seed, M, K, N)
    ref = oracle.linear(case["X"], case["W"])
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm_few_rows(w4_dev(case["W"]), t(case["X"]), Y.t)
    torch.cuda.synchronize()
    Y.check(f"gemm_few_rows M={M} K={K} N={N}")
    assert_close(host(Y.t).astype(np.float64), ref, f"gemm_few_rows M={M} K={K} N={N}")


@pytest.mark.parametrize("M,K,N,seed", [
    (1, 2048, 512, 30), (7, 128, 200, 31), (63, 1024, 1000, 32), (64, 2048, 8192, 33),
    (129, 256, 257, 34), (256, 2048, 8192, 35), (300, 4096, 700, 36), (513, 512, 384, 37),
    (1024, 2048, 8192, 38), (1500, 1024, 4100, 39),
])
def test_gemm_ksplit_matches_oracle(M, K, N, seed):
    """The K-split GEMM (two halves of K per workgroup, summed at the end):
    full parity over ragged M and N in both of its tile classes, K from one
    pair of groups up."""
    import torch
    say(f"gemm_ksplit M={M} K={K} N={N} seed={seed}")
    case = synth.gemm_case(seed, M, K, N)
    ref = oracle.linear(case["X"], case["W"])
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm_ksplit(w4_dev(case["W"]), t(case["X"]), Y.t)
    torch.cuda.synchronize()
    Y.check(f"gemm_ksplit M={M} K={K} N={N}")
    assert_close(host(Y.t).astype(np.float64), ref, f"gemm_ksplit M={M} K={K} N={N}")


def test_gemm_ksplit_row_invariance_and_determinism():
    """Row m of the K-split GEMM is the same bits for M = 1, 64, 256, 1024
    (both tile classes split K the same way), and repeated calls agree."""
    import torch
    K, N = 2048, 8192
    case = synth.gemm_case(40, 1024, K, N)
    W = w4_dev(case["W"])
    X = t(case["X"])
    full = host(ql.qlinear_gemm_ksplit(W, X))
    again = host(ql.qlinear_gemm_ksplit(W, X))
    torch.cuda.synchronize()
    assert np.array_equal(full.view(np.uint16), again.view(np.uint16))
    for M in (1, 64, 256):
        part = host(ql.qlinear_gemm_ksplit(W, X[:M].contiguous()))
        torch.cuda.synchronize()
        assert np.array_equal(part.view(np.uint16), full[:M].view(np.uint16)), M


def test_gemm_ksplit_integer_case_bit_exact():
    """Scale 1, bias 0 and small integer activations: every fp32 partial sum
    is exact, so both halves and their sum are too, and the K-split GEMM
    equals the oracle's rounded result bit for bit."""
    import torch
    rng = np.random.default_rng(41)
    M, K, N = 200, 1024, 300
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    W = {"qweight": words, "scales": np.ones((N, K // 64), np.float16),
         "biases": np.zeros((N, K // 64), np.float16), "K": K, "N": N}
    X = rng.integers(-2, 3, size=(M, K)).astype(np.float16)
    ref = oracle.round_f16(oracle.linear(X, W))
    Y = host(ql.qlinear_gemm_ksplit(w4_dev(W), t(X)))
    torch.cuda.synchronize()
    assert np.array_equal(Y.view(np.uint16), ref.view(np.uint16))


def test_gemm_few_rows_row_invariance_and_determinism():
    """Row m of the few-row GEMM depends only on row m of X (the same bits
    for M = 1, 7, 96, 300), and repeated calls give identical bits."""
    import torch
    K, N = 2048, 1000
    case = synth.gemm_case(21, 300, K, N)
    W = w4_dev(case["W"])
    X = t(case["X"])
    full = host(ql.qlinear_gemm_few_rows(W, X))
    again = host(ql.qlinear_gemm_few_rows(W, X))
    torch.cuda.synchronize()
    assert np.array_equal(full.view(np.uint16), again.view(np.uint16))
    for M in (1, 7, 96):
        part = host(ql.qlinear_gemm_few_rows(W, X[:M].contiguous()))
        torch.cuda.synchronize()
        assert np.array_equal(part.view(np.uint16), full[:M].view(np.uint16)), M
