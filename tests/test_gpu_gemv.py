"""GPU parity of qlinear_gemv (and qlinear_pack) against the oracle."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, host, say, t, w4_dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("K,N,seed", [
    (512, 512, 0), (512, 512, 1), (512, 512, 2),    # the small GEMV workload
    (2048, 8192, 0), (2048, 8192, 1),               # model-size projection
    (64, 5, 3), (192, 33, 4), (640, 70, 5),         # runtime-group fallbacks, ragged N
    (1024, 1000, 6), (4096, 129, 7), (8192, 65, 8), (16384, 17, 9),
    (2048, 1, 10), (2048, 3, 11),
    (32768, 40, 12),                                # the largest K (QL_MAX_K)
])
def test_gemv_matches_oracle(K, N, seed):
    say(f"gemv K={K} N={N} seed={seed}")
    case = synth.gemv_case(seed, K, N)
    ref = oracle.linear(case["x"], case["W"])[0]
    y = ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]))
    import torch
    torch.cuda.synchronize()
    assert_close(host(y).astype(np.float64), ref, f"gemv K={K} N={N}")


def test_gemv_vocab_head_sampled():
    """K = 2048, N = 151552 (vocabulary head): every output computed on the
    GPU, a sample of 4096 rows (first, last and strided) checked."""
    import torch
    K, N = 2048, synth.VOCAB
    say(f"gemv head K={K} N={N}")
    case = synth.gemv_case(1, K, N)
    y = host(ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]))).astype(np.float64)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N),
                                     np.linspace(0, N - 1, 3968).astype(np.int64)]))
    W = case["W"]
    sub = {"qweight": W["qweight"][rows], "scales": W["scales"][rows], "biases": W["biases"][rows],
           "K": K, "N": len(rows)}
    ref = oracle.linear(case["x"], sub)[0]
    assert_close(y[rows], ref, "gemv head sample")
    assert np.all(np.isfinite(y))


def test_gemv_integer_case_bit_exact():
    """scale 1, bias 0, small integer x: every product and partial sum is an
    exact integer in fp32, so the fp16 result must equal the oracle's
    rounded result bit for bit."""
    import torch
    rng = np.random.default_rng(12)
    for K, N in [(512, 256), (2048, 130), (192, 9)]:
        words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
        W = {"qweight": words, "scales": np.ones((N, K // 64), np.float16),
             "biases": np.zeros((N, K // 64), np.float16), "K": K, "N": N}
        x = rng.integers(-2, 3, size=K).astype(np.float16)
        ref = oracle.round_f16(oracle.linear(x, W)[0])
        y = host(ql.qlinear_gemv(w4_dev(W), t(x)))
        torch.cuda.synchronize()
        assert np.array_equal(y.view(np.uint16), ref.view(np.uint16)), f"K={K} N={N}"


def test_gemv_empty_is_noop():
    import torch
    W = {"qweight": torch.zeros((0, 64), dtype=torch.int32, device="cuda"),
         "scales": torch.zeros((0, 8), dtype=torch.float16, device="cuda"),
         "biases": torch.zeros((0, 8), dtype=torch.float16, device="cuda"), "K": 512, "N": 0}
    y = ql.qlinear_gemv(W, torch.zeros(512, dtype=torch.float16, device="cuda"))
    torch.cuda.synchronize()
    assert y.numel() == 0


def test_pack_matches_oracle():
    import torch
    rng = np.random.default_rng(3)
    for N, K in [(7, 64), (300, 2048), (1, 8)]:
        codes = rng.integers(0, 16, size=(N, K)).astype(np.uint8)
        ref = oracle.pack_codes(codes)
        got = host(ql.qlinear_pack(t(codes))).view(np.uint32)
        torch.cuda.synchronize()
        assert np.array_equal(got, ref)
