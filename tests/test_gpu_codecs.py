"""GPU parity of the second weight codecs (FP8-E4M3 and NVFP4 single-row
GEMV) against the oracle, at the fp16 output tolerance."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, host, say, t

pytestmark = pytest.mark.gpu


def fp8_dev(W):
    return {"codes": t(W["codes"]), "scales": t(W["scales"]), "K": W["K"], "N": W["N"]}


def nvfp4_dev(W):
    return {"qweight": t(W["qweight"]), "block_scales": t(W["block_scales"]),
            "global_scale": float(W["global_scale"]), "K": W["K"], "N": W["N"]}


@pytest.mark.parametrize("K,N,seed", [
    (2048, 8192, 0), (256, 100, 1), (512, 513, 2), (1024, 1000, 3), (4096, 257, 4),
    (8192, 65, 5), (2048, 1, 6), (2048, 3, 7),
])
def test_gemv_fp8_matches_oracle(K, N, seed):
    import torch
    say(f"gemv_fp8 K={K} N={N} seed={seed}")
    rng = synth.rng_for(seed)
    x = synth.activations(rng, 1, K)
    W = synth.fp8_matrix(rng, K, N)
    ref = oracle.linear_fp8(x, W)[0]
    y = ql.qlinear_gemv_fp8(fp8_dev(W), t(x[0]))
    torch.cuda.synchronize()
    rel, mx = assert_close(host(y).astype(np.float64), ref, f"gemv_fp8 K={K} N={N}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("K,N,seed", [
    (2048, 8192, 0), (256, 100, 1), (512, 513, 2), (1024, 1000, 3), (4096, 257, 4),
    (8192, 65, 5), (16384, 33, 6), (2048, 1, 7),
])
def test_gemv_nvfp4_matches_oracle(K, N, seed):
    import torch
    say(f"gemv_nvfp4 K={K} N={N} seed={seed}")
    rng = synth.rng_for(seed)
    x = synth.activations(rng, 1, K)
    W = synth.nvfp4_matrix(rng, K, N)
    ref = oracle.linear_nvfp4(x, W)[0]
    y = ql.qlinear_gemv_nvfp4(nvfp4_dev(W), t(x[0]))
    torch.cuda.synchronize()
    rel, mx = assert_close(host(y).astype(np.float64), ref, f"gemv_nvfp4 K={K} N={N}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("codec", ["fp8", "nvfp4"])
def test_codec_vocab_head_sampled(codec):
    """K = 2048, N = 151552: every output computed, 4096 sampled rows checked."""
    import torch
    K, N = 2048, synth.VOCAB
    say(f"gemv_{codec} head")
    rng = synth.rng_for(11)
    x = synth.activations(rng, 1, K)
    if codec == "fp8":
        W = synth.fp8_matrix(rng, K, N)
        y = host(ql.qlinear_gemv_fp8(fp8_dev(W), t(x[0]))).astype(np.float64)
    else:
        W = synth.nvfp4_matrix(rng, K, N)
        y = host(ql.qlinear_gemv_nvfp4(nvfp4_dev(W), t(x[0]))).astype(np.float64)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(64), np.arange(N - 64, N),
                                     np.linspace(0, N - 1, 3968).astype(np.int64)]))
    if codec == "fp8":
        sub = {"codes": W["codes"][rows], "scales": W["scales"][rows], "K": K, "N": len(rows)}
        ref = oracle.linear_fp8(x, sub)[0]
    else:
        sub = {"qweight": W["qweight"][rows], "block_scales": W["block_scales"][rows],
               "global_scale": W["global_scale"], "K": K, "N": len(rows)}
        ref = oracle.linear_nvfp4(x, sub)[0]
    assert_close(y[rows], ref, f"gemv_{codec} head sample")


def test_codecs_integer_case_bit_exact():
    """Codes of +-1 and halves, unit scales and small integer activations:
    every product and fp32 sum is exact, so the outputs equal the oracle's
    rounded results bit for bit (a check of the decodes themselves)."""
    import torch
    rng = np.random.default_rng(21)
    K, N = 1024, 200
    x = rng.integers(-3, 4, size=K).astype(np.float16)
    codes = rng.choice(np.array([0x38, 0xB8, 0x30, 0xB0, 0x00, 0x40], np.uint8), size=(N, K))
    W8 = {"codes": codes, "scales": np.ones((N, K // 64), np.float16), "K": K, "N": N}
    ref8 = oracle.round_f16(oracle.linear_fp8(x, W8)[0])
    words = rng.integers(0, 2**32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    W4 = {"qweight": words, "block_scales": np.full((N, K // 16), 0x38, np.uint8),
          "global_scale": np.float32(1.0), "K": K, "N": N}
    ref4 = oracle.round_f16(oracle.linear_nvfp4(x, W4)[0])
    y8 = host(ql.qlinear_gemv_fp8(fp8_dev(W8), t(x)))
    y4 = host(ql.qlinear_gemv_nvfp4(nvfp4_dev(W4), t(x)))
    torch.cuda.synchronize()
    assert np.array_equal(y8.view(np.uint16), ref8.view(np.uint16))
    assert np.array_equal(y4.view(np.uint16), ref4.view(np.uint16))


@pytest.mark.parametrize("M,K,N,seed", [
    (1, 2048, 512, 0), (7, 512, 200, 1), (256, 2048, 8192, 2), (300, 2048, 1000, 3),
    (129, 64, 257, 4), (1024, 1024, 640, 5), (2048, 512, 384, 6), (2500, 192, 300, 7),
    (700, 1024, 3000, 8), (2100, 256, 4100, 9), (130, 32768, 70, 10),
])
def test_gemm_fp8_matches_oracle(M, K, N, seed):
    """FP8 weights on the MFMA tiles: ragged M and N in every tile class,
    the largest K."""
    import torch
    say(f"gemm_fp8 M={M} K={K} N={N} seed={seed}")
    rng = synth.rng_for(seed)
    X = synth.activations(rng, M, K)
    W = synth.fp8_matrix(rng, K, N)
    ref = oracle.linear_fp8(X, W)
    Y = ql.qlinear_gemm_fp8(fp8_dev(W), t(X))
    torch.cuda.synchronize()
    rel, mx = assert_close(host(Y).astype(np.float64), ref, f"gemm_fp8 M={M} K={K} N={N}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemm_fp8_prefill_sampled_rows_and_row_invariance():
    """The prefill shape (M = 4096, K = 2048, N = 8192): 64 sampled rows
    against the oracle, and every row's bits equal to the same row computed
    with M = 1 and M = 256 (no split over K, the same K order)."""
    import torch
    M, K, N = 4096, 2048, 8192
    rng = synth.rng_for(20)
    X = synth.activations(rng, M, K)
    W = synth.fp8_matrix(rng, K, N)
    Wd, Xd = fp8_dev(W), t(X)
    Y = host(ql.qlinear_gemm_fp8(Wd, Xd))
    rows = np.sort(synth.rng_for(21).choice(M, 64, replace=False))
    ref = oracle.linear_fp8(X[rows], W)
    assert_close(Y[rows].astype(np.float64), ref, "gemm_fp8 sampled rows")
    for m in (0, 255, 4095):
        for MM in (1, 256):
            lo = min(m, M - MM)
            part = host(ql.qlinear_gemm_fp8(Wd, Xd[lo:lo + MM].contiguous()))
            assert np.array_equal(part[m - lo].view(np.uint16), Y[m].view(np.uint16)), (m, MM)
    torch.cuda.synchronize()


def test_gemm_fp8_integer_case_bit_exact():
    """Codes of small integers (E4M3 exact), scale 1, integer activations:
    every product and fp32 sum is exact, so the fp16 output equals the
    oracle's rounded value bit for bit."""
    import torch
    M, K, N = 300, 512, 260
    rng = synth.rng_for(30)
    # E4M3 codes of -4 .. 4: 0x00 (0), 0x38 (1), 0x40 (2), 0x44 (3), 0x48 (4), sign bit 0x80
    mags = np.array([0x00, 0x38, 0x40, 0x44, 0x48], dtype=np.uint8)
    codes = mags[rng.integers(0, 5, size=(N, K))] | (rng.integers(0, 2, size=(N, K)) * 0x80).astype(np.uint8)
    W = {"codes": codes.astype(np.uint8), "scales": np.ones((N, K // 64), dtype=np.float16), "K": K, "N": N}
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    ref = oracle.linear_fp8(X, W)
    Y = host(ql.qlinear_gemm_fp8(fp8_dev(W), t(X)))
    torch.cuda.synchronize()
    assert np.array_equal(Y.view(np.uint16), ref.astype(np.float16).view(np.uint16))


@pytest.mark.parametrize("M,K,N,seed", [
    (1, 2048, 512, 0), (7, 512, 200, 1), (256, 2048, 8192, 2), (300, 2048, 1000, 3),
    (129, 64, 257, 4), (1024, 1024, 640, 5), (2500, 192, 300, 7), (2100, 256, 4100, 9),
    (130, 32768, 70, 10),
])
def test_gemm_nvfp4_matches_oracle(M, K, N, seed):
    """NVFP4 weights on the MFMA tiles: ragged M and N in every tile class,
    the largest K."""
    import torch
    say(f"gemm_nvfp4 M={M} K={K} N={N} seed={seed}")
    rng = synth.rng_for(seed)
    X = synth.activations(rng, M, K)
    W = synth.nvfp4_matrix(rng, K, N)
    ref = oracle.linear_nvfp4(X, W)
    Y = ql.qlinear_gemm_nvfp4(nvfp4_dev(W), t(X))
    torch.cuda.synchronize()
    rel, mx = assert_close(host(Y).astype(np.float64), ref, f"gemm_nvfp4 M={M} K={K} N={N}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemm_nvfp4_prefill_sampled_rows_and_row_invariance():
    import torch
    M, K, N = 4096, 2048, 8192
    rng = synth.rng_for(22)
    X = synth.activations(rng, M, K)
    W = synth.nvfp4_matrix(rng, K, N)
    Wd, Xd = nvfp4_dev(W), t(X)
    Y = host(ql.qlinear_gemm_nvfp4(Wd, Xd))
    rows = np.sort(synth.rng_for(23).choice(M, 64, replace=False))
    ref = oracle.linear_nvfp4(X[rows], W)
    assert_close(Y[rows].astype(np.float64), ref, "gemm_nvfp4 sampled rows")
    for m in (0, 255, 4095):
        for MM in (1, 256):
            lo = min(m, M - MM)
            part = host(ql.qlinear_gemm_nvfp4(Wd, Xd[lo:lo + MM].contiguous()))
            assert np.array_equal(part[m - lo].view(np.uint16), Y[m].view(np.uint16)), (m, MM)
    torch.cuda.synchronize()


def test_gemm_nvfp4_integer_case_bit_exact():
    """E2M1 codes of integers (0, 1, 2, 3, 4, 6 and their negatives), block
    scales 1.0, global scale 1, integer activations: every product and fp32
    sum is exact, so the output equals the oracle's rounded value bit for
    bit."""
    import torch
    M, K, N = 300, 512, 260
    rng = synth.rng_for(31)
    nib = np.array([0x0, 0x2, 0x4, 0x5, 0x6, 0x7], dtype=np.uint32)[rng.integers(0, 6, size=(N, K))]
    nib = nib | (rng.integers(0, 2, size=(N, K)).astype(np.uint32) << 3)
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for j in range(8):
        words |= nib[:, j::8] << np.uint32(4 * j)
    W = {"qweight": words, "block_scales": np.full((N, K // 16), 0x38, dtype=np.uint8),
         "global_scale": np.float32(1.0), "K": K, "N": N}
    X = rng.integers(-3, 4, size=(M, K)).astype(np.float16)
    ref = oracle.linear_nvfp4(X, W)
    Y = host(ql.qlinear_gemm_nvfp4(nvfp4_dev(W), t(X)))
    torch.cuda.synchronize()
    assert np.array_equal(Y.view(np.uint16), ref.astype(np.float16).view(np.uint16))
