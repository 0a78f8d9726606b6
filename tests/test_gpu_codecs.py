"""GPU parity of the second weight codecs (FP8-E4M3 and NVFP4 single-row
GEMV) against the oracle, at the fp16 output tolerance."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, assert_close_nan, guarded, host, say, t

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
def test_codec_vocab_head_full(codec):
    """K = 2048, N = 151552 in the benchmark's launch configuration: every
    output against the oracle, behind guard regions."""
    import torch
    K, N = 2048, synth.VOCAB
    say(f"gemv_{codec} head")
    rng = synth.rng_for(11)
    x = synth.activations(rng, 1, K)
    y = guarded(N, torch.float16)
    if codec == "fp8":
        W = synth.fp8_matrix(rng, K, N)
        ql.qlinear_gemv_fp8(fp8_dev(W), t(x[0]), y=y.t)
    else:
        W = synth.nvfp4_matrix(rng, K, N)
        ql.qlinear_gemv_nvfp4(nvfp4_dev(W), t(x[0]), y=y.t)
    torch.cuda.synchronize()
    y.check(f"gemv_{codec} head")
    ref = oracle.linear_fp8(x, W)[0] if codec == "fp8" else oracle.linear_nvfp4(x, W)[0]
    rel, mx = assert_close(host(y.t).astype(np.float64), ref, f"gemv_{codec} head")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("codec,K,N,seed", [
    ("fp8", 2048, 40001, 13), ("fp8", 1024, 65601, 14), ("fp8", 4096, 33001, 15),
    ("nvfp4", 2048, 40001, 16), ("nvfp4", 1024, 65601, 17), ("nvfp4", 4096, 33001, 18),
])
def test_codec_gemv_eight_rows_ragged(codec, K, N, seed):
    """The 8-rows-per-lane instances with a ragged last block."""
    import torch
    say(f"gemv_{codec} 8-row K={K} N={N}")
    rng = synth.rng_for(seed)
    x = synth.activations(rng, 1, K)
    y = guarded(N, torch.float16)
    if codec == "fp8":
        W = synth.fp8_matrix(rng, K, N)
        ql.qlinear_gemv_fp8(fp8_dev(W), t(x[0]), y=y.t)
        ref = oracle.linear_fp8(x, W)[0]
    else:
        W = synth.nvfp4_matrix(rng, K, N)
        ql.qlinear_gemv_nvfp4(nvfp4_dev(W), t(x[0]), y=y.t)
        ref = oracle.linear_nvfp4(x, W)[0]
    torch.cuda.synchronize()
    y.check(f"gemv_{codec}")
    assert_close(host(y.t).astype(np.float64), ref, f"gemv_{codec} K={K} N={N}")


@pytest.mark.parametrize("K,N,seed", [(256, 4096, 40), (512, 2000, 41), (2048, 300, 42)])
def test_gemv_fp8_all_codes_nan_aware(K, N, seed):
    """Codes drawn over all 256 bytes, the two NaN codes included: a row
    holding a NaN code gives NaN, as in the oracle, and every other row is
    within the bar.  Rows 0..N/2 draw from all codes, the rest from the
    number codes only, so both kinds of rows are present at every K."""
    import torch
    say(f"gemv_fp8 all codes K={K} N={N}")
    rng = synth.rng_for(seed)
    x = synth.activations(rng, 1, K)
    Wa = synth.fp8_matrix(rng, K, N // 2, all_codes=True)
    Wf = synth.fp8_matrix(rng, K, N - N // 2)
    W = {"codes": np.concatenate([Wa["codes"], Wf["codes"]]),
         "scales": np.concatenate([Wa["scales"], Wf["scales"]]), "K": K, "N": N}
    ref = oracle.linear_fp8(x, W)[0]
    y = guarded(N, torch.float16)
    ql.qlinear_gemv_fp8(fp8_dev(W), t(x[0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv_fp8 all codes")
    n_nan = assert_close_nan(host(y.t), ref, "gemv_fp8 all codes")
    say(f"  NaN rows {n_nan} of {N}")
    assert 0 < n_nan < N


@pytest.mark.parametrize("K,N,seed", [(256, 3000, 43), (2048, 700, 44)])
def test_gemv_nvfp4_all_block_scales_nan_aware(K, N, seed):
    """E4M3 block scales over all 256 bytes (negative, subnormal, 448, NaN):
    rows with a NaN block scale give NaN, the others are within the bar."""
    import torch
    say(f"gemv_nvfp4 all block scales K={K} N={N}")
    rng = synth.rng_for(seed)
    x = synth.activations(rng, 1, K)
    W = synth.nvfp4_matrix(rng, K, N, all_codes=True)
    ref = oracle.linear_nvfp4(x, W)[0]
    y = guarded(N, torch.float16)
    ql.qlinear_gemv_nvfp4(nvfp4_dev(W), t(x[0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv_nvfp4 all codes")
    n_nan = assert_close_nan(host(y.t), ref, "gemv_nvfp4 all block scales")
    say(f"  NaN rows {n_nan} of {N}")
    assert 0 < n_nan < N


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


def test_gemm_fp8_prefill_full_and_row_invariance():
    """The prefill shape (M = 4096, K = 2048, N = 8192): every output against
    the oracle, behind guard regions, and every row's bits equal to the same
    row computed with M = 1 and M = 256 (no split over K, the same K
    order)."""
    import torch
    M, K, N = 4096, 2048, 8192
    rng = synth.rng_for(20)
    X = synth.activations(rng, M, K)
    W = synth.fp8_matrix(rng, K, N)
    Wd, Xd = fp8_dev(W), t(X)
    Yg = guarded((M, N), torch.float16)
    ql.qlinear_gemm_fp8(Wd, Xd, Yg.t)
    torch.cuda.synchronize()
    Yg.check("gemm_fp8 prefill")
    Y = host(Yg.t)
    rel, mx = assert_close(Y.astype(np.float64), oracle.linear_fp8(X, W), "gemm_fp8 prefill")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")
    for m in (0, 255, 4095):
        for MM in (1, 256):
            lo = min(m, M - MM)
            part = host(ql.qlinear_gemm_fp8(Wd, Xd[lo:lo + MM].contiguous()))
            assert np.array_equal(part[m - lo].view(np.uint16), Y[m].view(np.uint16)), (m, MM)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K,N,seed", [(100, 64, 300, 50), (300, 256, 520, 51)])
def test_gemm_fp8_all_codes_nan_aware(M, K, N, seed):
    """FP8 codes over all 256 bytes in the first half of the columns (a
    column holding a NaN code is NaN in every row, as in the oracle), number
    codes only in the rest."""
    import torch
    say(f"gemm_fp8 all codes M={M} K={K} N={N}")
    rng = synth.rng_for(seed)
    X = synth.activations(rng, M, K)
    Wa = synth.fp8_matrix(rng, K, N // 2, all_codes=True)
    Wf = synth.fp8_matrix(rng, K, N - N // 2)
    W = {"codes": np.concatenate([Wa["codes"], Wf["codes"]]),
         "scales": np.concatenate([Wa["scales"], Wf["scales"]]), "K": K, "N": N}
    ref = oracle.linear_fp8(X, W)
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm_fp8(fp8_dev(W), t(X), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm_fp8 all codes")
    n_nan = assert_close_nan(host(Y.t), ref, "gemm_fp8 all codes")
    say(f"  NaN outputs {n_nan} of {M * N}")
    assert 0 < n_nan < M * N


@pytest.mark.parametrize("lo,hi", [(200.0, 400.0), (4000.0, 30000.0)])
def test_gemm_fp8_large_scales(lo, hi):
    """Group scales near the top of the fp16 range (up to 30000), with codes
    of magnitude at most 2 (|e4m3 * scale| <= 60000, inside fp16): the staged
    weight is fp16(e4m3 * scale) with no intermediate overflow, so the output
    is within the bar."""
    import torch
    M, K, N = 200, 512, 384
    say(f"gemm_fp8 scales U({lo}, {hi})")
    rng = synth.rng_for(52)
    X = synth.f16(1e-4 * rng.standard_normal((M, K)))
    W = synth.fp8_matrix(rng, K, N, scale_range=(lo, hi))
    # keep |e4m3| <= 2: codes of larger magnitude become sign | 1.mmm (0x38 | m)
    c = W["codes"]
    W["codes"] = np.where((c & 0x7F) > 0x40, (c & 0x80) | 0x38 | (c & 0x07), c).astype(np.uint8)
    ref = oracle.linear_fp8(X, W)
    assert np.abs(oracle.dequantize_fp8(W["codes"], W["scales"])).max() < 65504
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm_fp8(fp8_dev(W), t(X), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm_fp8 large scales")
    rel, mx = assert_close(host(Y.t).astype(np.float64), ref, "gemm_fp8 large scales")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


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


def test_gemm_nvfp4_prefill_full_and_row_invariance():
    """M = 4096, K = 2048, N = 8192: every output against the oracle behind
    guard regions, and rows bit-identical across M."""
    import torch
    M, K, N = 4096, 2048, 8192
    rng = synth.rng_for(22)
    X = synth.activations(rng, M, K)
    W = synth.nvfp4_matrix(rng, K, N)
    Wd, Xd = nvfp4_dev(W), t(X)
    Yg = guarded((M, N), torch.float16)
    ql.qlinear_gemm_nvfp4(Wd, Xd, Yg.t)
    torch.cuda.synchronize()
    Yg.check("gemm_nvfp4 prefill")
    Y = host(Yg.t)
    rel, mx = assert_close(Y.astype(np.float64), oracle.linear_nvfp4(X, W), "gemm_nvfp4 prefill")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")
    for m in (0, 255, 4095):
        for MM in (1, 256):
            lo = min(m, M - MM)
            part = host(ql.qlinear_gemm_nvfp4(Wd, Xd[lo:lo + MM].contiguous()))
            assert np.array_equal(part[m - lo].view(np.uint16), Y[m].view(np.uint16)), (m, MM)
    torch.cuda.synchronize()


@pytest.mark.parametrize("M,K,N,seed", [(100, 64, 300, 53), (300, 256, 520, 54)])
def test_gemm_nvfp4_all_block_scales_nan_aware(M, K, N, seed):
    """E4M3 block scales over all 256 bytes: columns with a NaN block scale
    are NaN in every row, the rest within the bar."""
    import torch
    say(f"gemm_nvfp4 all block scales M={M} K={K} N={N}")
    rng = synth.rng_for(seed)
    X = synth.activations(rng, M, K)
    W = synth.nvfp4_matrix(rng, K, N, all_codes=True)
    ref = oracle.linear_nvfp4(X, W)
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm_nvfp4(nvfp4_dev(W), t(X), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm_nvfp4 all block scales")
    n_nan = assert_close_nan(host(Y.t), ref, "gemm_nvfp4 all block scales")
    say(f"  NaN outputs {n_nan} of {M * N}")
    assert 0 < n_nan < M * N


def test_gemm_nvfp4_large_global_scale():
    """A global scale of 10000 with block scales 0.25 .. 7.5: block scales up
    to 75000, above fp16's largest value, with E2M1 codes of magnitude 0 and
    0.5 only, so every weight (at most 37500) is representable.  The block
    scale and the product are formed in fp32 and rounded once, so the
    output is within the bar."""
    import torch
    M, K, N = 200, 512, 384
    rng = synth.rng_for(55)
    X = synth.f16(1e-4 * rng.standard_normal((M, K)))
    W = synth.nvfp4_matrix(rng, K, N, global_scale=10000.0)
    W["qweight"] = (W["qweight"] & np.uint32(0x99999999)).astype(np.uint32)  # sign and 0 / 0.5
    bs = oracle.e4m3_to_f64(W["block_scales"]) * float(W["global_scale"])
    assert bs.max() > 65504
    assert np.abs(oracle.dequantize_nvfp4(W["qweight"], W["block_scales"], W["global_scale"], K)).max() < 65504
    ref = oracle.linear_nvfp4(X, W)
    Y = guarded((M, N), torch.float16)
    ql.qlinear_gemm_nvfp4(nvfp4_dev(W), t(X), Y.t)
    torch.cuda.synchronize()
    Y.check("gemm_nvfp4 large global")
    rel, mx = assert_close(host(Y.t).astype(np.float64), ref, "gemm_nvfp4 large global scale")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


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
