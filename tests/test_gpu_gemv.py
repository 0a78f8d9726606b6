"""GPU parity of qlinear_gemv (and qlinear_pack) against the oracle."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, guarded, host, say, t, w4_dev

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
    import torch
    say(f"gemv K={K} N={N} seed={seed}")
    case = synth.gemv_case(seed, K, N)
    ref = oracle.linear(case["x"], case["W"])[0]
    y = guarded(N, torch.float16)
    ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check(f"gemv K={K} N={N}")
    assert_close(host(y.t).astype(np.float64), ref, f"gemv K={K} N={N}")


def test_gemv_vocab_head_full():
    """K = 2048, N = 151552 (the vocabulary head, in the benchmark's launch
    configuration: 8 rows per lane): every output against the oracle."""
    import torch
    K, N = 2048, synth.VOCAB
    say(f"gemv head K={K} N={N}")
    case = synth.gemv_case(1, K, N)
    y = guarded(N, torch.float16)
    ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv head")
    ref = oracle.linear(case["x"], case["W"])[0]
    rel, mx = assert_close(host(y.t).astype(np.float64), ref, "gemv head")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("K,N,seed", [
    (2048, 40001, 13), (4096, 33001, 14), (1024, 65601, 15), (512, 131101, 16), (256, 262201, 17),
])
def test_gemv_eight_rows_ragged(K, N, seed):
    """Shapes that launch at least 1024 blocks, where each lane walks 8 rows,
    with N not a multiple of the rows per block: the ragged last block's
    clamped loads and its owner mask, at every K of the chunked kernel that
    has this instance."""
    import torch
    say(f"gemv 8-row K={K} N={N}")
    case = synth.gemv_case(seed, K, N)
    y = guarded(N, torch.float16)
    ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check(f"gemv K={K} N={N}")
    ref = oracle.linear(case["x"], case["W"])[0]
    assert_close(host(y.t).astype(np.float64), ref, f"gemv K={K} N={N}")


@pytest.mark.parametrize("scale", [1e-4, 3e-5])
@pytest.mark.parametrize("K,N", [(2048, 8192), (512, 512), (1024, 1000)])
def test_gemv_small_activations(K, N, scale):
    """Activations of order 1e-4 and 3e-5, many of them fp16 subnormals: the
    products must stay exact (no rescaled copy of x may lose bits)."""
    import torch
    say(f"gemv small x K={K} N={N} scale={scale}")
    case = synth.gemv_case(40, K, N, x_scale=scale)
    ref = oracle.linear(case["x"], case["W"])[0]
    y = guarded(N, torch.float16)
    ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv small x")
    rel, mx = assert_close(host(y.t).astype(np.float64), ref, f"gemv small x {scale}")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemv_subnormal_outputs():
    """K = 64 with activations of order 3e-5: the outputs lie in fp16's
    subnormal range, where rounding the exact result alone costs more than
    the 1e-3 bar (1.5e-3 rel-L2 here).  The GPU must then round the exact
    result itself: every output within one subnormal step (2**-24) of the
    oracle's rounded value, and almost all of them equal to it."""
    import torch
    K, N = 64, 4000
    case = synth.gemv_case(41, K, N, x_scale=3e-5)
    ref16 = oracle.round_f16(oracle.linear(case["x"], case["W"])[0])
    assert np.mean(np.abs(ref16.astype(np.float64)) < 2.0**-14) > 0.9
    y = guarded(N, torch.float16)
    ql.qlinear_gemv(w4_dev(case["W"]), t(case["x"][0]), y=y.t)
    torch.cuda.synchronize()
    y.check("gemv subnormal outputs")
    g = host(y.t)
    diff = np.abs(g.astype(np.float64) - ref16.astype(np.float64))
    assert diff.max() <= 2.0**-24
    assert np.mean(g.view(np.uint16) == ref16.view(np.uint16)) > 0.99


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


@pytest.mark.parametrize("K,Ns,seed", [
    (2048, (8192, synth.VOCAB), 20),        # the decode step's projection and vocabulary head
    (512, (512, 100, 0, 7), 21),            # a skipped empty matrix, ragged N, fallback rows
    (8192, (1000, 33), 22),                 # fixed rows per wave
    (1024, (64,) * 8, 23),                  # QL_GEMV_MULTI_MAX matrices
])
def test_gemv_multi_matches_separate_calls(K, Ns, seed):
    """qlinear_gemv_multi: every output has the bits of qlinear_gemv on its
    matrix (same x), the guard regions stay intact, and the matrices that
    the oracle finishes quickly match it."""
    import torch
    say(f"gemv multi K={K} Ns={Ns}")
    cases = [synth.gemv_case(seed + 100 * i, K, N) if N > 0 else None for i, N in enumerate(Ns)]
    x = synth.gemv_case(seed, K, 1)["x"]
    Ws = [w4_dev(c["W"]) if c is not None else
          {"qweight": torch.empty(0, dtype=torch.int32, device="cuda"),
           "scales": torch.empty(0, dtype=torch.int16, device="cuda"),
           "biases": torch.empty(0, dtype=torch.int16, device="cuda"), "K": K, "N": 0} for c in cases]
    ys = [guarded(max(N, 1), torch.float16) for N in Ns]
    ql.qlinear_gemv_multi(Ws, t(x[0]), [y.t[:N] for y, N in zip(ys, Ns)])
    torch.cuda.synchronize()
    for i, (N, y) in enumerate(zip(Ns, ys)):
        y.check(f"multi matrix {i}")
        if N == 0:
            continue
        ref = torch.empty(N, dtype=torch.float16, device="cuda")
        ql.qlinear_gemv(Ws[i], t(x[0]), ref)
        torch.cuda.synchronize()
        assert np.array_equal(host(y.t[:N]).view(np.uint16), host(ref).view(np.uint16)), f"matrix {i}"
        if N * K <= 8192 * 2048:
            assert_close(host(y.t[:N]).astype(np.float64), oracle.linear(x, cases[i]["W"])[0], f"matrix {i}")
