"""GPU parity of the decode steps beside the single-row linear layer:
RMSNorm-fused projection, vocabulary head with on-GPU token choice, and the
embedding row of a token held in device memory."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, guarded, host, say, t, w4_dev

pytestmark = pytest.mark.gpu

EPS = 1e-6
# The token is decided on fp32 logits; they differ from the oracle's float64
# logits by fp32 rounding of the K-long sums (about 1e-6 of max|logit| at
# K = 16384), so a decision is only pinned to one id when the oracle's two
# best logits are further apart than this.
ARGMAX_TOL_FRAC = 1e-4


@pytest.mark.parametrize("K,N,seed", [
    (2048, 8192, 0), (2048, 8192, 1),               # fused QKV/gate-sized projection
    (256, 100, 2), (512, 513, 3), (1024, 1000, 4),  # every chunked K, ragged N
    (4096, 257, 5), (8192, 65, 6), (16384, 33, 7), (2048, 1, 8),
])
def test_gemv_rmsnorm_matches_oracle(K, N, seed):
    import torch
    say(f"gemv_rmsnorm K={K} N={N} seed={seed}")
    c = synth.decode_norm_case(seed, K, N)
    ref, _ = oracle.gemv_rmsnorm(c["x"][0], c["gamma"], EPS, c["W"])
    y = ql.qlinear_gemv_rmsnorm(w4_dev(c["W"]), t(c["x"][0]), t(c["gamma"]), EPS)
    torch.cuda.synchronize()
    assert_close(host(y).astype(np.float64), ref, f"gemv_rmsnorm K={K} N={N}")


def test_gemv_rmsnorm_scale_invariance_and_eps():
    """With eps = 0 the normalized row does not depend on the scale of x:
    x and 4x give the same bits (a power-of-four scale passes exactly
    through the squares, the mean, the root and the products).  A large
    eps shrinks the output as the oracle says."""
    import torch
    K, N = 2048, 512
    c = synth.decode_norm_case(11, K, N)
    W = w4_dev(c["W"])
    g = t(c["gamma"])
    y1 = host(ql.qlinear_gemv_rmsnorm(W, t(c["x"][0]), g, 0.0))
    y2 = host(ql.qlinear_gemv_rmsnorm(W, t((c["x"][0].astype(np.float64) * 4).astype(np.float16)), g, 0.0))
    big = 50.0
    y3 = host(ql.qlinear_gemv_rmsnorm(W, t(c["x"][0]), g, big)).astype(np.float64)
    torch.cuda.synchronize()
    assert np.array_equal(y1.view(np.uint16), y2.view(np.uint16))
    ref3, _ = oracle.gemv_rmsnorm(c["x"][0], c["gamma"], big, c["W"])
    assert_close(y3, ref3, "gemv_rmsnorm eps=50")


def _check_token(tok, logits_ref, what):
    """tok must be the oracle's id when the two best oracle logits are
    further apart than the fp32 error bound, else one within the bound."""
    order = np.argsort(-logits_ref, kind="stable")
    best, second = logits_ref[order[0]], logits_ref[order[1]] if logits_ref.size > 1 else -np.inf
    tol = ARGMAX_TOL_FRAC * max(np.abs(logits_ref).max(), 1e-30)
    assert 0 <= tok < logits_ref.size, f"{what}: token {tok} out of range"
    if best - second > tol:
        assert tok == oracle.argmax_first(logits_ref), f"{what}: token {tok} != {order[0]}"
    else:
        assert logits_ref[tok] >= best - tol, f"{what}: token {tok} not within {tol} of the max"


@pytest.mark.parametrize("K,N,seed", [
    (2048, 8192, 0), (256, 1, 1), (512, 37, 2), (1024, 1000, 3),
    (4096, 4097, 4), (8192, 300, 5), (16384, 129, 6),
])
def test_gemv_argmax_matches_oracle(K, N, seed):
    import torch
    say(f"gemv_argmax K={K} N={N} seed={seed}")
    c = synth.gemv_case(seed, K, N)
    tok_ref, logits_ref = oracle.lm_head_token(c["x"][0], c["W"])
    logits = torch.empty(N, dtype=torch.float16, device="cuda")
    tok = ql.qlinear_gemv_argmax(w4_dev(c["W"]), t(c["x"][0]), logits=logits)
    torch.cuda.synchronize()
    _check_token(int(host(tok)[0]), logits_ref, f"argmax K={K} N={N}")
    assert_close(host(logits).astype(np.float64), logits_ref, f"argmax logits K={K} N={N}")


def test_gemv_argmax_vocab_head():
    """The vocabulary head at its full size (K = 2048, N = 151552), in the
    launch configuration the benchmark times; every logit from the oracle."""
    import torch
    K, N = 2048, synth.VOCAB
    say(f"gemv_argmax head K={K} N={N}")
    c = synth.gemv_case(1, K, N)
    tok_ref, logits_ref = oracle.lm_head_token(c["x"][0], c["W"])
    logits = guarded(N, torch.float16)
    tok = ql.qlinear_gemv_argmax(w4_dev(c["W"]), t(c["x"][0]), logits=logits.t)
    torch.cuda.synchronize()
    logits.check("argmax head logits")
    _check_token(int(host(tok)[0]), logits_ref, "argmax head")
    rel, mx = assert_close(host(logits.t).astype(np.float64), logits_ref, "argmax head logits")
    say(f"  logits rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_gemv_argmax_ties_and_nan():
    """Equal largest logits pick the lower id (identical weight rows give
    bit-identical fp32 logits); a NaN logit is never chosen."""
    import torch
    K, N = 2048, 3000
    c = synth.gemv_case(21, K, N)
    W = {k: (v.copy() if isinstance(v, np.ndarray) else v) for k, v in c["W"].items()}
    _, logits_ref = oracle.lm_head_token(c["x"][0], W)
    top = oracle.argmax_first(logits_ref)
    lo, hi = 17, 2999                      # the tie: rows lo < hi both copy row `top`, scaled up
    for r in (lo, hi):
        W["qweight"][r] = W["qweight"][top]
        W["scales"][r] = (W["scales"][top].astype(np.float64) * 2).astype(np.float16)
        W["biases"][r] = (W["biases"][top].astype(np.float64) * 2).astype(np.float16)
    nanrow = 5
    W["scales"][nanrow, 0] = np.float16(np.nan)
    lref = oracle.linear(c["x"], W)[0]
    assert np.isnan(lref[nanrow]) and not np.isnan(np.delete(lref, nanrow)).any()
    tok_ref = oracle.argmax_first(np.where(np.isnan(lref), -np.inf, lref))
    assert tok_ref == lo
    tok = ql.qlinear_gemv_argmax(w4_dev(W), t(c["x"][0]))
    torch.cuda.synchronize()
    assert int(host(tok)[0]) == lo


def test_embed_token_bit_exact():
    import torch
    K, N = 2048, 5000
    rng = synth.rng_for(31)
    E = synth.w4_matrix(rng, K, N)
    Ed = w4_dev(E)
    slot = torch.empty(1, dtype=torch.int32, device="cuda")
    for tok in (0, 1, 2499, N - 1):
        slot.fill_(tok)
        x = host(ql.qlinear_embed_token(Ed, slot))
        torch.cuda.synchronize()
        assert np.array_equal(x.view(np.uint16), oracle.embed_row(E, tok).view(np.uint16)), tok
    for bad in (-1, N, 2**31 - 1):
        slot.fill_(bad)
        x = host(ql.qlinear_embed_token(Ed, slot))
        torch.cuda.synchronize()
        assert not np.any(x.view(np.uint16)), bad


def test_token_handoff_graph_two_slots():
    """Decode steps chained on the GPU only: token = argmax(x . W_head), then
    x = embedding row of that token, with two alternating token slots,
    captured once in a HIP graph and replayed; every replay's tokens and
    rows are checked against the oracle's chain."""
    import torch
    K, V, steps = 2048, 4096, 4
    rng = synth.rng_for(41)
    Wh = synth.w4_matrix(rng, K, V)
    E = synth.w4_matrix(rng, K, V)
    x0 = synth.activations(rng, 1, K)[0]
    # the oracle's chain; every decision clears the fp32 bound ten times
    # over, so the GPU has to reproduce every id exactly
    toks, rows, x = [], [], x0
    for _ in range(steps):
        tok, logits = oracle.lm_head_token(x, Wh)
        srt = np.sort(logits)
        assert srt[-1] - srt[-2] > 10 * ARGMAX_TOL_FRAC * np.abs(logits).max(), "seed gives a near tie"
        x = oracle.embed_row(E, tok)
        toks.append(tok)
        rows.append(x)
    Whd, Ed = w4_dev(Wh), w4_dev(E)
    xbuf = [t(x0), torch.empty(K, dtype=torch.float16, device="cuda")]
    slots = torch.full((2,), -7, dtype=torch.int32, device="cuda")
    ws = ql.gemv_argmax_workspace(V, "cuda")
    xs = [torch.empty(K, dtype=torch.float16, device="cuda") for _ in range(steps)]
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            cur = xbuf[0]
            for i in range(steps):
                slot = slots[i % 2:i % 2 + 1]
                ql.qlinear_gemv_argmax(Whd, cur, token=slot, workspace=ws)
                ql.qlinear_embed_token(Ed, slot, xs[i])
                cur = xs[i]
    for rep in range(3):
        for b in xs:
            b.fill_(7.0)            # eager work between replays
        slots.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            assert np.array_equal(host(xs[i]).view(np.uint16), rows[i].view(np.uint16)), (rep, i)
        assert host(slots).tolist() == [toks[steps - 2], toks[steps - 1]], rep
