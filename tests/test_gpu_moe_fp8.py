"""GPU parity of the routed-expert layer with FP8-E4M3 experts (moe_route,
moe_grouped_gemm_fp8 for gate/up and down, moe_combine) against the
oracle's FP8 layer, with the fp16 bars of tests/gpu_util.py."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import host, say, t
from tests.test_gpu_moe import SCREENED, _compare

pytestmark = pytest.mark.gpu


def _fp8_dev(W):
    return {"codes": t(W["codes"]), "scales": t(W["scales"]), "K": int(W["K"]), "N": int(W["N"])}


def _dev_weights(w):
    return {"Wr": t(w["Wr"]), "gate_up": _fp8_dev(w["gate_up"]), "down": _fp8_dev(w["down"]),
            "shared_gate_up": _fp8_dev(w["shared_gate_up"]), "shared_down": _fp8_dev(w["shared_down"])}


def _run(dw, H, bias, topk, T, shared=True):
    route = ql.moe_route(H, dw["Wr"], bias, topk)
    act = ql.moe_grouped_gemm_fp8(dw["gate_up"], dw["shared_gate_up"] if shared else None, H, T, topk,
                                  ql.QL_OP_GATE_UP_SILU, route)
    ydown = ql.moe_grouped_gemm_fp8(dw["down"], dw["shared_down"] if shared else None, act, T, topk,
                                    ql.QL_OP_DOWN, route)
    out = ql.moe_combine(ydown, route["gates"], route["pos"], T, topk, shared)
    return route, act, ydown, out


def _check_routing(route, ref):
    assert np.array_equal(host(route["ids"]), ref["ids"])
    assert np.array_equal(host(route["counts"]), ref["counts"])
    assert np.array_equal(host(route["offsets"]), ref["offsets"])
    assert np.array_equal(host(route["sorted_assign"]), ref["sorted_assign"])
    assert np.array_equal(host(route["pos"]), ref["pos"])


@pytest.mark.parametrize("seed", SCREENED[:1])
def test_moe_fp8_prefill_4096(seed):
    """The prefill workload with FP8 experts: 4096 tokens, 256 experts +
    shared, Zipf logit bias.  The router weight is the w4 layer's (same
    weight seed), so the screened token seed routes without near ties."""
    import torch
    say(f"moe fp8 prefill T=4096 seed={seed}")
    w = synth.moe_weights_fp8(0)
    tok = synth.moe_tokens(seed, 4096, skewed=True)
    ref = oracle.moe_layer_fp8(tok["H"], w, tok["logit_bias"], 8)
    res = _run(_dev_weights(w), t(tok["H"]), t(tok["logit_bias"]), 8, 4096)
    torch.cuda.synchronize()
    _check_routing(res[0], ref)
    rel, mx = _compare(*res, ref, 4096, 8)
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("T,D,I,E,topk,seed,shared", [
    (1, 2048, 512, 256, 8, 0, True),     # one token on the tiled path
    (3, 512, 256, 16, 4, 1, True),
    (300, 256, 128, 16, 4, 3, True),     # MFMA router, ragged tiles
    (700, 512, 256, 64, 8, 7, True),     # tall and short tiles
    (200, 256, 64, 33, 5, 5, False),     # E % 8 != 0, no shared expert
    (70, 4096, 192, 8, 2, 6, True),      # long K, I not a multiple of 128
])
def test_moe_fp8_shapes(T, D, I, E, topk, seed, shared):
    import torch
    say(f"moe fp8 T={T} D={D} I={I} E={E} topk={topk} shared={shared}")
    w = synth.moe_weights_fp8(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 90, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer_fp8(tok["H"], w, tok["logit_bias"], topk, with_shared=shared)
    srt = -np.sort(-ref["logits"], axis=1)
    if topk < E:
        assert (srt[:, topk - 1] - srt[:, topk]).min() > 5e-5, "case not screened"
    res = _run(_dev_weights(w), t(tok["H"]), t(tok["logit_bias"]), topk, T, shared)
    torch.cuda.synchronize()
    _check_routing(res[0], ref)
    if shared:
        rel, mx = _compare(*res, ref, T, topk)
    else:
        from tests.gpu_util import assert_close
        assert_close(host(res[1]).astype(np.float64), ref["act"].astype(np.float64), "act")
        assert_close(host(res[2]).astype(np.float64), ref["ydown"], "ydown")
        rel, mx = assert_close(host(res[3]).astype(np.float64), ref["out"], "out")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_moe_fp8_integer_experts_bit_exact():
    """Expert codes of the integers -2..2 (exact in E4M3), scales 1/64 and
    inputs of small integers: every staged weight, product and fp32 sum of
    the down projection is exact, so its rows equal the oracle's rounded
    values bit for bit; the gate/up sums are exact too, and act (SiLU in
    fp32, then rounded) lies within one fp16 ulp of the oracle's."""
    import torch
    T, D, I, E, topk = 150, 256, 64, 8, 2
    rng = synth.rng_for(40)
    mags = np.array([0x00, 0x38, 0x40], dtype=np.uint8)

    def mat(lead, N, K):
        c = mags[rng.integers(0, 3, size=lead + (N, K))]
        c = c | (rng.integers(0, 2, size=lead + (N, K)) * 0x80).astype(np.uint8)
        return {"codes": c.astype(np.uint8), "scales": np.full(lead + (N, K // 64), 1 / 64, np.float16),
                "K": K, "N": N}

    w = {"Wr": synth.router_weight(rng, D, E), "gate_up": mat((E,), 2 * I, D), "down": mat((E,), D, I),
         "shared_gate_up": mat((), 2 * I, D), "shared_down": mat((), D, I)}
    H = rng.integers(-2, 3, size=(T, D)).astype(np.float16)
    Xi = rng.integers(-3, 4, size=(T * topk + T, I)).astype(np.float16)
    ref = oracle.moe_layer_fp8(H, w, None, topk)
    srt = -np.sort(-ref["logits"], axis=1)
    assert (srt[:, topk - 1] - srt[:, topk]).min() > 5e-5, "case not screened"
    dw = _dev_weights(w)
    route = ql.moe_route(t(H), dw["Wr"], None, topk)
    act = ql.moe_grouped_gemm_fp8(dw["gate_up"], dw["shared_gate_up"], t(H), T, topk,
                                  ql.QL_OP_GATE_UP_SILU, route)
    ydown = ql.moe_grouped_gemm_fp8(dw["down"], dw["shared_down"], t(Xi), T, topk, ql.QL_OP_DOWN, route)
    torch.cuda.synchronize()
    _check_routing(route, ref)
    ra = ref["act"].astype(np.float64)
    assert np.max(np.abs(host(act).astype(np.float64) - ra) / np.maximum(np.abs(ra), 2.0 ** -14)) <= 2.0 ** -10
    e_of_row = np.concatenate([np.repeat(np.arange(E), np.diff(ref["offsets"])), np.full(T, -1)])
    y = np.empty((T * topk + T, D))
    for e in range(-1, E):
        sel = e_of_row == e
        if not sel.any():
            continue
        W = w["shared_down"] if e < 0 else {"codes": w["down"]["codes"][e], "scales": w["down"]["scales"][e],
                                             "K": I, "N": D}
        y[sel] = oracle.linear_fp8(Xi[sel], W)
    assert np.array_equal(host(ydown).view(np.uint16), y.astype(np.float16).view(np.uint16))


def test_moe_fp8_down_combine_is_rejected():
    w = synth.moe_weights_fp8(0, D=256, I=64, E=8)
    dw = _dev_weights(w)
    tok = synth.moe_tokens(1, 2, D=256, E=8)
    route = ql.moe_route(t(tok["H"]), dw["Wr"], None, 2)
    with pytest.raises(ql.QLError):
        ql.moe_grouped_gemm_fp8(dw["down"], None, t(np.zeros((4, 64), np.float16)), 2, 2,
                                ql.QL_OP_DOWN_COMBINE, route)
