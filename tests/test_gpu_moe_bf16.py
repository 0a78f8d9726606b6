"""GPU parity of the bf16 routed-expert layer (moe_route_bf16,
moe_grouped_gemm_bf16, moe_combine_bf16) against the oracle's bf16 layer,
with the bf16 layer tolerance derived in tests/gpu_util.py."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import (MAX_ABS_FRAC_BF16_MOE, REL_L2_BF16_MOE, assert_close_bf16, host, say,
                            t)

pytestmark = pytest.mark.gpu


def _w4_dev_bits(W):
    return {"qweight": t(W["qweight"]), "scales": t(W["scales"]), "biases": t(W["biases"]),
            "K": int(W["K"]), "N": int(W["N"])}


def _dev_weights(w):
    return {"Wr": t(w["Wr"]), "gate_up": _w4_dev_bits(w["gate_up"]), "down": _w4_dev_bits(w["down"]),
            "shared_gate_up": _w4_dev_bits(w["shared_gate_up"]),
            "shared_down": _w4_dev_bits(w["shared_down"])}


def _bits(x):
    import torch
    return x.view(torch.int16).cpu().numpy().view(np.uint16)


def _run(dw, H, bias, topk, T, shared=True):
    route = ql.moe_route_bf16(H, dw["Wr"], bias, topk)
    act = ql.moe_grouped_gemm_bf16(dw["gate_up"], dw["shared_gate_up"] if shared else None, H, T, topk,
                                   ql.QL_OP_GATE_UP_SILU, route)
    ydown = ql.moe_grouped_gemm_bf16(dw["down"], dw["shared_down"] if shared else None, act, T, topk,
                                     ql.QL_OP_DOWN, route)
    out = ql.moe_combine_bf16(ydown, route["gates"], route["pos"], T, topk, shared)
    return route, act, ydown, out


def _check(route, act, ydown, out, ref, T, topk):
    """Routing exactly the oracle's (the cases are screened: no token's k-th
    and (k+1)-th logits lie within 30 times the fp32 logit error), the
    integer steps bit for bit, then act, ydown and out within the bf16 bar."""
    assert np.array_equal(host(route["ids"]), ref["ids"])
    assert np.abs(host(route["gates"]).astype(np.float64) - ref["gates"]).max() < 2e-5
    assert np.array_equal(host(route["counts"]), ref["counts"])
    assert np.array_equal(host(route["offsets"]), ref["offsets"])
    assert np.array_equal(host(route["sorted_assign"]), ref["sorted_assign"])
    assert np.array_equal(host(route["pos"]), ref["pos"])
    bar = dict(rel_l2=REL_L2_BF16_MOE, max_abs_frac=MAX_ABS_FRAC_BF16_MOE)
    assert_close_bf16(_bits(act), oracle.bf16_to_f64(ref["act"]), "act", **bar)
    assert_close_bf16(_bits(ydown), ref["ydown"], "ydown", **bar)
    return assert_close_bf16(_bits(out), ref["out"], "out", **bar)


def test_moe_bf16_prefill_4096():
    """The prefill workload in bf16: 4096 tokens, 256 experts + shared, Zipf
    logit bias; token seed 4 (smallest k/k+1 logit gap 5.5e-5 against an
    fp32 logit error of 1.4e-6)."""
    import torch
    say("moe bf16 prefill T=4096")
    w = synth.moe_weights_bf16(0)
    tok = synth.moe_tokens_bf16(4, 4096, skewed=True)
    ref = oracle.moe_layer_bf16(tok["H"], w, tok["logit_bias"], 8)
    dw = _dev_weights(w)
    res = _run(dw, t(tok["H"]), t(tok["logit_bias"]), 8, 4096)
    torch.cuda.synchronize()
    rel, mx = _check(*res, ref, 4096, 8)
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("T,D,I,E,topk,seed,shared", [
    (1, 2048, 512, 256, 8, 0, True),     # one token on the tiled path
    (3, 512, 256, 16, 4, 1, True),
    (16, 512, 128, 16, 4, 2, True),      # largest T of the one-block router
    (300, 256, 128, 16, 4, 3, True),     # MFMA router, ragged tiles
    (700, 512, 256, 64, 8, 7, True),
    (200, 256, 64, 33, 5, 5, False),     # E % 8 != 0, no shared expert
])
def test_moe_bf16_shapes(T, D, I, E, topk, seed, shared):
    import torch
    say(f"moe bf16 T={T} D={D} I={I} E={E} topk={topk} shared={shared}")
    w = synth.moe_weights_bf16(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens_bf16(seed + 70, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer_bf16(tok["H"], w, tok["logit_bias"], topk, with_shared=shared)
    srt = -np.sort(-ref["logits"], axis=1)
    if topk < E:
        assert (srt[:, topk - 1] - srt[:, topk]).min() > 5e-5, "case not screened"
    dw = _dev_weights(w)
    res = _run(dw, t(tok["H"]), t(tok["logit_bias"]), topk, T, shared)
    torch.cuda.synchronize()
    rel, mx = _check(*res, ref, T, topk)
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_moe_bf16_down_combine_is_rejected():
    w = synth.moe_weights_bf16(0, D=256, I=64, E=8)
    dw = _dev_weights(w)
    tok = synth.moe_tokens_bf16(1, 2, D=256, E=8)
    route = ql.moe_route_bf16(t(tok["H"]), dw["Wr"], None, 2)
    with pytest.raises(ql.QLError):
        ql.moe_grouped_gemm_bf16(dw["down"], None, t(np.zeros((4, 64), np.uint16)), 2, 2,
                                 ql.QL_OP_DOWN_COMBINE, route)


@pytest.mark.parametrize("T,D,I,E,topk,seed,shared", [
    (1, 2048, 512, 256, 8, 0, True),     # the decode shape
    (1, 2048, 512, 256, 8, 1, True),
    (4, 2048, 512, 256, 8, 2, True),
    (3, 512, 256, 16, 1, 3, True),
    (2, 512, 128, 1000, 32, 4, True),    # 16 keys per lane in the top-k
    (3, 256, 64, 33, 5, 5, False),       # scalar router partials, no shared expert
])
def test_moe_decode_bf16(T, D, I, E, topk, seed, shared):
    """moe_decode_bf16 (routing fused into the bf16 gate/up rows) against
    the oracle's bf16 layer."""
    import torch
    say(f"moe_decode_bf16 T={T} D={D} I={I} E={E} topk={topk} shared={shared}")
    w = synth.moe_weights_bf16(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens_bf16(seed + 80, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer_bf16(tok["H"], w, tok["logit_bias"], topk, with_shared=shared)
    srt = -np.sort(-ref["logits"], axis=1)
    assert (srt[:, topk - 1] - srt[:, topk]).min() > 5e-5, "case not screened"
    dw = _dev_weights(w)
    res = ql.moe_decode(t(tok["H"]), dw["Wr"], t(tok["logit_bias"]), topk, dw["gate_up"], dw["down"],
                        dw["shared_gate_up"] if shared else None, dw["shared_down"] if shared else None,
                        bf16=True)
    torch.cuda.synchronize()
    assert np.array_equal(host(res["ids"]), ref["ids"])
    assert np.abs(host(res["gates"]).astype(np.float64) - ref["gates"]).max() < 2e-5
    rel, mx = assert_close_bf16(_bits(res["out"]), ref["out"], "out", rel_l2=REL_L2_BF16_MOE,
                                max_abs_frac=MAX_ABS_FRAC_BF16_MOE)
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("D,I", [(2048, 512), (512, 1024)])
def test_moe_bf16_tile_row_boundaries(D, I):
    """The bf16 grouped GEMMs on experts with 1, 31, 32, 33, 0, 97, 256 and
    300 rows (moe_dispatch on given ids, topk 1) and the shared expert, at
    K = 2048 / 512 and 512 / 1024: every act and ydown row against the
    oracle's bf16 FFN of its own expert."""
    import torch
    from tests.test_gpu_moe import BOUNDARY_COUNTS, boundary_route, expert_rows_reference
    E = len(BOUNDARY_COUNTS)
    say(f"moe bf16 tile boundaries D={D} I={I}")
    ids = boundary_route(E, BOUNDARY_COUNTS, D + I + 5)
    T = ids.shape[0]
    w = synth.moe_weights_bf16(D + I, D=D, I=I, E=E)
    H = synth.moe_tokens_bf16(D + I + 1, T, D=D, E=E)["H"]
    dw = _dev_weights(w)
    route = ql.moe_dispatch(t(ids), E)
    act = ql.moe_grouped_gemm_bf16(dw["gate_up"], dw["shared_gate_up"], t(H), T, 1, ql.QL_OP_GATE_UP_SILU, route)
    yd = ql.moe_grouped_gemm_bf16(dw["down"], dw["shared_down"], act, T, 1, ql.QL_OP_DOWN, route)
    torch.cuda.synchronize()
    ref_act, ref_yd = expert_rows_reference(ids, host(route["sorted_assign"]), H, w, oracle.expert_ffn_bf16)
    bar = dict(rel_l2=REL_L2_BF16_MOE, max_abs_frac=MAX_ABS_FRAC_BF16_MOE)
    assert_close_bf16(_bits(act), oracle.bf16_to_f64(ref_act), "act", **bar)
    assert_close_bf16(_bits(yd), ref_yd, "ydown", **bar)


@pytest.mark.parametrize("T", [600, 4096])
def test_moe_bf16_shared_expert_split(T):
    """The bf16 routed rows (shared = None) and the shared expert's rows
    (QL_OP_SHARED_ONLY) as two launches into one buffer, the shared ones on
    a second stream: act and ydown equal the single launch's bit for bit."""
    import torch
    topk = 8
    say(f"bf16 shared-expert split T={T}")
    w = synth.moe_weights_bf16(0)
    dw = _dev_weights(w)
    tk = synth.moe_tokens_bf16(4, T, skewed=True)
    H, b = t(tk["H"]), t(tk["logit_bias"])
    route, act, yd, _ = _run(dw, H, b, topk, T, shared=True)
    torch.cuda.synchronize()
    act2 = torch.zeros_like(act)
    yd2 = torch.zeros_like(yd)
    side = torch.cuda.Stream()
    fork = torch.cuda.Event()
    fork.record(torch.cuda.current_stream())
    side.wait_event(fork)
    with torch.cuda.stream(side):
        ql.moe_grouped_gemm_bf16(dw["gate_up"], dw["shared_gate_up"], H, T, topk,
                                 ql.QL_OP_GATE_UP_SILU | ql.QL_OP_SHARED_ONLY, None, act2, stream=side)
        ql.moe_grouped_gemm_bf16(dw["down"], dw["shared_down"], act, T, topk,
                                 ql.QL_OP_DOWN | ql.QL_OP_SHARED_ONLY, None, yd2, stream=side)
    ql.moe_grouped_gemm_bf16(dw["gate_up"], None, H, T, topk, ql.QL_OP_GATE_UP_SILU, route, act2)
    ql.moe_grouped_gemm_bf16(dw["down"], None, act, T, topk, ql.QL_OP_DOWN, route, yd2)
    torch.cuda.synchronize()
    assert np.array_equal(_bits(act2), _bits(act))
    assert np.array_equal(_bits(yd2), _bits(yd))
