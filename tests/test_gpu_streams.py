"""Stream ordering: every entry point works on the caller's stream only.
The prefill MoE sequence, a GEMM and the GEMVs run on a side stream while
unrelated work keeps the default stream busy; the results must equal, bit
for bit, the same calls made on the default stream."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import synth
from tests.gpu_util import host, say, t, w4_dev

pytestmark = pytest.mark.gpu


def _run(dw, H, bias, gemm_w, X, gemv_w, x, stream):
    T, topk = H.shape[0], 8
    route = ql.moe_route(H, dw["Wr"], bias, topk, stream=stream)
    act = ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk, ql.QL_OP_GATE_UP_SILU, route,
                              stream=stream)
    yd = ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk, ql.QL_OP_DOWN, route, stream=stream)
    out = ql.moe_combine(yd, route["gates"], route["pos"], T, topk, True, stream=stream)
    Y = ql.qlinear_gemm(gemm_w, X, stream=stream)
    y = ql.qlinear_gemv(gemv_w, x, stream=stream)
    return [route["ids"], route["sorted_assign"], act, yd, out, Y, y]


def test_side_stream_matches_default_stream():
    import torch
    say("streams: MoE T=700, GEMM 1000x2048x3000, GEMV 2048x8192 on a side stream")
    w = synth.moe_weights(7, D=512, I=256, E=64)
    tok = synth.moe_tokens(97, 700, D=512, E=64, skewed=True)
    dw = {"Wr": t(w["Wr"])}
    for k in ("gate_up", "down", "shared_gate_up", "shared_down"):
        dw[k] = w4_dev(w[k])
    H, bias = t(tok["H"]), t(tok["logit_bias"])
    g = synth.gemm_case(3, 1000, 2048, 3000)
    gemm_w, X = w4_dev(g["W"]), t(g["X"])
    v = synth.gemm_case(4, 1, 2048, 8192)
    gemv_w, x = w4_dev(v["W"]), t(v["X"][0])

    ref = [host(a).copy() for a in _run(dw, H, bias, gemm_w, X, gemv_w, x, None)]
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    big = torch.randn(4096, 4096, device="cuda")
    with torch.cuda.stream(side):
        res = _run(dw, H, bias, gemm_w, X, gemv_w, x, side)
    for _ in range(8):  # unrelated work on the default stream meanwhile
        big = torch.tanh(big @ big * 1e-3)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(res, ref)):
        assert np.array_equal(host(a).view(np.uint8), b.view(np.uint8)), i
