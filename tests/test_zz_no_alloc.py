"""moe_decode_noalloc, the decode layer on the library's own device scratch
(for callers that cannot allocate), against moe_decode with a workspace:
the same kernels, so ids, gates and output must agree bit for bit, on calls
in a row of different (shrinking, then growing) sizes, eagerly and in a
HIP graph."""
import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, guarded, host, say, t, w4_dev

pytestmark = pytest.mark.gpu


def _dev(w):
    return {"Wr": t(w["Wr"]), "gate_up": w4_dev(w["gate_up"]), "down": w4_dev(w["down"]),
            "shared_gate_up": w4_dev(w["shared_gate_up"]), "shared_down": w4_dev(w["shared_down"])}


# (T, D, I, E, topk, seed): the decode shape with four tokens, then a smaller
# layer, then the decode shape with one token.
CASES = [(4, 2048, 512, 256, 8, 1), (1, 512, 256, 16, 2, 2), (1, 2048, 512, 256, 8, 3)]


def _one(T, D, I, E, topk, seed):
    import torch
    say(f"moe_decode_noalloc T={T} D={D} I={I} E={E} topk={topk}")
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 70, T, D=D, E=E, skewed=True)
    dw = _dev(w)
    H, bias = t(tok["H"]), t(tok["logit_bias"])
    ref = ql.moe_decode(H, dw["Wr"], bias, topk, dw["gate_up"], dw["down"], dw["shared_gate_up"],
                        dw["shared_down"])
    ids = guarded((T, topk), torch.int32)
    gates = guarded((T, topk), torch.float32)
    out = guarded((T, D), torch.float16)
    ql.moe_decode_noalloc(H, dw["Wr"], bias, topk, dw["gate_up"], dw["down"], dw["shared_gate_up"],
                          dw["shared_down"], ids=ids.t, gates=gates.t, out=out.t)
    torch.cuda.synchronize()
    for g, name in ((ids, "ids"), (gates, "gates"), (out, "out")):
        g.check(name)
    assert np.array_equal(host(ids.t), host(ref["ids"]))
    assert np.array_equal(host(gates.t).view(np.uint32), host(ref["gates"]).view(np.uint32))
    assert np.array_equal(host(out.t).view(np.uint16), host(ref["out"]).view(np.uint16))
    o = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk)
    assert all(set(a) == set(b) for a, b in zip(host(ids.t).tolist(), o["ids"].tolist()))
    assert_close(host(out.t).astype(np.float64), o["out"], "noalloc out")
    return dw, H, bias, host(out.t).copy()


def test_noalloc_matches_moe_decode_in_a_row():
    for c in CASES:
        _one(*c)


def test_noalloc_graph_replays():
    """Captured in a HIP graph after an eager call: every replay equals the
    eager bits (the scratch keeps nothing that a later call depends on)."""
    import torch
    T, D, I, E, topk, seed = CASES[0]
    dw, H, bias, eager = _one(T, D, I, E, topk, seed)
    out = torch.empty((T, D), dtype=torch.float16, device=H.device)
    ids = torch.empty((T, topk), dtype=torch.int32, device=H.device)
    gates = torch.empty((T, topk), dtype=torch.float32, device=H.device)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ql.moe_decode_noalloc(H, dw["Wr"], bias, topk, dw["gate_up"], dw["down"],
                                  dw["shared_gate_up"], dw["shared_down"], ids=ids, gates=gates, out=out)
    for rep in range(3):
        out.fill_(7.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint16), eager.view(np.uint16)), rep
        _one(*CASES[1])  # a different call on the same scratch between replays
