"""GPU parity of the routed-expert layer: decode (one token, fused
row-parallel path) and prefill (ragged MFMA grouped GEMM), each against the
oracle's own routing and expert FFN."""
import json
import os

import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import assert_close, guarded, host, say, t, w4_dev

pytestmark = pytest.mark.gpu


def _dev_weights(w):
    return {"Wr": t(w["Wr"]), "gate_up": w4_dev(w["gate_up"]), "down": w4_dev(w["down"]),
            "shared_gate_up": w4_dev(w["shared_gate_up"]), "shared_down": w4_dev(w["shared_down"])}


def _run_layer(dw, H, bias, topk, T, fused_down):
    route = ql.moe_route(H, dw["Wr"], bias, topk)
    act = ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk,
                              ql.QL_OP_GATE_UP_SILU, route)
    if fused_down:
        out = ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk,
                                  ql.QL_OP_DOWN_COMBINE, route)
        return route, act, None, out
    ydown = ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk, ql.QL_OP_DOWN, route)
    out = ql.moe_combine(ydown, route["gates"], route["pos"], T, topk, True)
    return route, act, ydown, out


def _ref_rows(route, ref, T, topk):
    """Index of the oracle row holding the same (token, expert) pair as each
    GPU row.  Equal expert sets are required; the order of two experts
    whose logits are nearly tied may differ, which permutes rows."""
    ids_g = host(route["ids"])
    sa_g = host(route["sorted_assign"])
    a = sa_g.astype(np.int64)
    tok = a // topk
    e = ids_g[tok, a % topk]
    match = ref["ids"][tok] == e[:, None]
    assert np.all(match.sum(axis=1) == 1), "routed expert sets differ"
    j_ref = match.argmax(axis=1)
    routed = ref["pos"][tok * topk + j_ref]
    return np.concatenate([routed, np.arange(T * topk, ref["act"].shape[0])])


def _compare(route, act, ydown, out, ref, T, topk):
    rows = _ref_rows(route, ref, T, topk)
    assert_close(host(act).astype(np.float64), ref["act"][rows].astype(np.float64), "act")
    if ydown is not None:
        assert_close(host(ydown).astype(np.float64), ref["ydown"][rows], "ydown")
    return assert_close(host(out).astype(np.float64), ref["out"], "out")


@pytest.mark.parametrize("seed", [0, 1, 2])
@pytest.mark.parametrize("fused_down", [True, False])
def test_moe_decode(seed, fused_down):
    import torch
    say(f"moe decode seed={seed} fused={fused_down}")
    w = synth.moe_weights(seed)
    tok = synth.moe_tokens(seed + 1000, 1)
    ref = oracle.moe_layer(tok["H"], w, None, 8)
    dw = _dev_weights(w)
    res = _run_layer(dw, t(tok["H"]), None, 8, 1, fused_down)
    torch.cuda.synchronize()
    rel, mx = _compare(*res, ref, 1, 8)
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_moe_decode_reads_only_selected_experts():
    """Scales of every expert the token did not choose are NaN: any read of
    them would poison the output."""
    import torch
    seed = 5
    w = synth.moe_weights(seed)
    tok = synth.moe_tokens(seed + 1000, 1)
    ref = oracle.moe_layer(tok["H"], w, None, 8)
    chosen = set(ref["ids"][0].tolist())
    for key in ("gate_up", "down"):
        for e in range(256):
            if e not in chosen:
                w[key]["scales"][e] = np.float16(np.nan)
    dw = _dev_weights(w)
    res = _run_layer(dw, t(tok["H"]), None, 8, 1, True)
    torch.cuda.synchronize()
    _compare(*res, ref, 1, 8)


@pytest.mark.parametrize("T,D,I,E,topk,seed", [
    (2, 512, 256, 16, 4, 0),     # row-parallel path, several tokens
    (4, 2048, 512, 256, 8, 1),
    (5, 512, 128, 16, 4, 2),     # smallest T of the tiled path
    (300, 256, 128, 16, 4, 3),   # ragged tiles
    (700, 512, 256, 64, 8, 4),
])
def test_moe_small_shapes(T, D, I, E, topk, seed):
    import torch
    say(f"moe T={T} D={D} I={I} E={E} topk={topk}")
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 50, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk)
    dw = _dev_weights(w)
    res = _run_layer(dw, t(tok["H"]), t(tok["logit_bias"]), topk, T, False)
    torch.cuda.synchronize()
    _compare(*res, ref, T, topk)


@pytest.mark.parametrize("T,D,I,E,topk,seed", [
    (1, 512, 256, 16, 2, 5),      # 3 rows per token: a wave of the block has none
    (3, 512, 256, 16, 1, 6),      # 2 rows per token
    (4, 2048, 512, 256, 8, 7),    # the decode shape, 4 tokens
    (2, 1024, 512, 32, 13, 8),    # 14 rows per token: two rounds for some waves
])
def test_moe_decode_fused_down_shapes(T, D, I, E, topk, seed):
    """The fused decode down projection (gate-weighted sum over the token's
    rows and the shared row) over row counts below, at and above one row per
    wave of its block."""
    import torch
    say(f"moe fused down T={T} D={D} I={I} E={E} topk={topk}")
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 60, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk)
    dw = _dev_weights(w)
    res = _run_layer(dw, t(tok["H"]), t(tok["logit_bias"]), topk, T, True)
    torch.cuda.synchronize()
    _compare(*res, ref, T, topk)


_SEEDS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prefill_seeds.json")))
SCREENED = _SEEDS["kept_seeds_by_gap"]
FULL_ORDER = _SEEDS["kept_seeds_full_order"]


@pytest.mark.parametrize("seed", FULL_ORDER[:1])
def test_moe_prefill_4096(seed):
    """The prefill workload: 4096 tokens, 256 experts + shared, Zipf logit
    bias, in the benchmark's launch configuration, on a full-order screened
    seed: routing ids, counts, offsets, permutation and inverse equal the
    oracle's bit for bit, and act, ydown and out are compared row by row in
    the oracle's own row order, every output behind guard regions."""
    import torch
    say(f"moe prefill T=4096 seed={seed}")
    T, topk = 4096, 8
    w = synth.moe_weights(0)
    tok = synth.moe_tokens(seed, T, skewed=True)
    ref = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk)
    dw = _dev_weights(w)
    from tests.test_gpu_route import guarded_route_outputs
    route, check_route = guarded_route_outputs(T, 256, topk)
    act = guarded((T * topk + T, 512), torch.float16)
    ydown = guarded((T * topk + T, 2048), torch.float16)
    out = guarded((T, 2048), torch.float16)
    H = t(tok["H"])
    ql.moe_route(H, dw["Wr"], t(tok["logit_bias"]), topk, route)
    ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk, ql.QL_OP_GATE_UP_SILU, route, act.t)
    ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act.t, T, topk, ql.QL_OP_DOWN, route, ydown.t)
    ql.moe_combine(ydown.t, route["gates"], route["pos"], T, topk, True, out.t)
    torch.cuda.synchronize()
    check_route()
    for g, name in ((act, "act"), (ydown, "ydown"), (out, "out")):
        g.check(name)
    assert np.array_equal(host(route["ids"]), ref["ids"])
    assert np.array_equal(host(route["counts"]), ref["counts"])
    assert np.array_equal(host(route["offsets"]), ref["offsets"])
    assert np.array_equal(host(route["sorted_assign"]), ref["sorted_assign"])
    assert np.array_equal(host(route["pos"]), ref["pos"])
    assert_close(host(act.t).astype(np.float64), ref["act"].astype(np.float64), "act")
    assert_close(host(ydown.t).astype(np.float64), ref["ydown"], "ydown")
    rel, mx = assert_close(host(out.t).astype(np.float64), ref["out"], "out")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_moe_decode_graph_replays_match_eager():
    """The decode chain captured in a HIP graph: every replay (with eager work
    and synchronizations in between) reproduces the eager output bit for bit."""
    import torch
    w = synth.moe_weights(6)
    dw = _dev_weights(w)
    toks = [t(synth.moe_tokens(3000 + i, 1)["H"]) for i in range(3)]
    route = ql.alloc_route_outputs(1, 256, 8, toks[0].device)
    act = torch.empty((9, 512), dtype=torch.float16, device=toks[0].device)
    outs = [torch.empty((1, 2048), dtype=torch.float16, device=toks[0].device) for _ in toks]

    def step(i):
        ql.moe_route(toks[i], dw["Wr"], None, 8, route)
        ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], toks[i], 1, 8,
                            ql.QL_OP_GATE_UP_SILU, route, act)
        ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, 1, 8, ql.QL_OP_DOWN_COMBINE,
                            route, outs[i])

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    eager = [host(o).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(3):
            step(i)
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert np.array_equal(host(outs[i]).view(np.uint16), eager[i].view(np.uint16)), (rep, i)
        # eager work between replays
        ql.qlinear_gemv(dw["shared_down"], act[0].contiguous())
        torch.cuda.synchronize()
    ref = oracle.moe_layer(synth.moe_tokens(3000, 1)["H"], w, None, 8)
    assert_close(eager[0].astype(np.float64), ref["out"], "decode out")


def _decode_args(dw, shared=True):
    return dict(gate_up=dw["gate_up"], down=dw["down"],
                shared_gate_up=dw["shared_gate_up"] if shared else None,
                shared_down=dw["shared_down"] if shared else None)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_moe_decode_entry(seed):
    """moe_decode (routing fused into the gate/up rows) on the decode shape:
    the oracle's routing exactly, its output within the fp16 bar, and the
    same bits as the three-call path."""
    import torch
    say(f"moe_decode seed={seed}")
    w = synth.moe_weights(seed)
    tok = synth.moe_tokens(seed + 1000, 1)
    ref = oracle.moe_layer(tok["H"], w, None, 8)
    dw = _dev_weights(w)
    H = t(tok["H"])
    res = ql.moe_decode(H, dw["Wr"], None, 8, **_decode_args(dw))
    route, act, _, out3 = _run_layer(dw, H, None, 8, 1, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(res["ids"]), ref["ids"])
    assert np.abs(host(res["gates"]).astype(np.float64) - ref["gates"]).max() < 2e-5
    rel, mx = assert_close(host(res["out"]).astype(np.float64), ref["out"], "out")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")
    assert np.array_equal(host(res["ids"]), host(route["ids"]))
    assert np.array_equal(host(res["gates"]).view(np.uint32), host(route["gates"]).view(np.uint32))
    assert np.array_equal(host(res["out"]).view(np.uint16), host(out3).view(np.uint16))
    off = ql.moe_decode_logits_offset(1, 256, 8)
    Lg = host(res["workspace"])[off:off + 4 * 256].view(np.float32)
    assert np.abs(Lg - ref["logits"][0]).max() < 2e-5


@pytest.mark.parametrize("T,D,I,E,topk,seed,shared", [
    (1, 512, 256, 16, 2, 5, True),
    (3, 512, 256, 16, 1, 6, True),
    (4, 2048, 512, 256, 8, 7, True),
    (2, 1024, 512, 32, 13, 8, True),
    (2, 512, 128, 1000, 32, 9, True),    # E > 256: 16 keys per lane in the top-k
    (3, 256, 64, 33, 5, 10, True),       # E % 8 != 0: scalar router partials
    (2, 2048, 512, 256, 8, 11, False),   # no shared expert
])
def test_moe_decode_entry_shapes(T, D, I, E, topk, seed, shared):
    import torch
    say(f"moe_decode T={T} D={D} I={I} E={E} topk={topk} shared={shared}")
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 60, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk, with_shared=shared)
    dw = _dev_weights(w)
    res = ql.moe_decode(t(tok["H"]), dw["Wr"], t(tok["logit_bias"]), topk, **_decode_args(dw, shared))
    torch.cuda.synchronize()
    ids = host(res["ids"])
    near = oracle.topk_near_ties(ref["logits"], topk, 1e-4)
    assert not near[:, -1].any(), "seed has a near tie at the top-k cut"
    assert all(set(a) == set(b) for a, b in zip(ids.tolist(), ref["ids"].tolist()))
    assert np.array_equal(ids[~near], ref["ids"][~near])
    assert_close(host(res["out"]).astype(np.float64), ref["out"], "out")


def test_moe_decode_entry_reads_only_selected_experts():
    """NaN scales in every expert the token did not choose leave moe_decode's
    output finite and correct."""
    import torch
    seed = 5
    w = synth.moe_weights(seed)
    tok = synth.moe_tokens(seed + 1000, 1)
    ref = oracle.moe_layer(tok["H"], w, None, 8)
    chosen = set(ref["ids"][0].tolist())
    for key in ("gate_up", "down"):
        for e in range(256):
            if e not in chosen:
                w[key]["scales"][e] = np.float16(np.nan)
    dw = _dev_weights(w)
    res = ql.moe_decode(t(tok["H"]), dw["Wr"], None, 8, **_decode_args(dw))
    torch.cuda.synchronize()
    assert_close(host(res["out"]).astype(np.float64), ref["out"], "out")


def test_moe_decode_entry_graph_replays():
    """moe_decode captured in a HIP graph for three tokens: every replay
    matches the eager bits."""
    import torch
    w = synth.moe_weights(6)
    dw = _dev_weights(w)
    toks = [t(synth.moe_tokens(3100 + i, 1)["H"]) for i in range(3)]
    outs = [ql.alloc_decode_outputs(1, 256, 8, 2048, 512, toks[0].device) for _ in toks]

    def step(i):
        ql.moe_decode(toks[i], dw["Wr"], None, 8, **_decode_args(dw), out=outs[i])

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    eager = [host(o["out"]).copy() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(3):
            step(i)
    for rep in range(3):
        for o in outs:
            o["out"].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(3):
            assert np.array_equal(host(outs[i]["out"]).view(np.uint16), eager[i].view(np.uint16)), (rep, i)
        ql.qlinear_gemv(dw["shared_down"], toks[0][:, :512].contiguous())
        torch.cuda.synchronize()
    ref = oracle.moe_layer(synth.moe_tokens(3100, 1)["H"], w, None, 8)
    assert_close(eager[0].astype(np.float64), ref["out"], "decode out")


def test_decode_token_loop_through_moe_graph():
    """A decode loop that never leaves the GPU: the routed-expert layer
    (moe_decode) on the current row, the vocabulary head's token choice into
    a device slot, the next row read from the embedding table by that slot;
    four steps with two alternating slots, captured once in a HIP graph and
    replayed.  Every replay's tokens and rows equal the oracle's chain, and
    each step's layer output is within the fp16 bar.  The seed is screened
    by the oracle: every top-8 cut clears 1e-3 and every token choice 1% of
    the largest logit."""
    import torch
    K, V, steps, seed = 2048, 4096, 4, 66
    w = synth.moe_weights(seed)
    rng = synth.rng_for(seed + 500)
    Wh = synth.w4_matrix(rng, K, V)
    E = synth.w4_matrix(rng, K, V)
    x0 = synth.activations(rng, 1, K)[0]
    toks, rows, outs, x = [], [], [], x0
    for _ in range(steps):
        ref = oracle.moe_layer(x[None, :], w, None, 8)
        srt = -np.sort(-ref["logits"][0])
        assert srt[7] - srt[8] > 1e-3, "routing near a tie"
        tok, logits = oracle.lm_head_token(oracle.round_f16(ref["out"][0]), Wh)
        s2 = np.sort(logits)
        assert s2[-1] - s2[-2] > 1e-2 * np.abs(logits).max(), "token choice near a tie"
        x = oracle.embed_row(E, tok)
        toks.append(tok)
        rows.append(x)
        outs.append(ref["out"][0])
    dev = torch.device("cuda")
    dw = _dev_weights(w)
    Whd, Ed = w4_dev(Wh), w4_dev(E)
    xs = [t(x0[None, :])] + [torch.empty((1, K), dtype=torch.float16, device=dev) for _ in range(steps)]
    dec = [ql.alloc_decode_outputs(1, 256, 8, K, 512, dev) for _ in range(steps)]
    slots = torch.full((2,), -7, dtype=torch.int32, device=dev)
    ws = ql.gemv_argmax_workspace(V, dev)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                slot = slots[i % 2:i % 2 + 1]
                ql.moe_decode(xs[i], dw["Wr"], None, 8, dw["gate_up"], dw["down"],
                              dw["shared_gate_up"], dw["shared_down"], out=dec[i])
                ql.qlinear_gemv_argmax(Whd, dec[i]["out"][0], token=slot, workspace=ws)
                ql.qlinear_embed_token(Ed, slot, xs[i + 1][0])
    for rep in range(3):
        for b in xs[1:]:
            b.fill_(7.0)  # eager work between replays
        slots.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i in range(steps):
            assert np.array_equal(host(xs[i + 1][0]).view(np.uint16), rows[i].view(np.uint16)), (rep, i)
            assert_close(host(dec[i]["out"][0]).astype(np.float64), outs[i], f"layer output {i}")
        assert host(slots).tolist() == [toks[steps - 2], toks[steps - 1]], rep


@pytest.mark.parametrize("where,scale", [("h", 1e-4), ("h", 3e-5), ("act", 1e-4), ("act", 3e-5)])
def test_moe_decode_small_activations(where, scale):
    """Row-kernel inputs of order 1e-4 and 3e-5, many of them fp16
    subnormals, on the decode shape.  where = "h": the tokens are that small
    (the router weight and the gate/up scales are scaled up by the inverse,
    so logits and act keep their usual size); where = "act": the gate/up
    scales are scaled down so that act is that small (the down scales are
    scaled up by the inverse).  moe_decode and the three-call path against
    the oracle, routing exact."""
    import torch
    say(f"moe_decode small {where} scale={scale}")
    D, I, E = 2048, 512, 256
    if where == "h":
        w = synth.moe_weights(7, scale_range=(0.002 / scale, 0.02 / scale), router_std=0.02 / scale)
        rng = synth.rng_for(8)
        w["down"] = synth.w4_matrix(rng, I, D, lead=(E,))
        w["shared_down"] = synth.w4_matrix(rng, I, D)
        tok = synth.moe_tokens(1007, 1, h_scale=scale)
    else:
        f = np.sqrt(2.0 * scale) / 2.25  # |u| ~ 2.25 f, act ~ u^2 / 2 ~ scale
        w = synth.moe_weights(7, scale_range=(0.002 * f, 0.02 * f))
        rng = synth.rng_for(8)
        w["down"] = synth.w4_matrix(rng, I, D, lead=(E,), scale_range=(0.002 / scale, 0.02 / scale))
        w["shared_down"] = synth.w4_matrix(rng, I, D, scale_range=(0.002 / scale, 0.02 / scale))
        tok = synth.moe_tokens(1007, 1)
    ref = oracle.moe_layer(tok["H"], w, None, 8)
    a = np.abs(ref["act"].astype(np.float64))
    say(f"  act: median {np.median(a):.2e}, fp16-subnormal share {np.mean(a < 2.0**-14):.2f}")
    srt = -np.sort(-ref["logits"][0])
    assert srt[7] - srt[8] > 1e-4 * max(1.0, abs(srt[0])), "routing near a tie"
    dw = _dev_weights(w)
    H = t(tok["H"])
    res = ql.moe_decode(H, dw["Wr"], None, 8, **_decode_args(dw))
    route, act, _, out3 = _run_layer(dw, H, None, 8, 1, True)
    torch.cuda.synchronize()
    assert np.array_equal(host(res["ids"]), ref["ids"])
    rel, mx = assert_close(host(res["out"]).astype(np.float64), ref["out"], "moe_decode out")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")
    assert_close(host(act).astype(np.float64), ref["act"][_ref_rows(route, ref, 1, 8)].astype(np.float64), "act")
    assert_close(host(out3).astype(np.float64), ref["out"], "three-call out")


@pytest.mark.parametrize("T,seed", [(1, 2037), (2, 677), (4, 75)])
def test_moe_decode_exact_routing_every_token(T, seed):
    """moe_decode on router inputs with exact fp32 logits; each seed holds a
    token with two equal logits across the top-k cut (found by searching
    seeds with the oracle).  The ids equal the oracle's for every token (the
    tie goes to the lower expert index), the logits bit for bit, the gates
    within 2e-6."""
    import torch
    say(f"moe_decode exact routing T={T}")
    c = synth.router_exact_case(seed, T)
    w = synth.moe_weights(seed)
    w["Wr"] = c["Wr"]
    ref = oracle.moe_layer(c["H"], w, c["logit_bias"], 8)
    dw = _dev_weights(w)
    res = ql.moe_decode(t(c["H"]), dw["Wr"], t(c["logit_bias"]), 8, **_decode_args(dw))
    torch.cuda.synchronize()
    assert np.array_equal(host(res["ids"]), ref["ids"])
    assert np.abs(host(res["gates"]).astype(np.float64) - ref["gates"]).max() < 2e-6
    off = ql.moe_decode_logits_offset(T, 256, 8)
    Lg = host(res["workspace"])[off:off + 4 * T * 256].view(np.float32).reshape(T, 256)
    assert np.array_equal(Lg.astype(np.float64), ref["logits"])
    assert_close(host(res["out"]).astype(np.float64), ref["out"], "out")


# Per-expert row counts at the edges of the tile kinds: at most 32 rows
# (register-streamed tile), 33 (staged short tile), tall tiles of 256 rows
# and a short remainder, and an empty expert.
BOUNDARY_COUNTS = [1, 31, 32, 33, 0, 97, 256, 300]


def boundary_route(E, counts, seed):
    """ids [T][1] that give expert e exactly counts[e] rows, in a seeded
    token order."""
    rng = np.random.default_rng(seed)
    return rng.permutation(np.repeat(np.arange(E), counts)).astype(np.int32).reshape(-1, 1)


def w4_expert(W, e):
    return {"qweight": W["qweight"][e], "scales": W["scales"][e], "biases": W["biases"][e],
            "K": W["K"], "N": W["N"]}


def expert_rows_reference(ids, sorted_assign, H, w, ffn, with_shared=True, expert=w4_expert):
    """Oracle act / ydown in the GPU's row order: the rows of expert e are
    its tokens in the order of sorted_assign (checked against the stable
    permutation), then one shared row per token.  expert(W, e) slices
    expert e out of a stacked matrix."""
    T = ids.shape[0]
    E = int(ids.max()) + 1
    ref_sorted, _ = oracle.stable_permutation(ids, E)
    assert np.array_equal(sorted_assign, ref_sorted)
    tok = sorted_assign.astype(np.int64)  # topk = 1: assignment a is token a
    acts, yds = [None] * T, [None] * T
    for e in range(E):
        rows = np.nonzero(ids[tok, 0] == e)[0]
        if rows.size == 0:
            continue
        a, y = ffn(H[tok[rows]], expert(w["gate_up"], e), expert(w["down"], e))
        for i, r in enumerate(rows):
            acts[r], yds[r] = a[i], y[i]
    act, yd = np.stack(acts), np.stack(yds)
    if with_shared:
        sa, sy = ffn(H, w["shared_gate_up"], w["shared_down"])
        act, yd = np.concatenate([act, sa]), np.concatenate([yd, sy])
    return act, yd


@pytest.mark.parametrize("D,I", [(2048, 512), (1024, 256), (512, 1024)])
def test_moe_tile_row_boundaries(D, I):
    """Experts with 1, 31, 32, 33, 0, 97, 256 and 300 rows (moe_dispatch on
    given ids, topk 1) and the shared expert, at K = 2048, 1024 and 512 for
    both projections: every act and ydown row against the oracle's FFN of
    its own expert."""
    import torch
    E = len(BOUNDARY_COUNTS)
    say(f"moe tile boundaries D={D} I={I}")
    ids = boundary_route(E, BOUNDARY_COUNTS, D + I)
    T = ids.shape[0]
    w = synth.moe_weights(D + I, D=D, I=I, E=E)
    H = synth.moe_tokens(D + I + 1, T, D=D, E=E)["H"]
    dw = _dev_weights(w)
    route = ql.moe_dispatch(t(ids), E)
    act = ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], t(H), T, 1, ql.QL_OP_GATE_UP_SILU, route)
    yd = ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, 1, ql.QL_OP_DOWN, route)
    torch.cuda.synchronize()
    ref_act, ref_yd = expert_rows_reference(ids, host(route["sorted_assign"]), H, w, oracle.expert_ffn)
    assert_close(host(act).astype(np.float64), ref_act.astype(np.float64), "act")
    assert_close(host(yd).astype(np.float64), ref_yd, "ydown")


def test_moe_shared_expert_on_a_second_stream():
    """The layer split across two streams: routing and the routed rows
    (shared = None) on one, the shared expert's rows (QL_OP_SHARED_ONLY, no
    routing inputs) on another, joined by events.  Every act, ydown and out
    bit equals the single-stream layer's, over several back-to-back steps
    that alternate two token sets."""
    import torch
    T, topk = 4096, 8
    w = synth.moe_weights(0)
    dw = _dev_weights(w)
    seeds = FULL_ORDER[:2]
    toks = [synth.moe_tokens(sd, T, skewed=True) for sd in seeds]
    Hs = [t(tk["H"]) for tk in toks]
    bs = [t(tk["logit_bias"]) for tk in toks]
    ref = []
    for H, b in zip(Hs, bs):
        route, act, yd, out = _run_layer(dw, H, b, topk, T, False)
        ref.append((host(act), host(yd), host(out)))
    dev = Hs[0].device
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    routes = [ql.alloc_route_outputs(T, 256, topk, dev) for _ in seeds]
    act = torch.empty((T * topk + T, 512), dtype=torch.float16, device=dev)
    yd = torch.empty((T * topk + T, 2048), dtype=torch.float16, device=dev)
    outs = [torch.empty((T, 2048), dtype=torch.float16, device=dev) for _ in seeds]
    for step in range(6):
        i = step % 2
        fork = torch.cuda.Event()
        fork.record(main)
        side.wait_event(fork)
        with torch.cuda.stream(side):
            ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], Hs[i], T, topk,
                                ql.QL_OP_GATE_UP_SILU | ql.QL_OP_SHARED_ONLY, None, act, stream=side)
            ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk,
                                ql.QL_OP_DOWN | ql.QL_OP_SHARED_ONLY, None, yd, stream=side)
        join = torch.cuda.Event()
        join.record(side)
        ql.moe_route(Hs[i], dw["Wr"], bs[i], topk, routes[i])
        ql.moe_grouped_gemm(dw["gate_up"], None, Hs[i], T, topk, ql.QL_OP_GATE_UP_SILU, routes[i], act)
        ql.moe_grouped_gemm(dw["down"], None, act, T, topk, ql.QL_OP_DOWN, routes[i], yd)
        main.wait_event(join)
        ql.moe_combine(yd, routes[i]["gates"], routes[i]["pos"], T, topk, True, outs[i])
        if step >= 4:
            torch.cuda.synchronize()
            a_ref, y_ref, o_ref = ref[i]
            assert np.array_equal(host(act).view(np.uint16), a_ref.view(np.uint16))
            assert np.array_equal(host(yd).view(np.uint16), y_ref.view(np.uint16))
            assert np.array_equal(host(outs[i]).view(np.uint16), o_ref.view(np.uint16))


@pytest.mark.gpu
@pytest.mark.parametrize("T", [40, 600])
def test_moe_shared_only_ragged_rows(T):
    """A launch of the shared expert alone (QL_OP_SHARED_ONLY) with a token
    count that ends in a partial tile: the shared rows of act and ydown
    equal the single launch's bit for bit and the routed rows are left
    untouched (guard value)."""
    import torch
    topk = 8
    say(f"shared-only ragged T={T}")
    w = synth.moe_weights(0)
    dw = _dev_weights(w)
    tk = synth.moe_tokens(7, T, skewed=True)
    H, b = t(tk["H"]), t(tk["logit_bias"])
    route, act, yd, _ = _run_layer(dw, H, b, topk, T, False)
    torch.cuda.synchronize()
    fill = np.float16(-3.0).view(np.uint16)
    act2 = torch.full_like(act, -3.0)
    yd2 = torch.full_like(yd, -3.0)
    ql.moe_grouped_gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk,
                        ql.QL_OP_GATE_UP_SILU | ql.QL_OP_SHARED_ONLY, None, act2)
    ql.moe_grouped_gemm(dw["down"], dw["shared_down"], act, T, topk,
                        ql.QL_OP_DOWN | ql.QL_OP_SHARED_ONLY, None, yd2)
    torch.cuda.synchronize()
    r = T * topk
    a_g, a_r = host(act2).view(np.uint16), host(act).view(np.uint16)
    y_g, y_r = host(yd2).view(np.uint16), host(yd).view(np.uint16)
    assert np.array_equal(a_g[r:], a_r[r:])
    assert np.array_equal(y_g[r:], y_r[r:])
    assert np.all(a_g[:r] == fill) and np.all(y_g[:r] == fill)
