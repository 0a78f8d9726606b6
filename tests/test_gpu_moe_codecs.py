"""GPU parity of the routed-expert layer with FP8-E4M3 or NVFP4 experts
(moe_route, moe_grouped_gemm_fp8 / moe_grouped_gemm_nvfp4 for gate/up and
down, moe_combine) against the oracle's codec layers, with the fp16 bars of
tests/gpu_util.py."""
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


def _nvfp4_dev(W):
    import torch
    g = W["global_scale"]
    g = torch.from_numpy(np.ascontiguousarray(g)).cuda() if np.ndim(g) else float(g)
    return {"qweight": t(W["qweight"]), "block_scales": t(W["block_scales"]), "global_scale": g,
            "K": int(W["K"]), "N": int(W["N"])}


def _dev_weights_nvfp4(w):
    return {"Wr": t(w["Wr"]), "gate_up": _nvfp4_dev(w["gate_up"]), "down": _nvfp4_dev(w["down"]),
            "shared_gate_up": _nvfp4_dev(w["shared_gate_up"]), "shared_down": _nvfp4_dev(w["shared_down"])}


def _run(dw, H, bias, topk, T, shared=True, gemm=None):
    gemm = gemm or ql.moe_grouped_gemm_fp8
    route = ql.moe_route(H, dw["Wr"], bias, topk)
    act = gemm(dw["gate_up"], dw["shared_gate_up"] if shared else None, H, T, topk,
               ql.QL_OP_GATE_UP_SILU, route)
    ydown = gemm(dw["down"], dw["shared_down"] if shared else None, act, T, topk, ql.QL_OP_DOWN, route)
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
    (1, 2048, 512, 256, 8, 0, True),     # one token: the row-parallel decode path
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


def test_moe_fp8_down_combine_needs_the_decode_path():
    """QL_OP_DOWN_COMBINE runs on the row-parallel decode path only
    (T <= QL_DECODE_MAX_T); more tokens are rejected."""
    w = synth.moe_weights_fp8(0, D=256, I=64, E=8)
    dw = _dev_weights(w)
    tok = synth.moe_tokens(1, 5, D=256, E=8)
    route = ql.moe_route(t(tok["H"]), dw["Wr"], None, 2)
    with pytest.raises(ql.QLError):
        ql.moe_grouped_gemm_fp8(dw["down"], None, t(np.zeros((10, 64), np.float16)), 5, 2,
                                ql.QL_OP_DOWN_COMBINE, route)


@pytest.mark.parametrize("seed", SCREENED[:1])
def test_moe_nvfp4_prefill_4096(seed):
    """The prefill workload with NVFP4 experts (a global scale per expert)."""
    import torch
    say(f"moe nvfp4 prefill T=4096 seed={seed}")
    w = synth.moe_weights_nvfp4(0)
    tok = synth.moe_tokens(seed, 4096, skewed=True)
    ref = oracle.moe_layer_nvfp4(tok["H"], w, tok["logit_bias"], 8)
    res = _run(_dev_weights_nvfp4(w), t(tok["H"]), t(tok["logit_bias"]), 8, 4096,
               gemm=ql.moe_grouped_gemm_nvfp4)
    torch.cuda.synchronize()
    _check_routing(res[0], ref)
    rel, mx = _compare(*res, ref, 4096, 8)
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


@pytest.mark.parametrize("T,D,I,E,topk,seed,shared", [
    (1, 2048, 512, 256, 8, 0, True),
    (300, 256, 128, 16, 4, 3, True),
    (700, 512, 256, 64, 8, 7, True),
    (200, 256, 64, 33, 5, 5, False),
    (70, 4096, 192, 8, 2, 6, True),
])
def test_moe_nvfp4_shapes(T, D, I, E, topk, seed, shared):
    import torch
    from tests.gpu_util import assert_close
    say(f"moe nvfp4 T={T} D={D} I={I} E={E} topk={topk} shared={shared}")
    w = synth.moe_weights_nvfp4(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 90, T, D=D, E=E, skewed=True)
    ref = oracle.moe_layer_nvfp4(tok["H"], w, tok["logit_bias"], topk, with_shared=shared)
    srt = -np.sort(-ref["logits"], axis=1)
    assert (srt[:, topk - 1] - srt[:, topk]).min() > 5e-5, "case not screened"
    res = _run(_dev_weights_nvfp4(w), t(tok["H"]), t(tok["logit_bias"]), topk, T, shared,
               gemm=ql.moe_grouped_gemm_nvfp4)
    torch.cuda.synchronize()
    _check_routing(res[0], ref)
    assert_close(host(res[1]).astype(np.float64), ref["act"].astype(np.float64), "act")
    assert_close(host(res[2]).astype(np.float64), ref["ydown"], "ydown")
    rel, mx = assert_close(host(res[3]).astype(np.float64), ref["out"], "out")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")


def test_moe_nvfp4_and_fp8_bit_identical_on_common_weights():
    """NVFP4 experts whose weights the FP8 format holds exactly (block scales
    constant over each 64, power-of-two global scales): both kernels stage
    the same fp16 weights, so act and ydown agree bit for bit."""
    import torch
    T, D, I, E, topk = 500, 512, 128, 16, 4
    w = synth.moe_weights_nvfp4(21, D=D, I=I, E=E)
    E4M3_OF_E2M1 = np.array([0x00, 0x30, 0x38, 0x3C, 0x40, 0x44, 0x48, 0x4C], np.uint8)
    f8 = {"Wr": w["Wr"]}
    for key in ("gate_up", "down", "shared_gate_up", "shared_down"):
        W = w[key]
        W["block_scales"] = np.repeat(W["block_scales"][..., ::4], 4, axis=-1)
        stacked = np.ndim(W["global_scale"]) > 0
        W["global_scale"] = (np.exp2(-(np.arange(E) % 3) - 6).astype(np.float32) if stacked
                             else np.float32(2.0 ** -7))
        q = oracle.unpack_codes(W["qweight"], W["K"]).astype(np.int64)
        codes = (E4M3_OF_E2M1[q & 7] | np.where(q & 8, 0x80, 0)).astype(np.uint8)
        g = np.asarray(W["global_scale"], np.float64)
        g = g[:, None, None] if stacked else g
        scales = (oracle.e4m3_to_f64(W["block_scales"][..., ::4]) * g).astype(np.float16)
        f8[key] = {"codes": codes, "scales": scales, "K": W["K"], "N": W["N"]}
    tok = synth.moe_tokens(22, T, D=D, E=E, skewed=True)
    a = _run(_dev_weights_nvfp4(w), t(tok["H"]), t(tok["logit_bias"]), topk, T,
             gemm=ql.moe_grouped_gemm_nvfp4)
    b = _run(_dev_weights(f8), t(tok["H"]), t(tok["logit_bias"]), topk, T)
    torch.cuda.synchronize()
    for x, y in zip(a[1:], b[1:]):
        assert np.array_equal(host(x).view(np.uint16), host(y).view(np.uint16))


def _fp8_expert(W, e):
    return {"codes": W["codes"][e], "scales": W["scales"][e], "K": W["K"], "N": W["N"]}


def _nvfp4_expert(W, e):
    return {"qweight": W["qweight"][e], "block_scales": W["block_scales"][e],
            "global_scale": float(np.asarray(W["global_scale"])[e]), "K": W["K"], "N": W["N"]}


@pytest.mark.parametrize("codec", ["fp8", "nvfp4"])
@pytest.mark.parametrize("D,I", [(2048, 512), (512, 1024)])
def test_moe_codec_tile_row_boundaries(codec, D, I):
    """FP8 / NVFP4 grouped GEMMs on experts with 1, 31, 32, 33, 0, 97, 256
    and 300 rows (moe_dispatch on given ids, topk 1) and the shared expert:
    every act and ydown row against the oracle's codec FFN of its expert."""
    import torch
    from tests.gpu_util import assert_close
    from tests.test_gpu_moe import BOUNDARY_COUNTS, boundary_route, expert_rows_reference
    E = len(BOUNDARY_COUNTS)
    say(f"moe {codec} tile boundaries D={D} I={I}")
    ids = boundary_route(E, BOUNDARY_COUNTS, D + I + 9)
    T = ids.shape[0]
    if codec == "fp8":
        w = synth.moe_weights_fp8(D + I, D=D, I=I, E=E)
        dw, gemm, ffn, sl = _dev_weights(w), ql.moe_grouped_gemm_fp8, oracle.expert_ffn_fp8, _fp8_expert
    else:
        w = synth.moe_weights_nvfp4(D + I, D=D, I=I, E=E)
        dw, gemm, ffn, sl = _dev_weights_nvfp4(w), ql.moe_grouped_gemm_nvfp4, oracle.expert_ffn_nvfp4, _nvfp4_expert
    H = synth.moe_tokens(D + I + 1, T, D=D, E=E)["H"]
    route = ql.moe_dispatch(t(ids), E)
    act = gemm(dw["gate_up"], dw["shared_gate_up"], t(H), T, 1, ql.QL_OP_GATE_UP_SILU, route)
    yd = gemm(dw["down"], dw["shared_down"], act, T, 1, ql.QL_OP_DOWN, route)
    torch.cuda.synchronize()
    ref_act, ref_yd = expert_rows_reference(ids, host(route["sorted_assign"]), H, w, ffn, expert=sl)
    assert_close(host(act).astype(np.float64), ref_act.astype(np.float64), "act")
    assert_close(host(yd).astype(np.float64), ref_yd, "ydown")


def _codec_weights(codec, seed, **kw):
    if codec == "fp8":
        w = synth.moe_weights_fp8(seed, **kw)
        return w, _dev_weights(w), ql.moe_grouped_gemm_fp8, oracle.moe_layer_fp8
    w = synth.moe_weights_nvfp4(seed, **kw)
    return w, _dev_weights_nvfp4(w), ql.moe_grouped_gemm_nvfp4, oracle.moe_layer_nvfp4


@pytest.mark.parametrize("codec", ["fp8", "nvfp4"])
@pytest.mark.parametrize("T,D,I,E,topk,seed,shared", [
    (1, 2048, 512, 256, 8, 0, True),     # the decode shape
    (4, 2048, 512, 256, 8, 1, True),
    (2, 512, 256, 16, 4, 2, True),
    (3, 1024, 512, 32, 13, 3, True),     # 14 rows per token: two rounds for some waves
    (2, 2048, 512, 256, 8, 4, False),    # no shared expert
])
def test_moe_decode_codec(codec, T, D, I, E, topk, seed, shared):
    """moe_decode_fp8 / moe_decode_nvfp4 against the oracle's codec layer:
    routing exactly the oracle's (no token of these cases has two of its
    top-(k+1) logits within 1e-4), act and out within the fp16 bar; and the
    bits of the three-call path (moe_route, the codec grouped GEMM's gate/up
    rows and its QL_OP_DOWN_COMBINE)."""
    import torch
    from tests.gpu_util import assert_close
    from tests.test_gpu_moe import _ref_rows
    say(f"moe_decode_{codec} T={T} D={D} I={I} E={E} topk={topk} shared={shared}")
    w, dw, gemm, layer = _codec_weights(codec, seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 120, T, D=D, E=E, skewed=True)
    ref = layer(tok["H"], w, tok["logit_bias"], topk, with_shared=shared)
    assert not oracle.topk_near_ties(ref["logits"], topk, 1e-4).any(), "case not screened"
    H, bias = t(tok["H"]), t(tok["logit_bias"])
    sg = dw["shared_gate_up"] if shared else None
    sd = dw["shared_down"] if shared else None
    res = ql.moe_decode_codec(codec, H, dw["Wr"], bias, topk, dw["gate_up"], dw["down"], sg, sd)
    route = ql.moe_route(H, dw["Wr"], bias, topk)
    act = gemm(dw["gate_up"], sg, H, T, topk, ql.QL_OP_GATE_UP_SILU, route)
    out3 = gemm(dw["down"], sd, act, T, topk, ql.QL_OP_DOWN_COMBINE, route)
    torch.cuda.synchronize()
    assert np.array_equal(host(res["ids"]), ref["ids"])
    assert np.abs(host(res["gates"]).astype(np.float64) - ref["gates"]).max() < 2e-5
    _check_routing(route, ref)
    rows = _ref_rows(route, ref, T, topk)
    assert_close(host(act).astype(np.float64), ref["act"][rows].astype(np.float64), "act")
    rel, mx = assert_close(host(res["out"]).astype(np.float64), ref["out"], "out")
    say(f"  rel-L2 {rel:.2e} max-abs/max|ref| {mx:.2e}")
    assert np.array_equal(host(res["out"]).view(np.uint16), host(out3).view(np.uint16))


@pytest.mark.parametrize("codec", ["fp8", "nvfp4"])
def test_moe_decode_codec_reads_only_selected_experts(codec):
    """NaN in every expert the token did not choose (FP8: every code 0x7F;
    NVFP4: every block scale 0x7F) leaves the decode output finite and equal
    to the oracle's on the clean weights."""
    import torch
    from tests.gpu_util import assert_close
    w, _, _, layer = _codec_weights(codec, 8)
    tok = synth.moe_tokens(1008, 1)
    ref = layer(tok["H"], w, None, 8)
    chosen = set(ref["ids"][0].tolist())
    for key in ("gate_up", "down"):
        for e in range(256):
            if e not in chosen:
                if codec == "fp8":
                    w[key]["codes"][e] = 0x7F
                else:
                    w[key]["block_scales"][e] = 0x7F
    dw = _dev_weights(w) if codec == "fp8" else _dev_weights_nvfp4(w)
    res = ql.moe_decode_codec(codec, t(tok["H"]), dw["Wr"], None, 8, dw["gate_up"], dw["down"],
                              dw["shared_gate_up"], dw["shared_down"])
    torch.cuda.synchronize()
    assert_close(host(res["out"]).astype(np.float64), ref["out"], "out")


@pytest.mark.parametrize("codec", ["fp8", "nvfp4"])
@pytest.mark.parametrize("T", [600, 4096])
def test_moe_codec_shared_expert_split(codec, T):
    """The routed rows (shared = None) and the shared expert's rows
    (QL_OP_SHARED_ONLY, no routing inputs) as two launches into one buffer,
    the shared ones on a second stream: act and ydown equal the single
    launch's bit for bit."""
    import torch
    topk = 8
    say(f"{codec} shared-expert split T={T}")
    w = synth.moe_weights_fp8(0) if codec == "fp8" else synth.moe_weights_nvfp4(0)
    dw = _dev_weights(w) if codec == "fp8" else _dev_weights_nvfp4(w)
    gemm = ql.moe_grouped_gemm_fp8 if codec == "fp8" else ql.moe_grouped_gemm_nvfp4
    tk = synth.moe_tokens(SCREENED[0], T, skewed=True)
    H, b = t(tk["H"]), t(tk["logit_bias"])
    route, act, yd, _ = _run(dw, H, b, topk, T, shared=True, gemm=gemm)
    torch.cuda.synchronize()
    act2 = torch.full_like(act, float("nan"))
    yd2 = torch.full_like(yd, float("nan"))
    side = torch.cuda.Stream()
    fork = torch.cuda.Event()
    fork.record(torch.cuda.current_stream())
    side.wait_event(fork)
    with torch.cuda.stream(side):
        gemm(dw["gate_up"], dw["shared_gate_up"], H, T, topk, ql.QL_OP_GATE_UP_SILU | ql.QL_OP_SHARED_ONLY,
             None, act2, stream=side)
        gemm(dw["down"], dw["shared_down"], act, T, topk, ql.QL_OP_DOWN | ql.QL_OP_SHARED_ONLY, None, yd2,
             stream=side)
    gemm(dw["gate_up"], None, H, T, topk, ql.QL_OP_GATE_UP_SILU, route, act2)
    gemm(dw["down"], None, act, T, topk, ql.QL_OP_DOWN, route, yd2)
    torch.cuda.synchronize()
    assert np.array_equal(host(act2).view(np.uint16), host(act).view(np.uint16))
    assert np.array_equal(host(yd2).view(np.uint16), host(yd).view(np.uint16))
