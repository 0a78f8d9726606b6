"""GPU parity of the routing steps: moe_dispatch on seeded synthetic ids
(bit-exact against the oracle), and moe_route end to end (fp32 logits on
the GPU against float64 logits in the oracle)."""
import json
import os

import numpy as np
import pytest

import bit_group_quantized_amd as ql
import oracle
import synth
from tests.gpu_util import guarded, host, say, t

pytestmark = pytest.mark.gpu

# A token whose exact logits put two of its top-(k+1) within TAU of each
# other may be ordered either way by fp32 accumulation (its error on these
# inputs is a few 1e-6); such positions are checked for validity only.
TAU = 1e-4


def _ws_tiles(out):
    ws = host(out["workspace"]).view(np.int32)
    n = int(ws[0])
    return ws[:8], ws[8:8 + 4 * n].reshape(n, 4)


def guarded_route_outputs(T, E, topk):
    """moe_route / moe_dispatch outputs carved out of guarded buffers; the
    second value checks every guard."""
    import torch
    g = {"ids": guarded((T, topk), torch.int32), "gates": guarded((T, topk), torch.float32),
         "counts": guarded((E,), torch.int32), "offsets": guarded((E + 1,), torch.int32),
         "sorted_assign": guarded((T * topk,), torch.int32), "pos": guarded((T * topk,), torch.int32),
         "workspace": guarded((max(ql.moe_workspace_bytes(T, E, topk), 256),), torch.uint8)}
    out = {k: v.t for k, v in g.items()}

    def check():
        for k, v in g.items():
            v.check(k)
    return out, check


def _check_dispatch(out, ids, E, T, topk):
    counts = oracle.histogram(ids, E)
    offsets = oracle.exclusive_scan(counts)
    sa, pos = oracle.stable_permutation(ids, E)
    assert np.array_equal(host(out["counts"]), counts)
    assert np.array_equal(host(out["offsets"]), offsets)
    assert np.array_equal(host(out["sorted_assign"]), sa)
    assert np.array_equal(host(out["pos"]), pos)
    hdr, tiles = _ws_tiles(out)
    ref = oracle.load_matched_tile_map(counts, ql.QL_MOE_TILE_ROWS, 2 * ql.QL_MOE_TILE_ROWS)
    assert hdr[1] == ql.QL_MOE_TILE_ROWS and hdr[2] == 0
    assert hdr[3] == int(np.sum(ref[:, 3] == 2 * ql.QL_MOE_TILE_ROWS))
    assert np.array_equal(tiles, ref)


@pytest.mark.parametrize("T,E,topk,skew,seed", [
    (1, 256, 8, 0.0, 0), (3, 256, 8, 0.0, 1), (16, 256, 8, 1.1, 2), (17, 256, 8, 1.1, 3),
    (300, 256, 8, 1.1, 4), (4096, 256, 8, 1.1, 5), (4096, 256, 8, 0.0, 6),
    (257, 8, 8, 0.0, 7), (1000, 1000, 2, 0.5, 8), (513, 64, 1, 2.0, 9), (40, 33, 32, 0.0, 10),
    (32, 256, 8, 0.0, 11), (33, 256, 8, 1.1, 12),   # one full 32-token mask chunk, and one more token
    (4097, 256, 8, 1.1, 13), (2000, 1000, 4, 0.5, 14), (9000, 64, 2, 1.1, 15),  # masks past one block's LDS
])
def test_dispatch_bit_exact(T, E, topk, skew, seed):
    import torch
    say(f"dispatch T={T} E={E} topk={topk} skew={skew}")
    rng = np.random.default_rng(seed)
    ids = synth.synthetic_topk_ids(rng, T, E, topk, skew)
    out, check = guarded_route_outputs(T, E, topk)
    ql.moe_dispatch(t(ids), E, out)
    torch.cuda.synchronize()
    check()
    _check_dispatch(out, ids, E, T, topk)


@pytest.mark.parametrize("T,E,topk", [(300, 256, 8), (5000, 256, 8)])
def test_dispatch_invalid_ids_set_the_error_flag(T, E, topk):
    """Ids out of range or repeated within a token (both dispatch paths:
    masks in one block's LDS, and the three-launch path for more tokens)
    set the workspace error flag and write nothing outside the outputs."""
    import torch
    rng = np.random.default_rng(T)
    ids = synth.synthetic_topk_ids(rng, T, E, topk, 0.0)
    ids[7, 3] = E + 5          # out of range
    ids[11, 2] = ids[11, 1]    # repeated within token 11
    ids[T - 1, 0] = -1         # negative
    out, check = guarded_route_outputs(T, E, topk)
    ql.moe_dispatch(t(ids), E, out)
    torch.cuda.synchronize()
    check()
    hdr, _ = _ws_tiles(out)
    assert hdr[2] != 0
    pos = host(out["pos"]).reshape(T, topk)
    assert pos[7, 3] == -1 and pos[T - 1, 0] == -1
    valid = (ids >= 0) & (ids < E)
    assert np.all((pos[valid] >= 0) & (pos[valid] < T * topk))


def test_dispatch_one_hot_load():
    """Every token picks experts 0..7: eight experts hold all rows, the
    others none."""
    import torch
    T, E, topk = 1000, 256, 8
    ids = np.tile(np.arange(topk, dtype=np.int32), (T, 1))
    out = ql.moe_dispatch(t(ids), E)
    torch.cuda.synchronize()
    _check_dispatch(out, ids, E, T, topk)


def _check_route(out, H, Wr, bias, topk, T, E):
    L64 = oracle.router_logits(H, Wr, bias)
    ids_ref, gates_ref = oracle.topk_route(L64, topk)
    ids = host(out["ids"])
    gates = host(out["gates"]).astype(np.float64)
    # logits written by the GPU into the workspace (fp32)
    off = ql.ql_moe_logits_offset(T, E, topk)
    Lg = host(out["workspace"])[off:off + 4 * T * E].view(np.float32).reshape(T, E)
    # The seed screen (tests/golden/screen_prefill_seeds.py) relies on this bound.
    assert np.abs(Lg - L64).max() < 2e-5
    near = oracle.topk_near_ties(L64, topk, TAU)
    srt = -np.sort(-L64, axis=1)[:, :topk]
    for tt in range(T):
        assert len(set(ids[tt].tolist())) == topk
        for j in range(topk):
            if near[tt, j]:
                assert abs(L64[tt, ids[tt, j]] - srt[tt, j]) <= TAU
            else:
                assert ids[tt, j] == ids_ref[tt, j], (tt, j)
    assert np.abs(gates - gates_ref).max() < 2e-5
    assert np.allclose(gates.sum(axis=1), 1.0, atol=1e-5)
    return np.array_equal(ids, ids_ref), near, ids_ref


def _check_dispatch_properties(out, ids, E, T, topk):
    """Where near ties let the GPU pick another valid expert set, the integer
    steps are checked as properties of the ids it picked (no oracle run on
    GPU data)."""
    flat = ids.ravel()
    counts = host(out["counts"])
    offsets = host(out["offsets"])
    sa = host(out["sorted_assign"])
    pos = host(out["pos"])
    assert np.array_equal(counts, np.bincount(flat, minlength=E))
    assert offsets[0] == 0 and np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(sa, np.argsort(flat, kind="stable"))
    assert np.array_equal(pos[sa], np.arange(T * topk))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_route_decode_token(seed):
    import torch
    w = synth.moe_weights(seed)
    tok = synth.moe_tokens(seed + 1000, 1)
    out = ql.moe_route(t(tok["H"]), t(w["Wr"]), None, 8)
    torch.cuda.synchronize()
    exact, near, ids_ref = _check_route(out, tok["H"], w["Wr"], None, 8, 1, 256)
    assert exact and not near.any()
    _check_dispatch(out, ids_ref, 256, 1, 8)


_SEEDS = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "prefill_seeds.json")))
SCREENED = _SEEDS["kept_seeds_by_gap"]
# Seeds whose every adjacent gap among a token's 9 largest exact logits
# exceeds 2e-5 (tests/golden/screen_prefill_seeds.py); with an fp32 logit
# error below 1e-5 (asserted) every routing decision, order included, is
# determined.
FULL_ORDER = _SEEDS["kept_seeds_full_order"]
FULL_ORDER_LOGIT_ERR = 1e-5


@pytest.mark.parametrize("T,skewed,seed,screened", [
    (4096, True, FULL_ORDER[0], True), (4096, True, FULL_ORDER[1], True),
    (4096, True, SCREENED[0], False), (4096, True, 2, False), (333, False, 3, False),
    (16, True, 4, False)])
def test_route_prefill(T, skewed, seed, screened):
    """moe_route on the prefill workload.  On the full-order screened seeds
    (every adjacent gap among a token's 9 largest exact logits above 2e-5,
    tests/golden/screen_prefill_seeds.py) the GPU's fp32 logits must lie
    within 1e-5 of the exact ones, and then the ids (in order), counts,
    offsets, permutation, inverse and tile map must equal the oracle's bit
    for bit; elsewhere near-tied positions are checked for validity."""
    import torch
    say(f"route T={T} skewed={skewed} seed={seed} screened={screened}")
    w = synth.moe_weights(0)
    tok = synth.moe_tokens(seed, T, skewed=skewed)
    bias_dev = t(tok["logit_bias"]) if skewed else None
    out, check = guarded_route_outputs(T, 256, 8)
    ql.moe_route(t(tok["H"]), t(w["Wr"]), bias_dev, 8, out)
    torch.cuda.synchronize()
    check()
    exact, near, ids_ref = _check_route(out, tok["H"], w["Wr"], tok["logit_bias"], 8, T, 256)
    say(f"  near-tie positions: {int(near.sum())}, ids identical: {exact}")
    if screened:
        off = ql.ql_moe_logits_offset(T, 256, 8)
        Lg = host(out["workspace"])[off:off + 4 * T * 256].view(np.float32).reshape(T, 256)
        L64 = oracle.router_logits(tok["H"], w["Wr"], tok["logit_bias"])
        err = float(np.abs(Lg - L64).max())
        say(f"  fp32 logit error {err:.2e}")
        assert err < FULL_ORDER_LOGIT_ERR
        assert exact, "routing ids differ from the oracle's on a full-order screened seed"
    if exact:
        _check_dispatch(out, ids_ref, 256, T, 8)
    else:
        _check_dispatch_properties(out, host(out["ids"]), 256, T, 8)
    # Without a near tie at the k/k+1 boundary the chosen sets must agree.
    if not near[:, -1].any():
        assert all(set(a) == set(b) for a, b in zip(host(out["ids"]).tolist(), ids_ref.tolist()))


@pytest.mark.parametrize("T,E,topk,skewed,seed", [
    (4096, 256, 8, True, 0), (4096, 256, 8, True, 1), (4096, 256, 8, False, 2),
    (1, 256, 8, True, 3), (4, 256, 8, True, 4), (16, 256, 8, True, 5), (17, 256, 8, True, 6),
    (777, 256, 8, True, 7),
])
def test_route_exact_arithmetic_every_token(T, E, topk, skewed, seed):
    """Routing on inputs whose fp32 logits are exact (synth.router_exact_case:
    the GPU's logits then equal the oracle's float64 logits bit for bit), so
    the oracle's top-k, histogram, scan, permutation and tile map are the
    only correct answer for every token, exact ties and near ties included:
    everything must match bit for bit, on the many-token MFMA router and on
    the small-T path."""
    import torch
    say(f"route exact arithmetic T={T} skewed={skewed} seed={seed}")
    c = synth.router_exact_case(seed, T, E=E, skewed=skewed)
    L64 = oracle.router_logits(c["H"], c["Wr"], c["logit_bias"])
    ids_ref, gates_ref = oracle.topk_route(L64, topk)
    srt = -np.sort(-L64, axis=1)
    n_ties = int(np.sum(srt[:, topk - 1] == srt[:, topk]))
    out, check = guarded_route_outputs(T, E, topk)
    ql.moe_route(t(c["H"]), t(c["Wr"]), t(c["logit_bias"]) if skewed else None, topk, out)
    torch.cuda.synchronize()
    check()
    say(f"  tokens with an exact tie across the top-k cut: {n_ties}")
    off = ql.ql_moe_logits_offset(T, E, topk)
    Lg = host(out["workspace"])[off:off + 4 * T * E].view(np.float32).reshape(T, E)
    assert np.array_equal(Lg.astype(np.float64), L64)
    assert np.array_equal(host(out["ids"]), ids_ref)
    assert np.abs(host(out["gates"]).astype(np.float64) - gates_ref).max() < 2e-6
    _check_dispatch(out, ids_ref, E, T, topk)


@pytest.mark.parametrize("T,E,topk,seed", [
    (1, 256, 8, 0), (16, 256, 8, 1), (300, 256, 8, 2), (1, 1000, 32, 3), (40, 1000, 32, 4),
    (3, 33, 32, 5), (50, 33, 32, 6), (2, 64, 1, 7), (20, 200, 5, 8),
    (3, 1024, 32, 9), (100, 1024, 32, 10),  # QL_MAX_EXPERTS and QL_MAX_TOPK
])
def test_route_exact_ties(T, E, topk, seed):
    """Logits exact in fp32 with equal values at the top and across the
    top-k cut: the selection must follow (logit descending, index
    ascending) exactly, on every router and top-k path."""
    import torch
    say(f"route ties T={T} E={E} topk={topk}")
    c = synth.router_tie_case(seed, T, topk, E=E)
    out = ql.moe_route(t(c["H"]), t(c["Wr"]), None, topk)
    torch.cuda.synchronize()
    L64 = oracle.router_logits(c["H"], c["Wr"])
    ids_ref, gates_ref = oracle.topk_route(L64, topk)
    assert np.array_equal(host(out["ids"]), ids_ref)
    assert np.abs(host(out["gates"]).astype(np.float64) - gates_ref).max() < 2e-5
    off = ql.ql_moe_logits_offset(T, E, topk)
    Lg = host(out["workspace"])[off:off + 4 * T * E].view(np.float32).reshape(T, E)
    assert np.array_equal(Lg.astype(np.float64), L64)
    _check_dispatch(out, ids_ref, E, T, topk)


@pytest.mark.parametrize("T,E,topk", [(1, 256, 8), (64, 256, 8), (5, 1000, 32)])
def test_route_all_logits_equal(T, E, topk):
    """A zero router: every logit is 0, so experts 0..topk-1 win with equal
    gates."""
    import torch
    say(f"route all-equal T={T} E={E} topk={topk}")
    H = synth.activations(synth.rng_for(11), T, 2048)
    Wr = np.zeros((2048, E), dtype=np.float16)
    out = ql.moe_route(t(H), t(Wr), None, topk)
    torch.cuda.synchronize()
    ids = host(out["ids"])
    assert np.array_equal(ids, np.tile(np.arange(topk, dtype=np.int32), (T, 1)))
    assert np.abs(host(out["gates"]) - 1.0 / topk).max() < 1e-6
    _check_dispatch(out, ids, E, T, topk)


def test_route_workspace_reuse_across_sizes():
    """One workspace serves a sequence of routes of different sizes (small-T
    and many-token paths alternating); every call matches the oracle."""
    import torch
    say("route workspace reuse T = 1, 16, 5, 300, 1, 9")
    w = synth.moe_weights(3)
    big = ql.alloc_route_outputs(300, 256, 8, torch.device("cuda"))
    for i, T in enumerate((1, 16, 5, 300, 1, 9)):
        tok = synth.moe_tokens(5000 + i, T, skewed=True)
        out = dict(big)
        out["ids"] = big["ids"][:T]
        out["gates"] = big["gates"][:T]
        out["sorted_assign"] = big["sorted_assign"][: T * 8]
        out["pos"] = big["pos"][: T * 8]
        ql.moe_route(t(tok["H"]), t(w["Wr"]), t(tok["logit_bias"]), 8, out)
        torch.cuda.synchronize()
        exact, near, ids_ref = _check_route(out, tok["H"], w["Wr"], tok["logit_bias"], 8, T, 256)
        if exact:
            _check_dispatch(out, ids_ref, 256, T, 8)
        else:
            _check_dispatch_properties(out, host(out["ids"]), 256, T, 8)
