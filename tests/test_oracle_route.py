"""Pins of the oracle's router and dispatch steps: hand-worked fixtures,
brute force over subsets on tiny E, a library sort, invariants."""
import itertools
import json
import os

import numpy as np
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_route_hand_fixture():
    for case in _load("route_hand.json")["cases"]:
        ids, gates = oracle.topk_route(np.array([case["logits"]]), case["topk"])
        assert ids[0].tolist() == case["ids"]
        assert np.allclose(gates[0], case["gates"], rtol=0, atol=1e-15)


def test_equal_logits_pick_lowest_indices():
    ids, gates = oracle.topk_route(np.zeros((3, 256)), 8)
    assert (ids == np.arange(8)).all()
    assert np.all(gates == 1.0 / 8)


def test_bruteforce_subsets_tiny_E():
    """The chosen set maximises the sum of logits over all k-subsets (logits
    distinct), and the gates equal scipy's softmax over the chosen logits."""
    rng = np.random.default_rng(0)
    for E, k in [(5, 2), (6, 3), (7, 1), (8, 8), (9, 4)]:
        L = rng.standard_normal((20, E))
        ids, gates = oracle.topk_route(L, k)
        for t in range(20):
            best = max(itertools.combinations(range(E), k), key=lambda S: sum(L[t, list(S)]))
            assert set(ids[t].tolist()) == set(best)
            ref = scipy.special.softmax(L[t, ids[t]])
            assert np.allclose(gates[t], ref, rtol=1e-13, atol=0)
            assert np.all(np.diff(L[t, ids[t]]) <= 0)


def test_route_invariants_and_shift():
    rng = np.random.default_rng(1)
    case = synth.moe_tokens(1, 64, D=64, E=32)
    Wr = synth.router_weight(rng, 64, 32)
    L = oracle.router_logits(case["H"], Wr)
    ids, gates = oracle.topk_route(L, 8)
    for t in range(64):
        assert len(set(ids[t].tolist())) == 8
    assert np.all(gates > 0)
    assert np.all(np.diff(gates, axis=1) <= 0)
    assert np.allclose(gates.sum(axis=1), 1.0, rtol=0, atol=1e-12)
    ids2, gates2 = oracle.topk_route(L + 3.25, 8)
    assert np.array_equal(ids, ids2) and np.allclose(gates, gates2, atol=1e-13)


def test_logit_bias_enters_choice_and_gates():
    H = np.zeros((2, 16), np.float16)
    Wr = np.zeros((16, 10), np.float16)
    bias = np.zeros(10, np.float32)
    bias[7] = 2.0
    bias[3] = 1.0
    L = oracle.router_logits(H, Wr, bias)
    ids, gates = oracle.topk_route(L, 2)
    assert ids[0].tolist() == [7, 3]
    assert np.allclose(gates[0], [np.e / (np.e + 1), 1 / (np.e + 1)], atol=1e-15)


def test_router_logits_library_matmul():
    rng = np.random.default_rng(4)
    H = synth.activations(rng, 5, 48)
    Wr = synth.router_weight(rng, 48, 12)
    L = oracle.router_logits(H, Wr)
    for t in range(5):
        for e in range(12):
            ref = sum(float(H[t, d]) * float(Wr[d, e]) for d in range(48))
            assert abs(L[t, e] - ref) < 1e-12


def test_near_ties_flags():
    L = np.array([[5.0, 4.0, 3.0, 2.99999, 1.0, 0.0]])
    near = oracle.topk_near_ties(L, 3, 1e-4)
    assert near[0].tolist() == [False, False, True]
    near = oracle.topk_near_ties(L, 4, 1e-4)
    assert near[0].tolist() == [False, False, True, True]


def test_dispatch_hand_fixture():
    c = _load("dispatch_hand.json")
    ids = np.array(c["ids"])
    counts = oracle.histogram(ids, c["E"])
    offsets = oracle.exclusive_scan(counts)
    sa, pos = oracle.stable_permutation(ids, c["E"])
    assert counts.tolist() == c["counts"]
    assert offsets.tolist() == c["offsets"]
    assert sa.tolist() == c["sorted_assign"]
    assert pos.tolist() == c["pos"]
    assert oracle.tile_map(counts, c["tile_rows"]).tolist() == c["tiles"]


def test_dispatch_invariants_and_library_sort():
    rng = np.random.default_rng(8)
    for T, E, k, skew in [(1, 256, 8, 0.0), (37, 16, 4, 1.1), (300, 256, 8, 1.1), (50, 8, 8, 0.0)]:
        ids = synth.synthetic_topk_ids(rng, T, E, k, skew)
        counts = oracle.histogram(ids, E)
        offsets = oracle.exclusive_scan(counts)
        sa, pos = oracle.stable_permutation(ids, E)
        flat = ids.ravel()
        assert counts.sum() == T * k and offsets[-1] == T * k
        assert np.all(np.diff(offsets) >= 0)
        assert np.array_equal(np.sort(sa), np.arange(T * k))
        assert np.array_equal(sa, np.argsort(flat, kind="stable"))   # library stable sort
        assert np.array_equal(pos[sa], np.arange(T * k))
        assert np.all(np.diff(flat[sa]) >= 0)
        for e in range(E):
            seg = sa[offsets[e]:offsets[e + 1]]
            assert np.all(np.diff(seg) > 0)
            assert np.all(flat[seg] == e)
        assert np.array_equal(counts, np.bincount(flat, minlength=E))
        for bm in (1, 32, 128):
            tiles = oracle.tile_map(counts, bm)
            assert len(tiles) <= (T * k) // bm + E
            per = np.zeros(E, np.int64)
            for e, r0, rows in tiles:
                assert 1 <= rows <= bm
                assert offsets[e] <= r0 and r0 + rows <= offsets[e + 1]
                per[e] += rows
            assert np.array_equal(per, counts)


def test_load_matched_tile_map_hand_fixture():
    c = _load("tiles_hand.json")
    for case in c["cases"]:
        got = oracle.load_matched_tile_map(case["counts"], c["small_rows"], c["big_rows"])
        assert got.tolist() == case["tiles"]


def test_load_matched_tile_map_invariants():
    """Brute force over random loads: every routed row is in exactly one
    tile of its own expert, tall tiles are full and come first, short tiles
    cover only what is left after the full tall tiles."""
    rng = np.random.default_rng(11)
    for T, E, k, skew in [(1, 256, 8, 0.0), (300, 256, 8, 1.1), (4096, 256, 8, 1.1), (50, 8, 8, 0.0),
                          (1000, 16, 4, 2.0)]:
        ids = synth.synthetic_topk_ids(rng, T, E, k, skew)
        counts = oracle.histogram(ids, E)
        offsets = oracle.exclusive_scan(counts)
        for small, big in ((128, 256), (2, 4), (32, 96)):
            tiles = oracle.load_matched_tile_map(counts, small, big)
            owner = np.full(T * k, -1)
            seen_short = False
            for e, r0, rows, h in tiles:
                assert h in (small, big) and 1 <= rows <= h
                if h == big:
                    assert not seen_short and rows == big
                else:
                    seen_short = True
                assert offsets[e] <= r0 and r0 + rows <= offsets[e + 1]
                assert np.all(owner[r0:r0 + rows] == -1)
                owner[r0:r0 + rows] = e
            flat = np.repeat(np.arange(E), counts)
            assert np.array_equal(owner, flat)
            for e in range(E):
                n_tall = sum(1 for t in tiles if t[0] == e and t[3] == big)
                n_short = sum(1 for t in tiles if t[0] == e and t[3] == small)
                assert n_tall == counts[e] // big
                assert n_short == -(-(counts[e] % big) // small)
            assert len(tiles) <= (T * k) // small + E


def test_tie_inputs_are_exact_in_float32():
    """The exact-tie router inputs used by the GPU tests: float32 products
    summed in a different order give the float64 logits bit for bit, the
    copied columns tie, and the oracle takes the tied experts lowest index
    first, with the cut inside the second group."""
    for seed, T, E, topk in [(0, 4, 256, 8), (3, 2, 1000, 32), (5, 3, 33, 32)]:
        c = synth.router_tie_case(seed, T, topk, E=E)
        L64 = oracle.router_logits(c["H"], c["Wr"])
        H32, W32 = c["H"].astype(np.float32), c["Wr"].astype(np.float32)
        L32 = np.zeros((T, E), dtype=np.float32)
        for d in range(H32.shape[1] - 1, -1, -1):  # reversed order
            L32 += H32[:, d:d + 1] * W32[d:d + 1, :]
        assert np.array_equal(L32.astype(np.float64), L64)
        assert np.all(L64[:, c["top"]] == L64[:, [c["top"][0]]])
        assert np.all(L64[:, c["edge"]] == L64[:, [c["edge"][0]]])
        ids, _ = oracle.topk_route(L64, topk)
        n_top = len(c["top"])
        assert np.array_equal(ids[:, :n_top], np.tile(c["top"], (T, 1)))
        assert np.array_equal(ids[:, n_top:], np.tile(c["edge"][:topk - n_top], (T, 1)))
