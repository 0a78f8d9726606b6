"""Pins of the oracle's MoE layer: a library sigmoid, a per-token brute
force that never permutes rows, and two closed forms over specially built
expert sets."""
import numpy as np
import scipy.special

import oracle
import synth


def test_silu_library_and_limits():
    z = np.linspace(-30, 30, 1001)
    assert np.allclose(oracle.silu(z), z * scipy.special.expit(z), rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu(-1000.0) == 0.0
    assert oracle.silu(1000.0) == 1000.0


def _tiny(seed, T=5, D=64, I=64, E=6):
    w = synth.moe_weights(seed, D=D, I=I, E=E)
    tok = synth.moe_tokens(seed + 100, T, D=D, E=E, skewed=True)
    return w, tok


def _expert(Wstack, e):
    return {k: (v[e] if isinstance(v, np.ndarray) else v) for k, v in Wstack.items()}


def _ffn_one_token(h, gu, dn):
    u = oracle.linear(h, gu)[0]
    I = gu["N"] // 2
    act = oracle.round_f16(oracle.silu(u[:I]) * u[I:])
    return oracle.linear(act, dn)[0]


def test_moe_layer_matches_per_token_bruteforce():
    """Token by token: route, run each chosen expert on that token alone,
    weight, add the shared expert.  No histogram, scan or permutation."""
    for seed, topk in [(0, 2), (1, 3), (2, 6)]:
        w, tok = _tiny(seed)
        res = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk=topk)
        L = oracle.router_logits(tok["H"], w["Wr"], tok["logit_bias"])
        for t in range(tok["H"].shape[0]):
            p = oracle.softmax(L[t:t + 1])[0]
            chosen = sorted(range(len(p)), key=lambda e: (-p[e], e))[:topk]
            g = p[chosen] / p[chosen].sum()
            ref = _ffn_one_token(tok["H"][t], w["shared_gate_up"], w["shared_down"])
            for gj, e in zip(g, chosen):
                ref = ref + gj * _ffn_one_token(tok["H"][t], _expert(w["gate_up"], e), _expert(w["down"], e))
            assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


def test_identical_experts_give_twice_the_ffn():
    """All routed experts equal to the shared one: gates sum to 1, so
    out = 2 * FFN(h) whatever the routing."""
    w, tok = _tiny(3, T=7, E=5)
    E = 5
    for key, skey in (("gate_up", "shared_gate_up"), ("down", "shared_down")):
        for f in ("qweight", "scales", "biases"):
            w[key][f] = np.repeat(w[skey][f][None], E, axis=0)
    res = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk=3)
    for t in range(7):
        ref = 2 * _ffn_one_token(tok["H"][t], w["shared_gate_up"], w["shared_down"])
        assert np.allclose(res["out"][t], ref, rtol=1e-12, atol=1e-12)


def test_power_of_two_scaled_experts_pin_gate_to_id():
    """Expert e's down projection = 2^(e % 4) times a common one (scales and
    biases scaled by a power of two, exact in fp16), all gate_up equal:
    out[t] = (sum_j g_j 2^(id_j % 4)) * base(t) + shared(t)."""
    E = 6
    w, tok = _tiny(4, T=6, E=E)
    for f in ("qweight", "scales", "biases"):
        w["gate_up"][f] = np.repeat(w["shared_gate_up"][f][None], E, axis=0)
        w["down"][f] = np.repeat(w["shared_down"][f][None], E, axis=0)
    for e in range(E):
        for f in ("scales", "biases"):
            w["down"][f][e] = (w["down"][f][e].astype(np.float64) * 2 ** (e % 4)).astype(np.float16)
    res = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk=3)
    for t in range(6):
        base = _ffn_one_token(tok["H"][t], w["shared_gate_up"], w["shared_down"])
        factor = sum(res["gates"][t, j] * 2 ** (res["ids"][t, j] % 4) for j in range(3))
        assert np.allclose(res["out"][t], factor * base + base, rtol=1e-12, atol=1e-12)


def test_without_shared_expert():
    w, tok = _tiny(5, T=4, E=6)
    res = oracle.moe_layer(tok["H"], w, tok["logit_bias"], topk=2, with_shared=False)
    assert res["act"].shape[0] == 4 * 2
    ref = oracle.combine(res["ydown"], res["gates"], res["pos"], 4, 2, False)
    assert np.array_equal(ref, res["out"])
