"""Routed-expert MoE layer: expert FFN with gated activation, shared expert,
gate-weighted combine.

Test infrastructure only (see the package docstring).

Perplexity, "Optimizing on-device inference for Apple Silicon":

* "Qwen 创建了三种不同的工作负载形状": every token uses its 8 routed experts
  plus one shared expert that processes every token.
* "减少中间状态和流量": the decode path fuses the two expert input
  projections with the gated activation, and the expert output projection
  with the routing scores and the shared expert's result.
* "在矩阵乘法期间进行权重反量化": the expert matmuls accumulate in 32-bit
  floating point and write 16-bit outputs.

Readings taken where the pages are silent:

* the two input projections are one concatenated w4 matrix (gate_up,
  N = 2*I): columns [0, I) are the gate, [I, 2I) the up projection, and the
  gated activation is SiLU(gate) * up with SiLU(z) = z / (1 + exp(-z));
* the activation is a 16-bit GEMM output, so it is rounded to fp16 before
  the down projection;
* the shared expert has the same shape and is added with weight 1 (neither
  the pages nor the workload give it a gate);
* rows are kept in the expert-sorted order of the stable permutation
  (routed rows 0 .. T*topk-1), followed by the T shared rows in token order.
"""
from __future__ import annotations

import numpy as np

from .w4 import dequantize, round_f16
from .route import (router_logits, topk_route, histogram, exclusive_scan,
                    stable_permutation)


def silu(z) -> np.ndarray:
    """z * sigmoid(z) = z / (1 + exp(-z)) in float64."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def _expert(Wstack: dict, e: int) -> dict:
    return {"qweight": Wstack["qweight"][e], "scales": Wstack["scales"][e],
            "biases": Wstack["biases"][e], "K": Wstack["K"], "N": Wstack["N"]}


def expert_ffn(X, gate_up: dict, down: dict):
    """One expert on fp16 rows X [R][D].

    Returns (act fp16 [R][I], ydown float64 [R][D]) with
    u = X @ W_gu, act = fp16(SiLU(u[:, :I]) * u[:, I:]), ydown = act @ W_dn.
    """
    X = np.asarray(X).astype(np.float64)
    I2 = gate_up["N"]
    I = I2 // 2
    Wgu = dequantize(gate_up["qweight"], gate_up["scales"], gate_up["biases"], gate_up["K"])
    u = X @ Wgu.T
    act = round_f16(silu(u[:, :I]) * u[:, I:])
    Wdn = dequantize(down["qweight"], down["scales"], down["biases"], down["K"])
    ydown = act.astype(np.float64) @ Wdn.T
    return act, ydown


def combine(ydown, gates, pos, T: int, topk: int, has_shared: bool) -> np.ndarray:
    """float64 [T][N]: out[t] = sum_j gates[t][j] * ydown[pos[t*topk + j]]
    (+ ydown[T*topk + t] when a shared expert is present)."""
    ydown = np.asarray(ydown, dtype=np.float64)
    gates = np.asarray(gates, dtype=np.float64)
    out = np.zeros((T, ydown.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(topk):
            out[t] += gates[t, j] * ydown[pos[t * topk + j]]
        if has_shared:
            out[t] += ydown[T * topk + t]
    return out


def moe_layer(H, weights: dict, logit_bias=None, topk: int = 8,
              with_shared: bool = True) -> dict:
    """The whole routed-expert layer on fp16 tokens H [T][D].

    ``weights`` holds Wr [D][E] fp16, gate_up / down (experts stacked on the
    first axis) and shared_gate_up / shared_down.  Returns every
    intermediate: logits, ids, gates, counts, offsets, sorted_assign, pos,
    act [T*topk (+T)][I] fp16, ydown [T*topk (+T)][D] float64, out float64.
    Only the experts that received rows are dequantized.
    """
    H = np.asarray(H)
    T = H.shape[0]
    E = weights["Wr"].shape[1]
    logits = router_logits(H, weights["Wr"], logit_bias)
    ids, gates = topk_route(logits, topk)
    counts = histogram(ids, E)
    offsets = exclusive_scan(counts)
    sorted_assign, pos = stable_permutation(ids, E)

    I = weights["gate_up"]["N"] // 2
    D = weights["down"]["N"]
    R = T * topk + (T if with_shared else 0)
    act = np.zeros((R, I), dtype=np.float16)
    ydown = np.zeros((R, D), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        tokens = sorted_assign[r0:r1] // topk
        a, y = expert_ffn(H[tokens], _expert(weights["gate_up"], e), _expert(weights["down"], e))
        act[r0:r1] = a
        ydown[r0:r1] = y
    if with_shared:
        a, y = expert_ffn(H, weights["shared_gate_up"], weights["shared_down"])
        act[T * topk:] = a
        ydown[T * topk:] = y
    out = combine(ydown, gates, pos, T, topk, with_shared)
    return {"logits": logits, "ids": ids, "gates": gates, "counts": counts,
            "offsets": offsets, "sorted_assign": sorted_assign, "pos": pos,
            "act": act, "ydown": ydown, "out": out}
