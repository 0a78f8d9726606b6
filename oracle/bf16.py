"""bf16 variant of the group-affine 4-bit linear layer: bf16 scale, bias,
activations and outputs.

Test infrastructure only (see the package docstring).

Perplexity, "Optimizing on-device inference for Apple Silicon", section
"在矩阵乘法期间进行权重反量化": the page's checkpoint keeps the per-group
scale and bias in bfloat16 and the matrix path multiplies bf16 operands.
The reconstruction is the same as in w4.py, w = scale * code + bias per
group of 64 along K; only the 16-bit type changes.  The routed-expert layer
(moe_layer_bf16) is moe.moe_layer with bf16 tokens, router weight and
expert scales/biases, and its 16-bit intermediate (act) rounded to bf16.

numpy has no bf16 type, so bf16 values are carried as uint16 bit patterns
(the upper half of the float32 pattern) and decoded exactly.

Readings taken where the page is silent (as in w4.py, plus):
* rounding to bf16 is to nearest, ties to even, on 8 significant bits;
  beyond the largest finite bf16 the result is infinite; below 2**-126 the
  grid is the subnormal one (2**-133); NaN becomes the quiet NaN 0x7FC0;
* the linear layer's exact result is the fp64 sum of x * (scale * code +
  bias) with the bf16 inputs decoded exactly; rounding of the dequantized
  weights or of the output belongs to the GPU path and is covered by its
  tolerance, not modelled here.
"""
from __future__ import annotations

import numpy as np

from .moe import combine, silu
from .route import (exclusive_scan, histogram, router_logits, stable_permutation,
                    topk_route)
from .w4 import GROUP, unpack_codes

_BF16_MAX = (2.0 - 2.0 ** -7) * 2.0 ** 127


def bf16_to_f64(bits) -> np.ndarray:
    """uint16 bf16 patterns -> float64, exactly (a bf16 is the upper half of
    a float32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_bf16(a) -> np.ndarray:
    """float64 -> uint16 bf16 patterns, round to nearest even."""
    a = np.asarray(a, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        m, e = np.frexp(a)                    # a = m * 2**e, 0.5 <= |m| < 1
        val = np.ldexp(np.rint(m * 256.0), e - 8)   # 8 significant bits
        sub = np.abs(a) < 2.0 ** -126
        val = np.where(sub, np.rint(a / 2.0 ** -133) * 2.0 ** -133, val)
        val = np.where(np.abs(val) > _BF16_MAX, np.copysign(np.inf, a), val)
    bits = (val.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    return np.where(np.isnan(a), np.uint16(0x7FC0), bits).astype(np.uint16)


def dequantize_bf16(qweight, scales_bits, biases_bits, K: int) -> np.ndarray:
    """float64 [..., N, K] with W[n][k] = scale*code + bias, scale and bias
    given as bf16 patterns [..., N, K/64].  Exact: an 8-bit scale times a
    4-bit code plus an 8-bit bias fits easily in 53 bits."""
    if K % GROUP:
        raise ValueError("K must be a multiple of the group size 64")
    q = unpack_codes(qweight, K).astype(np.float64)
    s = np.repeat(bf16_to_f64(scales_bits), GROUP, axis=-1)
    b = np.repeat(bf16_to_f64(biases_bits), GROUP, axis=-1)
    assert s.shape == q.shape and b.shape == q.shape
    return s * q + b


def linear_bf16(X_bits, W: dict, row_chunk: int = 8192) -> np.ndarray:
    """Y[m][n] = sum_k X[m][k] * W[k][n] in float64 for bf16 X [M][K] (bit
    patterns) and a w4 matrix dict whose scales and biases are bf16 patterns.
    Output columns are processed in chunks as in w4.linear."""
    X = bf16_to_f64(np.atleast_2d(np.asarray(X_bits, dtype=np.uint16)))
    K, N = W["K"], W["N"]
    assert X.shape[1] == K
    Y = np.empty((X.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        Wd = dequantize_bf16(W["qweight"][n0:n1], W["scales"][n0:n1], W["biases"][n0:n1], K)
        Y[:, n0:n1] = X @ Wd.T
    return Y


def expert_ffn_bf16(X_bits, gate_up: dict, down: dict):
    """One expert on bf16 rows X [R][D]: u = X . Wgu in float64; act =
    bf16(SiLU(u[:, :I]) * u[:, I:]) (bf16 patterns, the 16-bit intermediate
    of the layer); ydown = act . Wdn in float64."""
    X = bf16_to_f64(np.atleast_2d(np.asarray(X_bits, dtype=np.uint16)))
    I = gate_up["N"] // 2
    Wgu = dequantize_bf16(gate_up["qweight"], gate_up["scales"], gate_up["biases"], gate_up["K"])
    u = X @ Wgu.T
    act = round_bf16(silu(u[:, :I]) * u[:, I:])
    Wdn = dequantize_bf16(down["qweight"], down["scales"], down["biases"], down["K"])
    ydown = bf16_to_f64(act) @ Wdn.T
    return act, ydown


def moe_layer_bf16(H_bits, weights: dict, logit_bias=None, topk: int = 8,
                   with_shared: bool = True) -> dict:
    """The routed-expert layer of moe.moe_layer with bf16 tokens H (patterns
    [T][D]), router weight and expert scales/biases: the same routing
    (logits from the exactly decoded bf16 values, fp64), dispatch and
    combine; act is rounded to bf16.  Returns logits, ids, gates, counts,
    offsets, sorted_assign, pos, act (bf16 patterns), ydown and out (float64).
    """
    H_bits = np.asarray(H_bits, dtype=np.uint16)
    T = H_bits.shape[0]
    E = weights["Wr"].shape[1]
    logits = router_logits(bf16_to_f64(H_bits), bf16_to_f64(weights["Wr"]), logit_bias)
    ids, gates = topk_route(logits, topk)
    counts = histogram(ids, E)
    offsets = exclusive_scan(counts)
    sorted_assign, pos = stable_permutation(ids, E)

    I = weights["gate_up"]["N"] // 2
    D = weights["down"]["N"]
    R = T * topk + (T if with_shared else 0)
    act = np.zeros((R, I), dtype=np.uint16)
    ydown = np.zeros((R, D), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        tokens = sorted_assign[r0:r1] // topk
        one = lambda W: {k: (v[e] if isinstance(v, np.ndarray) else v) for k, v in W.items()}
        a, y = expert_ffn_bf16(H_bits[tokens], one(weights["gate_up"]), one(weights["down"]))
        act[r0:r1] = a
        ydown[r0:r1] = y
    if with_shared:
        a, y = expert_ffn_bf16(H_bits, weights["shared_gate_up"], weights["shared_down"])
        act[T * topk:] = a
        ydown[T * topk:] = y
    out = combine(ydown, gates, pos, T, topk, with_shared)
    return {"logits": logits, "ids": ids, "gates": gates, "counts": counts,
            "offsets": offsets, "sorted_assign": sorted_assign, "pos": pos,
            "act": act, "ydown": ydown, "out": out}
