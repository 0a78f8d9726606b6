"""Second weight codecs for the single-row linear layer: FP8-E4M3 weights
and NVFP4 (E2M1 values with E4M3 block scales).

Test infrastructure only (see the package docstring).

Pages followed: "待验证｜lithos-metal补Apple推理内核", section
"一分钟内合并了什么" (what merged in one minute): lithos-metal decodes FP8
E4M3 weights, two codes per half2, and serves an NVFP4 checkpoint of a
Qwen model.  The pages name the formats but do not spell them out; the
readings below take the published definitions of the two formats.

Readings:
* E4M3 is the FN variant: 1 sign bit, 4 exponent bits with bias 7, 3
  mantissa bits; exponent 0 holds the subnormals m/8 * 2**-6; S.1111.111
  is NaN; there is no infinity; the largest value is 448;
* FP8 weights carry one fp16 scale per 64 consecutive k of one output (the
  group layout of the w4 format, without a bias): w = e4m3(code) * scale;
* E2M1: 1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit; the eight
  magnitudes are 0, 0.5, 1, 1.5, 2, 3, 4, 6;
* NVFP4 weights: E2M1 codes packed 8 per uint32 exactly as the w4 codes,
  one E4M3 block scale per 16 consecutive k of one output and one fp32
  scale for the whole matrix: w = e2m1(code) * e4m3(block scale) * global;
* an FP8 (or NVFP4) routed-expert layer stores every expert matrix (and
  the shared expert's) in that format, stacked over experts, an NVFP4
  expert with a global scale of its own; routing, the gated activation
  (rounded to fp16), the row order and the combine are those of the w4
  layer in oracle.moe.
"""
from __future__ import annotations

import numpy as np

from .w4 import unpack_codes, round_f16
from .moe import silu, combine
from .route import (router_logits, topk_route, histogram, exclusive_scan,
                    stable_permutation)

FP8_GROUP = 64
NVFP4_BLOCK = 16


def e4m3_to_f64(codes) -> np.ndarray:
    """uint8 E4M3FN codes -> float64 (NaN for S.1111.111)."""
    b = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(b & 0x80, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = (b & 0x7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    sub = (m / 8.0) * 2.0 ** -6
    v = s * np.where(e == 0, sub, normal)
    return np.where((b & 0x7F) == 0x7F, np.nan, v)


def e2m1_to_f64(nibbles) -> np.ndarray:
    """4-bit E2M1 codes (0..15) -> float64."""
    n = np.asarray(nibbles, dtype=np.int64)
    s = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = (n & 0x1).astype(np.float64)
    mag = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0))
    return s * mag


def dequantize_fp8(codes, scales) -> np.ndarray:
    """float64 [N, K]: e4m3(code[n][k]) * scale[n][k // 64] (exact)."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    if K % FP8_GROUP:
        raise ValueError("K must be a multiple of 64")
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), FP8_GROUP, axis=-1)
    assert s.shape == codes.shape
    return e4m3_to_f64(codes) * s


def dequantize_nvfp4(qweight, block_scales, global_scale: float, K: int) -> np.ndarray:
    """float64 [N, K]: e2m1(code) * e4m3(block_scale[n][k // 16]) * global."""
    if K % NVFP4_BLOCK:
        raise ValueError("K must be a multiple of 16")
    q = e2m1_to_f64(unpack_codes(qweight, K))
    bs = np.repeat(e4m3_to_f64(block_scales), NVFP4_BLOCK, axis=-1)
    assert bs.shape == q.shape
    return q * bs * float(np.float32(global_scale))


def linear_fp8(X, W: dict, row_chunk: int = 8192) -> np.ndarray:
    """Y = X . W in float64 for fp16 X [M][K] and an FP8 weight dict
    (codes uint8 [N][K], scales fp16 [N][K/64])."""
    X = np.atleast_2d(np.asarray(X)).astype(np.float64)
    N = W["N"]
    Y = np.empty((X.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        Y[:, n0:n1] = X @ dequantize_fp8(W["codes"][n0:n1], W["scales"][n0:n1]).T
    return Y


def linear_nvfp4(X, W: dict, row_chunk: int = 8192) -> np.ndarray:
    """Y = X . W in float64 for fp16 X [M][K] and an NVFP4 weight dict
    (qweight uint32 [N][K/8], block_scales uint8 [N][K/16], global_scale)."""
    X = np.atleast_2d(np.asarray(X)).astype(np.float64)
    K, N = W["K"], W["N"]
    Y = np.empty((X.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        Wd = dequantize_nvfp4(W["qweight"][n0:n1], W["block_scales"][n0:n1], W["global_scale"], K)
        Y[:, n0:n1] = X @ Wd.T
    return Y


def _expert_ffn(X, Wgu, Wdn):
    """One expert on fp16 rows X [R][D] with exact (float64) weights Wgu
    [2I][D] and Wdn [D][I]: u = X @ Wgu^T, act = fp16(SiLU(u[:, :I]) * u[:, I:]),
    ydown = act @ Wdn^T."""
    X = np.asarray(X).astype(np.float64)
    I = Wgu.shape[0] // 2
    u = X @ Wgu.T
    act = round_f16(silu(u[:, :I]) * u[:, I:])
    return act, act.astype(np.float64) @ Wdn.T


def expert_ffn_fp8(X, gate_up: dict, down: dict):
    """One FP8 expert (codes, scales) on fp16 rows X."""
    return _expert_ffn(X, dequantize_fp8(gate_up["codes"], gate_up["scales"]),
                       dequantize_fp8(down["codes"], down["scales"]))


def expert_ffn_nvfp4(X, gate_up: dict, down: dict):
    """One NVFP4 expert (qweight, block_scales, global_scale) on fp16 rows X."""
    return _expert_ffn(X, dequantize_nvfp4(gate_up["qweight"], gate_up["block_scales"],
                                           gate_up["global_scale"], gate_up["K"]),
                       dequantize_nvfp4(down["qweight"], down["block_scales"], down["global_scale"],
                                        down["K"]))


def _expert_slice(W: dict, e: int) -> dict:
    """Expert e of a stacked weight dict (every array indexed on its first axis)."""
    return {k: (v[e] if isinstance(v, np.ndarray) and v.ndim > 0 else v) for k, v in W.items()}


def _moe_layer_codec(H, weights: dict, logit_bias, topk: int, with_shared: bool, ffn) -> dict:
    H = np.asarray(H)
    T = H.shape[0]
    E = weights["Wr"].shape[1]
    logits = router_logits(H, weights["Wr"], logit_bias)
    ids, gates = topk_route(logits, topk)
    counts = histogram(ids, E)
    offsets = exclusive_scan(counts)
    sorted_assign, pos = stable_permutation(ids, E)

    gu, dn = weights["gate_up"], weights["down"]
    I = gu["N"] // 2
    D = dn["N"]
    R = T * topk + (T if with_shared else 0)
    act = np.zeros((R, I), dtype=np.float16)
    ydown = np.zeros((R, D), dtype=np.float64)
    for e in range(E):
        r0, r1 = int(offsets[e]), int(offsets[e + 1])
        if r1 == r0:
            continue
        tokens = sorted_assign[r0:r1] // topk
        a, y = ffn(H[tokens], _expert_slice(gu, e), _expert_slice(dn, e))
        act[r0:r1] = a
        ydown[r0:r1] = y
    if with_shared:
        a, y = ffn(H, weights["shared_gate_up"], weights["shared_down"])
        act[T * topk:] = a
        ydown[T * topk:] = y
    out = combine(ydown, gates, pos, T, topk, with_shared)
    return {"logits": logits, "ids": ids, "gates": gates, "counts": counts,
            "offsets": offsets, "sorted_assign": sorted_assign, "pos": pos,
            "act": act, "ydown": ydown, "out": out}


def moe_layer_fp8(H, weights: dict, logit_bias=None, topk: int = 8,
                  with_shared: bool = True) -> dict:
    """The routed-expert layer on fp16 tokens H [T][D] with FP8 experts.

    ``weights`` holds Wr [D][E] fp16 and gate_up / down / shared_gate_up /
    shared_down as FP8 dicts (codes, scales; experts stacked on the first
    axis).  Returns the same intermediates as oracle.moe.moe_layer.
    """
    return _moe_layer_codec(H, weights, logit_bias, topk, with_shared,
                            lambda X, g, d: expert_ffn_fp8(X, g, d))


def moe_layer_nvfp4(H, weights: dict, logit_bias=None, topk: int = 8,
                    with_shared: bool = True) -> dict:
    """The routed-expert layer on fp16 tokens H [T][D] with NVFP4 experts
    (qweight, block_scales stacked on the first axis, global_scale one fp32
    per expert; the shared expert one NVFP4 matrix)."""
    return _moe_layer_codec(H, weights, logit_bias, topk, with_shared,
                            lambda X, g, d: expert_ffn_nvfp4(X, g, d))
