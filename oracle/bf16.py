"""bf16 variant of the group-affine 4-bit linear layer: bf16 scale, bias,
activations and outputs.

Test infrastructure only (see the package docstring).

Perplexity, "Optimizing on-device inference for Apple Silicon", section
"在矩阵乘法期间进行权重反量化": the page's checkpoint keeps the per-group
scale and bias in bfloat16 and the matrix path multiplies bf16 operands.
The reconstruction is the same as in w4.py, w = scale * code + bias per
group of 64 along K; only the 16-bit type changes.

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
