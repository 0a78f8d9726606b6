"""Group-affine 4-bit weights: unpack, pack, dequantize, linear.

Test infrastructure only (see the package docstring).

The format follows Perplexity, "Optimizing on-device inference for Apple
Silicon", section "在矩阵乘法期间进行权重反量化": every weight is a 4-bit
integer code, and each group of 64 consecutive weights shares one scale and
one bias that reconstruct the value.  Readings taken where the page is silent:

* the reconstruction is ``w = scale * code + bias`` (no separate zero point);
* scale and bias are fp16 (the page's checkpoint uses bf16; the workload this
  library serves fixes fp16);
* orientation: the logical matrix is W[k][n] (K inputs, N outputs), stored
  per output n with K contiguous: ``qweight[n][k // 8]`` holds code k in bits
  [4*(k % 8), 4*(k % 8) + 4), least significant nibble first;
* groups are 64 consecutive k of one output n, aligned at multiples of 64
  (laya-mlx, "选择性量化", skips layers whose input width is not a multiple
  of the group size; here such K is rejected).
"""
from __future__ import annotations

import numpy as np

GROUP = 64


def round_f16(a) -> np.ndarray:
    """Round float64 values to the nearest fp16 (ties to even; beyond the
    largest finite fp16 the result is infinite)."""
    with np.errstate(over="ignore"):
        return np.asarray(a, dtype=np.float64).astype(np.float16)


def unpack_codes(qweight: np.ndarray, K: int) -> np.ndarray:
    """uint32 [..., N, K/8] -> int64 codes [..., N, K]: code k of output n is
    the nibble at bits 4*(k % 8) of word k // 8."""
    qweight = np.asarray(qweight, dtype=np.uint32)
    assert qweight.shape[-1] * 8 == K, "qweight last dim must be K/8"
    words = qweight.astype(np.int64)
    codes = np.empty(qweight.shape[:-1] + (K,), dtype=np.int64)
    for j in range(8):
        codes[..., j::8] = (words >> (4 * j)) & 0xF
    return codes


def pack_codes(codes: np.ndarray) -> np.ndarray:
    """int codes [..., N, K] in 0..15 -> uint32 [..., N, K/8] (inverse of
    unpack_codes)."""
    codes = np.asarray(codes, dtype=np.int64)
    K = codes.shape[-1]
    if K % 8:
        raise ValueError("K must be a multiple of 8")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("codes must lie in 0..15")
    words = np.zeros(codes.shape[:-1] + (K // 8,), dtype=np.int64)
    for j in range(8):
        words |= codes[..., j::8] << (4 * j)
    return words.astype(np.uint32)


def dequantize(qweight, scales, biases, K: int) -> np.ndarray:
    """float64 [..., N, K] with W[n][k] = scale[n][k//64]*code + bias[n][k//64].

    In float64 this is exact: an fp16 scale times an integer below 16 needs
    at most 15 significant bits, and adding an fp16 bias stays far inside 53.
    """
    if K % GROUP:
        raise ValueError("K must be a multiple of the group size 64")
    q = unpack_codes(qweight, K).astype(np.float64)
    s = np.repeat(np.asarray(scales, dtype=np.float16).astype(np.float64), GROUP, axis=-1)
    b = np.repeat(np.asarray(biases, dtype=np.float16).astype(np.float64), GROUP, axis=-1)
    assert s.shape == q.shape and b.shape == q.shape
    return s * q + b


def linear(X, W: dict, row_chunk: int = 8192) -> np.ndarray:
    """Y[m][n] = sum_k X[m][k] * W[k][n] in float64, for fp16 X [M][K] and a
    w4 matrix dict (qweight, scales, biases, K, N).

    This is the linear layer of the decode GEMV (M = 1) and of the prefill
    GEMM alike; the pages accumulate in fp32 and write 16-bit outputs, the
    oracle keeps float64 and leaves rounding to the caller.  The output
    columns are processed in chunks of ``row_chunk`` so that a vocabulary-
    sized W never exists in float64 all at once.
    """
    X = np.asarray(X)
    if X.ndim == 1:
        X = X[None, :]
    K, N = W["K"], W["N"]
    assert X.shape[1] == K
    Xd = X.astype(np.float64)
    Y = np.empty((X.shape[0], N), dtype=np.float64)
    for n0 in range(0, N, row_chunk):
        n1 = min(N, n0 + row_chunk)
        Wd = dequantize(W["qweight"][n0:n1], W["scales"][n0:n1], W["biases"][n0:n1], K)
        Y[:, n0:n1] = Xd @ Wd.T
    return Y
