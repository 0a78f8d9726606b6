"""The decode steps on either side of the single-row w4 linear layer: the
normalization in front of a projection, the choice of the next token after
the vocabulary head, and the lookup of that token's input row.

Test infrastructure only (see the package docstring).

Pages followed:

* Perplexity, "Optimizing on-device inference for Apple Silicon", section
  "减少中间状态和流量" (reducing intermediates and traffic): the decode path
  fuses chains whose intermediates stay in registers; normalization feeding
  the projections is one of the steps fused.  lithos-metal's page (layer-wise
  fusion) likewise folds normalization for the next stage into the kernel
  that produces its input.
* Same Perplexity page, section "将 token 交接保留在 GPU 上" (keeping the
  token hand-off on the GPU): each decode step ends by picking the
  highest-scoring token, the GPU writes its id straight into the next
  step's input slot, and the next step starts from that token.

Readings taken where the pages are silent:

* the normalization is RMSNorm, u = x / sqrt(mean(x^2) + eps) * gamma (the
  pages name normalization but not its form; RMSNorm is the normalization of
  the Qwen models the pages run), with an fp16 gamma;
* the normalized activation is rounded to fp16 once, where an unfused path
  would store it between the two kernels, and the projection then reads
  that fp16 vector;
* "highest-scoring" is the largest logit; among equal largest logits the
  smallest token id is taken;
* the next step's input row of a token is that token's row of an embedding
  table stored in the same w4 format as the linear layers (row v = output v
  of a w4 matrix with K = hidden width), rounded to fp16 like every other
  activation.
"""
from __future__ import annotations

import numpy as np

from .w4 import dequantize, linear, round_f16


def rms_norm(x, gamma, eps: float) -> np.ndarray:
    """u[k] = x[k] / sqrt(mean_k(x^2) + eps) * gamma[k], in float64."""
    x = np.asarray(x, dtype=np.float64)
    g = np.asarray(gamma, dtype=np.float64)
    assert x.ndim == 1 and g.shape == x.shape
    ms = float(np.mean(x * x))
    return x / np.sqrt(ms + float(eps)) * g


def gemv_rmsnorm(x, gamma, eps: float, W: dict):
    """The projection of a normalized decode row: y = fp16(rms_norm(x)) . W.

    Returns (y float64 [N], u fp16 [K]) where u is the rounded normalized
    activation the projection reads."""
    u = round_f16(rms_norm(x, gamma, eps))
    return linear(u[None, :], W)[0], u


def argmax_first(v) -> int:
    """The smallest index among the positions holding the largest value."""
    v = np.asarray(v, dtype=np.float64)
    assert v.ndim == 1 and v.size > 0
    top = np.max(v)
    return int(np.flatnonzero(v == top)[0])


def lm_head_token(x, W: dict):
    """Vocabulary head and token choice for one decode row: the logits
    x . W (float64 [N]) and the id of the largest one."""
    logits = linear(np.asarray(x)[None, :], W)[0]
    return argmax_first(logits), logits


def embed_row(E: dict, token: int) -> np.ndarray:
    """Input row of `token`: fp16 of the dequantized row `token` of a w4
    embedding table E (E["N"] tokens, E["K"] = hidden width)."""
    if not 0 <= token < E["N"]:
        raise IndexError("token id outside the table")
    row = dequantize(E["qweight"][token:token + 1], E["scales"][token:token + 1],
                     E["biases"][token:token + 1], E["K"])[0]
    return round_f16(row)
