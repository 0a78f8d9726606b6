"""Seeded synthetic inputs shared by the oracle-side tests, the GPU parity
tests, the benchmark and the smoke check.

This module only draws random numbers in fixed shapes and distributions.  It
holds none of the method's arithmetic: no unpacking, no dequantization, no
matmul, no routing.  Every array is produced on the host with
``numpy.random.default_rng(seed)`` in a fixed draw order, so the GPU path and
the oracle read the very same bytes.

Distributions (the workload the pages benchmark is a Qwen-style MoE with
group-affine 4-bit weights; no checkpoint or prompt text is available, so
these seeded draws stand in for it):

* activations: fp16 of N(0, 1);
* 4-bit codes: i.i.d. uniform in 0..15.  Eight independent uniform nibbles
  are exactly one uniform 32-bit word, so the packed words are drawn directly
  as uniform uint32 (this is a statement about the distribution, not a pack
  step: which nibble holds which k is fixed by the layout, not here);
* per-group scale: fp16 of U(0.002, 0.02);
* per-group bias: fp16 of (-8 * scale_fp16 + N(0, 1e-3)), so that code 8
  reconstructs to roughly zero;
* router weight [D][E]: fp16 of N(0, 0.02) (0.02 read as a standard
  deviation);
* skewed-load logit bias: b_e = -1.1 * ln(rank_e), ranks a seeded
  permutation of 1..E (the logarithm of a Zipf law with s = 1.1);
* decode row in front of a normalization (residual stream): fp16 of
  N(0, 16), i.e. 4 * N(0, 1); normalization gain: fp16 of U(0.5, 1.5);
* bf16 variants: the same draws stored as bf16 bit patterns (uint16, the
  upper half of the float32 pattern, nearest even);
* FP8-E4M3 weights: codes uniform over the 254 bytes that encode numbers
  (a checkpoint's weights are finite), or over all 256 bytes, the two NaN
  codes included, with ``all_codes=True``; one fp16 scale per 64 along K
  from U(1e-4, 1e-3), or any range the caller gives;
* NVFP4 weights: E2M1 codes uniform (uniform 32-bit words, as the w4 codes),
  E4M3 block scales with exponent field uniform in 5..9 and mantissa
  uniform (values 0.25 .. 7.5), positive, or uniform over all 256 bytes
  (signs, subnormals, 448 and NaN) with ``all_codes=True``; global scale
  0.01 (fp32), or the caller's;
* exact-arithmetic router inputs: H in {-1, 0, 1}, router weights integers
  in -16..16 times 2**-8, logit bias the Zipf bias rounded to a multiple of
  2**-8, so that every logit is a multiple of 2**-8 of magnitude below 2**8
  and fp32 sums in any order are exact (exact ties are frequent).
"""
from __future__ import annotations

import numpy as np

GROUP = 64

# Shapes of the Qwen-style MoE layer the pages benchmark (hidden 2048,
# 256 routed experts of width 512, top-8, plus one shared expert).
HIDDEN = 2048
EXPERT_WIDTH = 512
NUM_EXPERTS = 256
TOPK = 8
VOCAB = 151552


def rng_for(seed: int) -> np.random.Generator:
    return np.random.default_rng(seed)


def f16(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64).astype(np.float16)


def activations(rng: np.random.Generator, rows: int, cols: int) -> np.ndarray:
    """fp16 [rows][cols] drawn from N(0, 1)."""
    return f16(rng.standard_normal((rows, cols)))


def w4_matrix(rng: np.random.Generator, K: int, N: int, lead: tuple = (),
              scale_range=(0.002, 0.02)) -> dict:
    """One (or a stack of) group-affine 4-bit K x N matrices.

    Returns a dict with ``qweight`` uint32 [*lead, N, K/8], ``scales`` and
    ``biases`` fp16 [*lead, N, K/64], and the sizes.  ``lead=(E,)`` draws E
    experts stacked contiguously.  Scales are U(scale_range) (the workload's
    U(0.002, 0.02) by default); the bias noise grows with the scale.
    """
    if K % 8:
        raise ValueError("K must be a multiple of 8 to draw packed words")
    G = (K + GROUP - 1) // GROUP
    words = rng.integers(0, 2**32, size=lead + (N, K // 8), dtype=np.uint64).astype(np.uint32)
    scales = f16(rng.uniform(scale_range[0], scale_range[1], size=lead + (N, G)))
    noise = rng.normal(0.0, 1e-3 * scale_range[1] / 0.02, size=lead + (N, G))
    biases = f16(-8.0 * scales.astype(np.float64) + noise)
    return {"qweight": words, "scales": scales, "biases": biases, "K": K, "N": N}


def bf16_bits(a) -> np.ndarray:
    """Draws stored as bf16 patterns: float32, then the upper 16 bits with
    round to nearest even (finite draws only)."""
    u = np.asarray(a, dtype=np.float64).astype(np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def w4_matrix_bf16(rng: np.random.Generator, K: int, N: int, lead: tuple = ()) -> dict:
    """A K x N w4 matrix (or a stack of them, as w4_matrix) with bf16 scales
    and biases (uint16 patterns), drawn like w4_matrix."""
    if K % 8:
        raise ValueError("K must be a multiple of 8 to draw packed words")
    G = (K + GROUP - 1) // GROUP
    words = rng.integers(0, 2**32, size=lead + (N, K // 8), dtype=np.uint64).astype(np.uint32)
    s = rng.uniform(0.002, 0.02, size=lead + (N, G))
    scales = bf16_bits(s)
    s_dec = (scales.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    biases = bf16_bits(-8.0 * s_dec + rng.normal(0.0, 1e-3, size=lead + (N, G)))
    return {"qweight": words, "scales": scales, "biases": biases, "K": K, "N": N}


def gemm_case_bf16(seed: int, M: int, K: int, N: int) -> dict:
    """X bf16 [M][K] (N(0, 1) draws) and one bf16-scaled K x N w4 matrix."""
    rng = rng_for(seed)
    X = bf16_bits(rng.standard_normal((M, K)))
    W = w4_matrix_bf16(rng, K, N)
    return {"X": X, "W": W}


def fp8_matrix(rng: np.random.Generator, K: int, N: int, lead: tuple = (),
               all_codes: bool = False, scale_range=(1e-4, 1e-3)) -> dict:
    """FP8-E4M3 weights: codes uint8 [N][K], fp16 scales [N][K/64] from
    U(scale_range); ``lead`` stacks several such matrices (e.g. (E,) for E
    experts).  Codes are uniform over the 254 number codes (0x7F and 0xFF,
    the NaN codes, are skipped), or over all 256 with ``all_codes``."""
    if all_codes:
        codes = rng.integers(0, 256, size=lead + (N, K), dtype=np.uint16).astype(np.uint8)
    else:
        codes = rng.integers(0, 254, size=lead + (N, K), dtype=np.uint8)
        codes += codes >= 0x7F                                          # skip 0x7F (and 0xFF)
    scales = f16(rng.uniform(scale_range[0], scale_range[1], size=lead + (N, K // 64)))
    return {"codes": codes, "scales": scales, "K": K, "N": N}


def nvfp4_matrix(rng: np.random.Generator, K: int, N: int, lead: tuple = (),
                 all_codes: bool = False, global_scale: float = 0.01) -> dict:
    """NVFP4 weights: qweight uint32 [N][K/8] (E2M1 codes, w4 packing),
    block scales uint8 [N][K/16] (positive E4M3 of 0.25 .. 7.5, or every
    byte with ``all_codes``), global scale fp32 (``global_scale``).
    ``lead`` stacks several matrices; each then draws its own global scale
    (fp32 array of shape ``lead``, uniform in [0.005, 0.02))."""
    words = rng.integers(0, 2**32, size=lead + (N, K // 8), dtype=np.uint64).astype(np.uint32)
    if all_codes:
        block = rng.integers(0, 256, size=lead + (N, K // 16), dtype=np.uint16).astype(np.uint8)
    else:
        e = rng.integers(5, 10, size=lead + (N, K // 16))
        m = rng.integers(0, 8, size=lead + (N, K // 16))
        block = ((e << 3) | m).astype(np.uint8)
    g = np.float32(global_scale) if not lead else rng.uniform(0.005, 0.02, size=lead).astype(np.float32)
    return {"qweight": words, "block_scales": block, "global_scale": g, "K": K, "N": N}


def router_weight(rng: np.random.Generator, D: int = HIDDEN, E: int = NUM_EXPERTS) -> np.ndarray:
    """fp16 [D][E] drawn from N(0, 0.02)."""
    return f16(rng.normal(0.0, 0.02, size=(D, E)))


def zipf_logit_bias(rng: np.random.Generator, E: int = NUM_EXPERTS, s: float = 1.1) -> np.ndarray:
    """fp32 [E]: -s * ln(rank_e) with ranks a seeded permutation of 1..E."""
    ranks = rng.permutation(E) + 1
    return (-s * np.log(ranks.astype(np.float64))).astype(np.float32)


def synthetic_topk_ids(rng: np.random.Generator, T: int, E: int, topk: int,
                       skew: float = 0.0) -> np.ndarray:
    """int32 [T][topk]: distinct expert ids per token, drawn without
    replacement.  ``skew > 0`` weights expert e by (rank_e)^-skew so some
    experts get many rows and some none.  Used to drive the dispatch steps
    with routing that does not come from any router."""
    if topk > E:
        raise ValueError("topk > E")
    if skew > 0:
        ranks = rng.permutation(E) + 1
        w = ranks.astype(np.float64) ** (-skew)
        p = w / w.sum()
    else:
        p = None
    out = np.empty((T, topk), dtype=np.int32)
    for t in range(T):
        out[t] = rng.choice(E, size=topk, replace=False, p=p)
    return out


# ----------------------------------------------------------------------------
# Workloads.  Each builder fixes the order of its draws.
# ----------------------------------------------------------------------------

def gemv_case(seed: int, K: int, N: int, x_scale: float = 1.0) -> dict:
    """x fp16 [1][K] (N(0, x_scale**2) draws) and one K x N w4 matrix."""
    rng = rng_for(seed)
    x = activations(rng, 1, K) if x_scale == 1.0 else f16(x_scale * rng.standard_normal((1, K)))
    W = w4_matrix(rng, K, N)
    return {"x": x, "W": W}


def norm_gain(rng: np.random.Generator, K: int) -> np.ndarray:
    """fp16 [K] drawn from U(0.5, 1.5)."""
    return f16(rng.uniform(0.5, 1.5, size=K))


def decode_norm_case(seed: int, K: int, N: int) -> dict:
    """Residual-stream row x fp16 [1][K] (4 * N(0, 1)), its normalization
    gain fp16 [K] and one K x N w4 matrix."""
    rng = rng_for(seed)
    x = f16(4.0 * rng.standard_normal((1, K)))
    gamma = norm_gain(rng, K)
    W = w4_matrix(rng, K, N)
    return {"x": x, "gamma": gamma, "W": W}


def gemm_case(seed: int, M: int, K: int, N: int) -> dict:
    """X fp16 [M][K] and one K x N w4 matrix."""
    rng = rng_for(seed)
    X = activations(rng, M, K)
    W = w4_matrix(rng, K, N)
    return {"X": X, "W": W}


def moe_weights(seed: int, D: int = HIDDEN, I: int = EXPERT_WIDTH, E: int = NUM_EXPERTS,
                scale_range=(0.002, 0.02), router_std: float = 0.02) -> dict:
    """Router [D][E] fp16, E stacked experts and one shared expert.

    gate_up: K = D, N = 2*I (columns [0, I) gate, [I, 2I) up);
    down:    K = I, N = D.
    """
    rng = rng_for(seed)
    Wr = f16(rng.normal(0.0, router_std, size=(D, E)))
    gate_up = w4_matrix(rng, D, 2 * I, lead=(E,), scale_range=scale_range)
    down = w4_matrix(rng, I, D, lead=(E,), scale_range=scale_range)
    shared_gate_up = w4_matrix(rng, D, 2 * I, scale_range=scale_range)
    shared_down = w4_matrix(rng, I, D, scale_range=scale_range)
    return {"Wr": Wr, "gate_up": gate_up, "down": down,
            "shared_gate_up": shared_gate_up, "shared_down": shared_down,
            "D": D, "I": I, "E": E}


def moe_weights_fp8(seed: int, D: int = HIDDEN, I: int = EXPERT_WIDTH, E: int = NUM_EXPERTS) -> dict:
    """moe_weights with FP8-E4M3 experts (fp8_matrix draws).  The fp16 router
    weight is drawn first from the same seed, so it equals moe_weights(seed)'s
    and a token seed routes exactly as it does there."""
    rng = rng_for(seed)
    Wr = router_weight(rng, D, E)
    gate_up = fp8_matrix(rng, D, 2 * I, lead=(E,))
    down = fp8_matrix(rng, I, D, lead=(E,))
    shared_gate_up = fp8_matrix(rng, D, 2 * I)
    shared_down = fp8_matrix(rng, I, D)
    return {"Wr": Wr, "gate_up": gate_up, "down": down,
            "shared_gate_up": shared_gate_up, "shared_down": shared_down,
            "D": D, "I": I, "E": E}


def moe_weights_nvfp4(seed: int, D: int = HIDDEN, I: int = EXPERT_WIDTH, E: int = NUM_EXPERTS) -> dict:
    """moe_weights with NVFP4 experts (nvfp4_matrix draws, one global scale
    per expert).  The fp16 router weight is drawn first, as in moe_weights."""
    rng = rng_for(seed)
    Wr = router_weight(rng, D, E)
    gate_up = nvfp4_matrix(rng, D, 2 * I, lead=(E,))
    down = nvfp4_matrix(rng, I, D, lead=(E,))
    shared_gate_up = nvfp4_matrix(rng, D, 2 * I)
    shared_down = nvfp4_matrix(rng, I, D)
    return {"Wr": Wr, "gate_up": gate_up, "down": down,
            "shared_gate_up": shared_gate_up, "shared_down": shared_down,
            "D": D, "I": I, "E": E}


def moe_tokens(seed: int, T: int, D: int = HIDDEN, E: int = NUM_EXPERTS,
               skewed: bool = False, h_scale: float = 1.0) -> dict:
    """H fp16 [T][D] ~ N(0, h_scale**2) and, if ``skewed``, the Zipf logit
    bias."""
    rng = rng_for(seed)
    H = activations(rng, T, D) if h_scale == 1.0 else f16(h_scale * rng.standard_normal((T, D)))
    bias = zipf_logit_bias(rng, E) if skewed else None
    return {"H": H, "logit_bias": bias}


def router_tie_case(seed: int, T: int, topk: int, D: int = HIDDEN, E: int = NUM_EXPERTS) -> dict:
    """Router inputs whose logits are exact in fp32 under any summation order
    and hold exact ties at the top and across the top-k boundary.

    H entries are -1, 0 or 1, with the first 512 (or D/4) all 1; router
    weights are integers in -16..16 times 2**-8 (small integers in the
    all-ones rows), so every partial sum is a multiple of 2**-8 below 2**7.
    One column with weight 1/16 on the all-ones rows is copied to
    ``n_top = max(1, topk // 2)`` positions and one with weight 1/32 to
    ``n_edge`` further positions (up to two more than the top-k has room
    for), all at seeded random indices: the copies have identical logits,
    far above the rest, and the top-k cut falls inside the second group.
    """
    rng = rng_for(seed)
    ones = min(512, D // 4)
    H = rng.integers(-1, 2, size=(T, D)).astype(np.float64)
    H[:, :ones] = 1.0
    W = rng.integers(-16, 17, size=(D, E)).astype(np.float64)
    W[:ones, :] = rng.integers(-2, 3, size=(ones, E))
    cols = rng.permutation(E)
    n_top = max(1, topk // 2)
    n_edge = min(topk - n_top + 2, E - n_top)
    top, edge = cols[:n_top], cols[n_top:n_top + n_edge]
    W[:ones, top[0]] = 16.0
    W[:ones, edge[0]] = 8.0
    W[:, top] = W[:, [top[0]]]
    W[:, edge] = W[:, [edge[0]]]
    return {"H": f16(H), "Wr": f16(W / 256.0), "top": np.sort(top), "edge": np.sort(edge)}


def router_exact_case(seed: int, T: int, D: int = HIDDEN, E: int = NUM_EXPERTS,
                      skewed: bool = True) -> dict:
    """Router inputs whose fp32 logits are exact in any summation order, at
    any T (varied routing, unlike router_tie_case): H fp16 [T][D] in
    {-1, 0, 1}, router weight fp16 [D][E] of integers in -16..16 times
    2**-8, and (if ``skewed``) the Zipf logit bias rounded to a multiple of
    2**-8 (fp32).  Every logit is a multiple of 2**-8 below 2**8 in
    magnitude, so exact ties between experts are common."""
    rng = rng_for(seed)
    H = rng.integers(-1, 2, size=(T, D)).astype(np.float64)
    W = rng.integers(-16, 17, size=(D, E)).astype(np.float64) / 256.0
    bias = None
    if skewed:
        b = zipf_logit_bias(rng, E).astype(np.float64)
        bias = (np.round(b * 256.0) / 256.0).astype(np.float32)
    return {"H": f16(H), "Wr": f16(W), "logit_bias": bias}


def moe_weights_bf16(seed: int, D: int = HIDDEN, I: int = EXPERT_WIDTH, E: int = NUM_EXPERTS) -> dict:
    """moe_weights with every 16-bit array as bf16 patterns: the router
    weight (N(0, 0.02) draws) and the experts' scales and biases."""
    rng = rng_for(seed)
    Wr = bf16_bits(rng.normal(0.0, 0.02, size=(D, E)))
    gate_up = w4_matrix_bf16(rng, D, 2 * I, lead=(E,))
    down = w4_matrix_bf16(rng, I, D, lead=(E,))
    shared_gate_up = w4_matrix_bf16(rng, D, 2 * I)
    shared_down = w4_matrix_bf16(rng, I, D)
    return {"Wr": Wr, "gate_up": gate_up, "down": down,
            "shared_gate_up": shared_gate_up, "shared_down": shared_down,
            "D": D, "I": I, "E": E}


def moe_tokens_bf16(seed: int, T: int, D: int = HIDDEN, E: int = NUM_EXPERTS,
                    skewed: bool = False) -> dict:
    """H bf16 patterns [T][D] of N(0, 1) draws and, if ``skewed``, the Zipf
    logit bias (fp32)."""
    rng = rng_for(seed)
    H = bf16_bits(rng.standard_normal((T, D)))
    bias = zipf_logit_bias(rng, E) if skewed else None
    return {"H": H, "logit_bias": bias}


# Default configurations of the benchmarked workload.
CONFIGS = {
    0: dict(kind="gemv", K=512, N=512),
    1: dict(kind="gemv", K=2048, N=(8192, VOCAB)),
    2: dict(kind="gemm", M=4096, K=2048, N=8192, sweep=(256, 1024, 16384)),
    3: dict(kind="moe", T=1, skewed=False),
    4: dict(kind="moe", T=4096, skewed=True),
}
