"""CPU oracle for group-affine 4-bit linear layers and routed-expert MoE.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports, calls or
links anything in this package: only the test suite, the smoke check and the
benchmark's CPU-baseline leg do.  It shares no code with the HIP kernels or
their host library.

Everything here is plain numpy in float64, written for a reader to check by
eye against the pages it cites:

* Perplexity, "Optimizing on-device inference for Apple Silicon" (the Lily
  engine for Qwen3.6-35B-A3B), in particular the sections
  "在矩阵乘法期间进行权重反量化" (dequantizing weights inside the matrix
  multiply), "将专家路由保留在 GPU 上" (keeping expert routing on the GPU),
  "使瓦片大小与专家负载相匹配" (matching tile size to expert load),
  "Qwen 创建了三种不同的工作负载形状" (the three workload shapes),
  "优化单行权重路径" (the single-row weight path) and
  "减少中间状态和流量" (reducing intermediates and traffic) and
  "将 token 交接保留在 GPU 上" (keeping the token hand-off on the GPU);
* laya-mlx, "工程调查：这个 MLX 端口还能再快 10× 吗？", section
  "选择性量化" (affine quantization with group size 64);
* "待验证｜lithos-metal补Apple推理内核", section "一分钟内合并了什么" (FP8
  E4M3 decode and an NVFP4 checkpoint: the second codecs).

Where the pages leave a step open, the plainest reading is taken; each such
reading is named in the function that applies it.

Parity status of each function (what pins it, see tests/test_oracle_*.py):
all functions are pinned by hand-worked cases, closed forms, invariants or
brute force; the end-to-end fidelity on real checkpoint weights is
"parity unpinned" (no checkpoint and no page prints values for this path).
"""
from .w4 import (GROUP, unpack_codes, pack_codes, dequantize, linear,
                 round_f16)
from .route import (router_logits, softmax, topk_route, histogram,
                    exclusive_scan, stable_permutation, tile_map, load_matched_tile_map,
                    topk_near_ties)
from .moe import silu, expert_ffn, combine, moe_layer
from .decode import rms_norm, gemv_rmsnorm, argmax_first, lm_head_token, embed_row
from .bf16 import (bf16_to_f64, round_bf16, dequantize_bf16, linear_bf16, expert_ffn_bf16,
                   moe_layer_bf16)
from .codecs import (e4m3_to_f64, e2m1_to_f64, dequantize_fp8, dequantize_nvfp4, linear_fp8,
                     linear_nvfp4, expert_ffn_fp8, moe_layer_fp8, expert_ffn_nvfp4,
                     moe_layer_nvfp4)

__all__ = [
    "GROUP", "unpack_codes", "pack_codes", "dequantize", "linear", "round_f16",
    "router_logits", "softmax", "topk_route", "histogram", "exclusive_scan",
    "stable_permutation", "tile_map", "load_matched_tile_map", "topk_near_ties",
    "silu", "expert_ffn", "combine", "moe_layer",
    "rms_norm", "gemv_rmsnorm", "argmax_first", "lm_head_token", "embed_row",
    "bf16_to_f64", "round_bf16", "dequantize_bf16", "linear_bf16", "expert_ffn_bf16",
    "moe_layer_bf16",
    "e4m3_to_f64", "e2m1_to_f64", "dequantize_fp8", "dequantize_nvfp4", "linear_fp8", "linear_nvfp4",
    "expert_ffn_fp8", "moe_layer_fp8", "expert_ffn_nvfp4", "moe_layer_nvfp4",
]
