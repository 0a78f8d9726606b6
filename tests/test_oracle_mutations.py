"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin fails for each: the pins are only worth something if they
catch a dropped term, a wrong sign, a wrong index or a transposed operand."""
import numpy as np
import pytest

import oracle
import oracle.moe as omoe
import oracle.route as oroute
import oracle.w4 as ow4
from tests import test_oracle_moe as tm
from tests import test_oracle_route as tr
from tests import test_oracle_w4 as tw

W4_PINS = [tw.test_gemv_hand_fixture, tw.test_one_hot_picks_single_weight,
           tw.test_affine_identity_all_equal_codes, tw.test_zero_case_code8,
           tw.test_integer_special_case_exact, tw.test_bruteforce_fsum_small,
           tw.test_pack_words_hand, tw.test_dequantize_exact_rational]


def _fails(pins):
    for pin in pins:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            return True
    return False


_orig_unpack = ow4.unpack_codes


def _unpack_reversed(qweight, K):
    c = _orig_unpack(qweight, K)
    out = c.copy()
    for j in range(8):
        out[..., j::8] = c[..., (7 - j)::8]
    return out


def _dequant_no_bias(qweight, scales, biases, K):
    q = ow4.unpack_codes(qweight, K).astype(np.float64)
    s = np.repeat(np.asarray(scales, np.float16).astype(np.float64), 64, axis=-1)
    return s * q


def _dequant_bias_sign(qweight, scales, biases, K):
    q = ow4.unpack_codes(qweight, K).astype(np.float64)
    s = np.repeat(np.asarray(scales, np.float16).astype(np.float64), 64, axis=-1)
    b = np.repeat(np.asarray(biases, np.float16).astype(np.float64), 64, axis=-1)
    return s * q - b


def _dequant_wrong_group(qweight, scales, biases, K):
    q = ow4.unpack_codes(qweight, K).astype(np.float64)
    s = np.tile(np.asarray(scales, np.float16).astype(np.float64), 64)
    b = np.tile(np.asarray(biases, np.float16).astype(np.float64), 64)
    return s * q + b


def _linear_transposed(X, W, row_chunk=8192):
    X = np.atleast_2d(np.asarray(X)).astype(np.float64)
    Wd = ow4.dequantize(W["qweight"], W["scales"], W["biases"], W["K"])
    return X @ Wd.T[::-1, ::-1] if Wd.shape[0] == Wd.shape[1] else X @ Wd.T[:, ::-1]


@pytest.mark.parametrize("target,attr,mutant", [
    (ow4, "unpack_codes", _unpack_reversed),
    (ow4, "dequantize", _dequant_no_bias),
    (ow4, "dequantize", _dequant_bias_sign),
    (ow4, "dequantize", _dequant_wrong_group),
])
def test_w4_mutants_are_caught(monkeypatch, target, attr, mutant):
    monkeypatch.setattr(target, attr, mutant)
    assert _fails(W4_PINS)


def test_transposed_linear_is_caught(monkeypatch):
    monkeypatch.setattr(oracle, "linear", _linear_transposed)
    assert _fails(W4_PINS)


def _topk_ties_high(logits, topk):
    L = np.asarray(logits, np.float64)
    p = oroute.softmax(L)
    ids = np.empty((L.shape[0], topk), np.int32)
    gates = np.empty((L.shape[0], topk))
    for t in range(L.shape[0]):
        order = np.lexsort((-np.arange(L.shape[1]), -p[t]))[:topk]
        ids[t], gates[t] = order, p[t, order] / p[t, order].sum()
    return ids, gates


def _topk_unnormalised(logits, topk):
    ids, _ = _ORIG_TOPK(logits, topk)
    p = oroute.softmax(logits)
    return ids, np.take_along_axis(p, ids.astype(np.int64), axis=1)


_ORIG_TOPK = oroute.topk_route


def _perm_unstable(ids, E):
    flat = np.asarray(ids).ravel()
    sa = np.argsort(flat * 100000 - np.arange(flat.size))  # descending a inside groups
    pos = np.empty_like(sa)
    pos[sa] = np.arange(sa.size)
    return sa.astype(np.int32), pos.astype(np.int32)


def _scan_inclusive(counts):
    c = np.asarray(counts, np.int64)
    return np.concatenate([np.cumsum(c), [c.sum()]]).astype(np.int32)


ROUTE_PINS = [tr.test_route_hand_fixture, tr.test_equal_logits_pick_lowest_indices,
              tr.test_bruteforce_subsets_tiny_E, tr.test_dispatch_hand_fixture,
              tr.test_dispatch_invariants_and_library_sort]


@pytest.mark.parametrize("target,attr,mutant", [
    (oroute, "topk_route", _topk_ties_high),
    (oroute, "topk_route", _topk_unnormalised),
    (oroute, "stable_permutation", _perm_unstable),
    (oroute, "exclusive_scan", _scan_inclusive),
])
def test_route_mutants_are_caught(monkeypatch, target, attr, mutant):
    monkeypatch.setattr(target, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant)
    assert _fails(ROUTE_PINS)


_ORIG_COMBINE = omoe.combine


def _combine_no_shared(ydown, gates, pos, T, topk, has_shared):
    return _ORIG_COMBINE(ydown, gates, pos, T, topk, False)


def _combine_wrong_row(ydown, gates, pos, T, topk, has_shared):
    ident = np.arange(len(pos))
    return _ORIG_COMBINE(ydown, gates, ident, T, topk, has_shared)


def _combine_gates_reversed(ydown, gates, pos, T, topk, has_shared):
    return _ORIG_COMBINE(ydown, np.asarray(gates)[:, ::-1], pos, T, topk, has_shared)


def _silu_sign(z):
    z = np.asarray(z, np.float64)
    return z / (1.0 + np.exp(z))


MOE_PINS = [tm.test_moe_layer_matches_per_token_bruteforce, tm.test_identical_experts_give_twice_the_ffn,
            tm.test_power_of_two_scaled_experts_pin_gate_to_id, tm.test_silu_library_and_limits]


@pytest.mark.parametrize("attr,mutant", [
    ("combine", _combine_no_shared),
    ("combine", _combine_wrong_row),
    ("combine", _combine_gates_reversed),
    ("silu", _silu_sign),
])
def test_moe_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(omoe, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant)
    assert _fails(MOE_PINS)


import oracle.decode as odec
from tests import test_oracle_decode as td

DECODE_PINS = [td.test_rms_norm_hand_fixture, td.test_rms_norm_invariants,
               td.test_gemv_rmsnorm_hand_fixture, td.test_gemv_rmsnorm_rounds_the_normalized_row_once,
               td.test_argmax_hand_and_bruteforce, td.test_lm_head_hand_fixture,
               td.test_lm_head_one_hot_selects_a_weight_column, td.test_embed_hand_fixture,
               td.test_embed_matches_digit_decode]


def _rms_no_sqrt(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / (np.mean(x * x) + eps) * np.asarray(gamma, np.float64)


def _rms_eps_outside(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x)) + eps) * np.asarray(gamma, np.float64)


def _rms_sum_not_mean(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x) + eps) * np.asarray(gamma, np.float64)


def _rms_no_gamma(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.mean(x * x) + eps)


def _argmax_last(v):
    v = np.asarray(v, np.float64)
    return int(np.flatnonzero(v == v.max())[-1])


_ORIG_EMBED = odec.embed_row


def _embed_next_row(E, token):
    return _ORIG_EMBED(E, (token + 1) % E["N"])


def _gemv_rmsnorm_unrounded(x, gamma, eps, W):
    u = odec.rms_norm(x, gamma, eps)
    return odec.linear(u[None, :], W)[0], odec.round_f16(u)


@pytest.mark.parametrize("attr,mutant", [
    ("rms_norm", _rms_no_sqrt),
    ("rms_norm", _rms_eps_outside),
    ("rms_norm", _rms_sum_not_mean),
    ("rms_norm", _rms_no_gamma),
    ("argmax_first", _argmax_last),
    ("embed_row", _embed_next_row),
    ("gemv_rmsnorm", _gemv_rmsnorm_unrounded),
])
def test_decode_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(odec, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant)
    assert _fails(DECODE_PINS)


import oracle.bf16 as obf
from tests import test_oracle_bf16 as tb

BF16_PINS = [tb.test_decode_hand_patterns, tb.test_round_trip_every_pattern, tb.test_round_hand_ties,
             tb.test_linear_hand_fixture, tb.test_one_hot_and_bruteforce]


def _bf16_dec_shift15(bits):
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return b.view(np.float32).astype(np.float64)


def _bf16_round_truncate(a):
    a = np.asarray(a, dtype=np.float64)
    return (a.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def _bf16_dequant_no_bias(qweight, scales_bits, biases_bits, K):
    q = ow4.unpack_codes(qweight, K).astype(np.float64)
    return q * np.repeat(obf.bf16_to_f64(scales_bits), 64, axis=-1)


@pytest.mark.parametrize("attr,mutant", [
    ("bf16_to_f64", _bf16_dec_shift15),
    ("round_bf16", _bf16_round_truncate),
    ("dequantize_bf16", _bf16_dequant_no_bias),
])
def test_bf16_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(obf, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant)
    assert _fails(BF16_PINS)


import oracle.codecs as ocod
from tests import test_oracle_codecs as tc

CODEC_PINS = [tc.test_e4m3_hand_table_and_nan, tc.test_e2m1_table, tc.test_fp8_linear_hand_fixture,
              tc.test_fp8_one_hot_and_bruteforce, tc.test_nvfp4_block_scales_and_global,
              tc.test_nvfp4_bruteforce]

_ORIG_E4M3 = ocod.e4m3_to_f64


def _e4m3_bias8(codes):
    return _ORIG_E4M3(codes) / 2.0          # exponent bias 8 instead of 7


def _e2m1_no_subnormal(n):
    n = np.asarray(n, dtype=np.int64)
    s = np.where(n & 0x8, -1.0, 1.0)
    e = (n >> 1) & 0x3
    m = (n & 0x1).astype(np.float64)
    return s * (1.0 + m / 2.0) * np.exp2(e.astype(np.float64) - 1.0)


def _nvfp4_block32(qweight, block_scales, global_scale, K):
    q = ocod.e2m1_to_f64(ocod.unpack_codes(qweight, K))
    bs = np.repeat(ocod.e4m3_to_f64(block_scales), 32, axis=-1)[..., :K]
    bs = np.pad(bs, [(0, 0)] * (bs.ndim - 1) + [(0, K - bs.shape[-1])], mode="edge")
    return q * bs * float(global_scale)


def _fp8_scale_index(codes, scales):
    codes = np.asarray(codes, dtype=np.uint8)
    s = np.tile(np.asarray(scales, dtype=np.float16).astype(np.float64), 64)
    return ocod.e4m3_to_f64(codes) * s


@pytest.mark.parametrize("attr,mutant", [
    ("e4m3_to_f64", _e4m3_bias8),
    ("e2m1_to_f64", _e2m1_no_subnormal),
    ("dequantize_nvfp4", _nvfp4_block32),
    ("dequantize_fp8", _fp8_scale_index),
])
def test_codec_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(ocod, attr, mutant)
    monkeypatch.setattr(oracle, attr, mutant)
    assert _fails(CODEC_PINS)


import oracle.bf16 as obf
from tests import test_oracle_bf16 as tb

BF16_MOE_PINS = [tb.test_moe_layer_bf16_matches_per_token_bruteforce,
                 tb.test_moe_layer_bf16_without_shared_and_identical_experts]
_ORIG_FFN_BF16 = obf.expert_ffn_bf16


def _ffn_bf16_up_gate_swapped(X_bits, gate_up, down):
    gu = dict(gate_up)
    half = gate_up["N"] // 2
    for f in ("qweight", "scales", "biases"):
        gu[f] = np.concatenate([gate_up[f][..., half:, :], gate_up[f][..., :half, :]], axis=-2)
    return _ORIG_FFN_BF16(X_bits, gu, down)


def _ffn_bf16_no_act_rounding(X_bits, gate_up, down):
    X = obf.bf16_to_f64(np.atleast_2d(np.asarray(X_bits, dtype=np.uint16)))
    I = gate_up["N"] // 2
    u = X @ obf.dequantize_bf16(gate_up["qweight"], gate_up["scales"], gate_up["biases"], gate_up["K"]).T
    a = obf.silu(u[:, :I]) * u[:, I:]
    ydown = a @ obf.dequantize_bf16(down["qweight"], down["scales"], down["biases"], down["K"]).T
    return obf.round_bf16(a), ydown


def _bf16_combine_no_shared(ydown, gates, pos, T, topk, has_shared):
    return _ORIG_COMBINE(ydown, gates, pos, T, topk, False)


@pytest.mark.parametrize("attr,mutant", [
    ("expert_ffn_bf16", _ffn_bf16_up_gate_swapped),
    ("expert_ffn_bf16", _ffn_bf16_no_act_rounding),
    ("combine", _bf16_combine_no_shared),
])
def test_bf16_moe_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(obf, attr, mutant)
    assert _fails(BF16_MOE_PINS)


from tests import test_oracle_codecs as tcod

FP8_MOE_PINS = [lambda: tcod.test_moe_fp8_equals_w4_layer_on_common_weights(True),
                tcod.test_moe_fp8_token_loop_bruteforce]
_ORIG_FFN_FP8 = ocod.expert_ffn_fp8


def _ffn_fp8_up_gate_swapped(X, gate_up, down):
    half = gate_up["N"] // 2
    gu = {"codes": np.concatenate([gate_up["codes"][half:], gate_up["codes"][:half]]),
          "scales": np.concatenate([gate_up["scales"][half:], gate_up["scales"][:half]]),
          "N": gate_up["N"]}
    return _ORIG_FFN_FP8(X, gu, down)


def _ffn_fp8_no_act_rounding(X, gate_up, down):
    X = np.asarray(X).astype(np.float64)
    I = gate_up["N"] // 2
    u = X @ ocod.dequantize_fp8(gate_up["codes"], gate_up["scales"]).T
    a = ocod.silu(u[:, :I]) * u[:, I:]
    ydown = a @ ocod.dequantize_fp8(down["codes"], down["scales"]).T
    return a.astype(np.float16), ydown


def _fp8_combine_no_shared(ydown, gates, pos, T, topk, has_shared):
    return _ORIG_COMBINE(ydown, gates, pos, T, topk, False)


@pytest.mark.parametrize("attr,mutant", [
    ("expert_ffn_fp8", _ffn_fp8_up_gate_swapped),
    ("expert_ffn_fp8", _ffn_fp8_no_act_rounding),
    ("combine", _fp8_combine_no_shared),
])
def test_fp8_moe_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(ocod, attr, mutant)
    assert _fails(FP8_MOE_PINS)


NVFP4_MOE_PINS = [lambda: tcod.test_moe_nvfp4_equals_fp8_layer_on_common_weights(True),
                  tcod.test_moe_nvfp4_per_expert_global_scale]
_ORIG_SLICE = ocod._expert_slice
_ORIG_FFN_NVFP4 = ocod.expert_ffn_nvfp4


def _slice_first_global(W, e):
    out = _ORIG_SLICE(W, e)
    if "global_scale" in W:
        out["global_scale"] = np.asarray(W["global_scale"]).ravel()[0]
    return out


def _ffn_nvfp4_globals_swapped(X, gate_up, down):
    g, d = dict(gate_up), dict(down)
    g["global_scale"], d["global_scale"] = down["global_scale"], gate_up["global_scale"]
    return _ORIG_FFN_NVFP4(X, g, d)


@pytest.mark.parametrize("attr,mutant", [
    ("_expert_slice", _slice_first_global),
    ("expert_ffn_nvfp4", _ffn_nvfp4_globals_swapped),
])
def test_nvfp4_moe_mutants_are_caught(monkeypatch, attr, mutant):
    monkeypatch.setattr(ocod, attr, mutant)
    assert _fails(NVFP4_MOE_PINS)
