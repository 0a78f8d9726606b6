// E4M3 weight codes as exact fp16 values, shared by the FP8 GEMV and the
// FP8 GEMM.
//
// "待验证｜lithos-metal补Apple推理内核", section "一分钟内合并了什么": FP8
// E4M3 weights decoded two codes per half2.
#pragma once

#include "ql_device.h"

namespace ql {

// Two E4M3 codes -> fp16 pair holding e4m3 * 2**-8 each, exactly: the code
// bits seeeemmm go to fp16 bits s.0eeee.mmm0000000 (the exponent bias 15 of
// fp16 against 7 of E4M3 is the 2**-8; E4M3 subnormals land on fp16
// subnormals).  `t` holds the two codes in bits 15:8 and 31:24.
__device__ __forceinline__ uint32_t e4m3x2_to_f16x2(uint32_t t) {
    return (t & 0x80008000u) | ((t >> 1) & 0x3F803F80u);
}

// The four codes of a word (bytes b0..b3) as two fp16 pairs (b0, b1) and
// (b2, b3), each value e4m3 * 2**-8.
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, uint32_t& p01, uint32_t& p23) {
    p01 = e4m3x2_to_f16x2(__builtin_amdgcn_perm(w, w, 0x010C000Cu));
    p23 = e4m3x2_to_f16x2(__builtin_amdgcn_perm(w, w, 0x030C020Cu));
}

// E4M3 code -> float, exactly (via the fp16 pattern above).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t h = ((b & 0x80u) << 8) | ((b & 0x7Fu) << 7);
    return h2f((uint16_t)h) * 256.0f;
}

}  // namespace ql
