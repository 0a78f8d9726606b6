// FP8-E4M3 and E2M1 weight codes as exact fp16 values, shared by the codec
// GEMVs and the codec GEMMs.
//
// "待验证｜lithos-metal补Apple推理内核", section "一分钟内合并了什么": FP8
// E4M3 weights decoded two codes per half2, and an NVFP4 checkpoint (E2M1
// codes with E4M3 block scales).
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

// A word of 8 E2M1 codes (code k at bits 4k) -> 4 fp16 pairs in natural k
// order, each value e2m1 * 2**-14 exactly: that fp16 has high byte
// s000eem0 (the magnitude eem lands on bits 11..9; E2M1's subnormal 0.5 on
// the fp16 subnormal 2**-15) and low byte 0.  The high bytes of the even
// codes (A) and the odd codes (B) are built four at a time, then paired.
__device__ __forceinline__ void e2m1x8_to_f16x2(uint32_t u, uint32_t (&p)[4]) {
    const uint32_t A = ((u << 1) & 0x0E0E0E0Eu) | ((u << 4) & 0x80808080u);  // codes 0, 2, 4, 6
    const uint32_t B = ((u >> 3) & 0x0E0E0E0Eu) | (u & 0x80808080u);         // codes 1, 3, 5, 7
    p[0] = __builtin_amdgcn_perm(B, A, 0x040C000Cu);  // (code 0, code 1)
    p[1] = __builtin_amdgcn_perm(B, A, 0x050C010Cu);  // (2, 3)
    p[2] = __builtin_amdgcn_perm(B, A, 0x060C020Cu);  // (4, 5)
    p[3] = __builtin_amdgcn_perm(B, A, 0x070C030Cu);  // (6, 7)
}

}  // namespace ql
