// FP8-E4M3 and E2M1 weight codes decoded with the gfx950 conversion
// instructions, shared by the codec GEMVs and the codec GEMMs.
//
// "待验证｜lithos-metal补Apple推理内核", section "一分钟内合并了什么": FP8
// E4M3 weights decoded two codes per half2, and an NVFP4 checkpoint (E2M1
// codes with E4M3 block scales).
//
// The conversions take the OCP formats: E4M3FN (exponent bias 7, subnormals
// m/8 * 2**-6, S.1111.111 = NaN, no infinity) and E2M1 (magnitudes 0, 0.5,
// 1, 1.5, 2, 3, 4, 6).  Every E4M3 and E2M1 value is exact in fp16, so the
// decoded codes are the format's values, NaN codes included.  The scale
// operand of the scaled conversions only contributes its power of two; it
// is 1 here and every real scale is applied by the caller.
#pragma once

#include "ql_device.h"

namespace ql {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Codes in bytes 0 and 1 of w (HI = false) or bytes 2 and 3 (HI = true) ->
// their E4M3 values as an fp16 pair, lower byte first.
template <bool HI>
__device__ __forceinline__ f16x2 e4m3x2_to_f16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HI);
}

// Byte B of w as an E4M3 value in fp32 (exact; NaN for S.1111.111).
template <int B>
__device__ __forceinline__ float e4m3_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_f32_fp8(w, B);
}

// The two E2M1 codes of byte B of w (low nibble first) as an fp16 pair.
template <int B>
__device__ __forceinline__ f16x2 e2m1x2_to_f16x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, B);
}

// The same two codes as fp32 values.
template <int B>
__device__ __forceinline__ f32x2 e2m1x2_to_f32x2(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
}

// Two fp32 values -> fp16 pair, each rounded to nearest even.
__device__ __forceinline__ uint32_t f32x2_to_f16x2(float lo, float hi) {
    const f16x2 r = {(f16)lo, (f16)hi};
    return as_u32(r);
}

}  // namespace ql
