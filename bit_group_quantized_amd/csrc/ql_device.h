// Device-side helpers shared by the gfx950 kernels of this library.
//
// Group-affine 4-bit weights (Perplexity, "Optimizing on-device inference
// for Apple Silicon", section 在矩阵乘法期间进行权重反量化): a code q in
// 0..15 per weight, one fp16 scale s and bias b per 64 consecutive k of an
// output, w = s*q + b.  Codes are packed 8 per uint32 along K, least
// significant nibble first.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ql {

typedef _Float16 f16;
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kGroup = 64;

// fp16 with exponent field 25 (0x6400) is 1024 with a unit of 1 in the last
// mantissa place: OR-ing a value v < 1024 into the low 10 bits gives the
// fp16 number 1024 + v exactly.
constexpr uint32_t kMagic2 = 0x64006400u;

__device__ __forceinline__ float h2f(uint16_t bits) {
    return (float)__builtin_bit_cast(f16, bits);
}

// fp32 -> fp16, round to nearest even (the hardware conversion's default mode).
__device__ __forceinline__ uint16_t f2h(float v) {
    return __builtin_bit_cast(uint16_t, (f16)v);
}

__device__ __forceinline__ f16x2 as_f16x2(uint32_t u) { return __builtin_bit_cast(f16x2, u); }
__device__ __forceinline__ uint32_t as_u32(f16x2 h) { return __builtin_bit_cast(uint32_t, h); }

__device__ __forceinline__ float dot2(f16x2 a, f16x2 b, float c) {
    return __builtin_amdgcn_fdot2(a, b, c, false);
}

// (u & mask) | magic in one v_and_or_b32.  The compiler does not form this
// instruction by itself (it would need two literal operands); the mask goes
// in an SGPR and the magic constant in a VGPR.
__device__ __forceinline__ uint32_t and_or(uint32_t u, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(u), "s"(mask), "v"(magic));
    return r;
}

// Dequantize one word (codes k = 8w .. 8w+7 of one output) to 8 fp16 values
// in natural k order: out[j] = fp16(s*q_j + b), a single rounding (fma).
// Exact code pairs come from the 0x6400 exponent trick: (u & 0x000F000F) |
// magic = (1024 + q0, 1024 + q4), minus 1024; (u & 0x00F000F0) | magic =
// (1024 + 16 q1, 1024 + 16 q5), times 1/16 minus 64 (exact: 64 + q1 - 64).
__device__ __forceinline__ f16x8 dequant_word(uint32_t u, f16x2 s2, f16x2 b2) {
    const f16x2 off = {(f16)-1024.0f, (f16)-1024.0f};
    const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
    const f16x2 off64 = {(f16)-64.0f, (f16)-64.0f};
    const uint32_t magic = kMagic2;
    const uint32_t t = u >> 8;
    f16x2 p0 = as_f16x2(and_or(u, 0x000F000Fu, magic)) + off;                 // (q0, q4)
    f16x2 p1 = __builtin_elementwise_fma(as_f16x2(and_or(u, 0x00F000F0u, magic)), sixteenth, off64);  // (q1, q5)
    f16x2 p2 = as_f16x2(and_or(t, 0x000F000Fu, magic)) + off;                 // (q2, q6)
    f16x2 p3 = __builtin_elementwise_fma(as_f16x2(and_or(t, 0x00F000F0u, magic)), sixteenth, off64);  // (q3, q7)
    uint32_t w0 = as_u32(__builtin_elementwise_fma(p0, s2, b2));  // (w0, w4)
    uint32_t w1 = as_u32(__builtin_elementwise_fma(p1, s2, b2));  // (w1, w5)
    uint32_t w2 = as_u32(__builtin_elementwise_fma(p2, s2, b2));  // (w2, w6)
    uint32_t w3 = as_u32(__builtin_elementwise_fma(p3, s2, b2));  // (w3, w7)
    // Re-pair into natural order: (w0,w1) (w2,w3) (w4,w5) (w6,w7).
    uint32_t o0 = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
    uint32_t o1 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
    uint32_t o2 = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
    uint32_t o3 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
    u32x4 o = {o0, o1, o2, o3};
    return __builtin_bit_cast(f16x8, o);
}

// Activation pre-pairing for the dot-product form of the row GEMV.
// For one word u of codes q0..q7 (k = 8w .. 8w+7):
//   c0 = (u & 0x000F000F) | magic       = (1024 + q0,    1024 + q4)
//   c1 = (u & 0x00F000F0) | magic       = (1024 + 16 q1, 1024 + 16 q5)
//   c2 = ((u>>8) & 0x000F000F) | magic  = (1024 + q2,    1024 + q6)
//   c3 = ((u>>8) & 0x00F000F0) | magic  = (1024 + 16 q3, 1024 + 16 q7)
// With activation pairs x0 = (x0, x4), x1 = (x1/16, x5/16), x2 = (x2, x6),
// x3 = (x3/16, x7/16):  sum dot2(xi, ci) = sum_k x_k q_k + 1024 * (sum of
// all pair entries).  The constant is removed once per group.
struct XPairs {
    f16x2 p[4];
};

__device__ __forceinline__ XPairs make_xpairs(u32x4 xw) {
    // xw holds x0..x7 as fp16 pairs (x0,x1) (x2,x3) (x4,x5) (x6,x7).
    XPairs r;
    r.p[0] = as_f16x2(__builtin_amdgcn_perm(xw.z, xw.x, 0x05040100u));  // (x0, x4)
    r.p[2] = as_f16x2(__builtin_amdgcn_perm(xw.w, xw.y, 0x05040100u));  // (x2, x6)
    f16x2 a = as_f16x2(__builtin_amdgcn_perm(xw.z, xw.x, 0x07060302u));  // (x1, x5)
    f16x2 b = as_f16x2(__builtin_amdgcn_perm(xw.w, xw.y, 0x07060302u));  // (x3, x7)
    const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
    r.p[1] = a * sixteenth;
    r.p[3] = b * sixteenth;
    return r;
}

// Sum of the pair entries times 1024 (the constant of the dot-product form),
// and the plain sum of the eight activations (for the bias term).
__device__ __forceinline__ void xpairs_consts(const XPairs& r, u32x4 xw, float& c, float& xs) {
    // Sums of fp16 values as dot products with (1, 1): exact products, fp32 sums.
    const f16x2 one2 = {(f16)1.0f, (f16)1.0f};
    float sp = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sp = dot2(r.p[i], one2, sp);
    c = 1024.0f * sp;
    const f16x2 h[4] = {as_f16x2(xw.x), as_f16x2(xw.y), as_f16x2(xw.z), as_f16x2(xw.w)};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = dot2(h[i], one2, s);
    xs = s;
}

// Accumulate sum dot2(x pairs, code pairs) for one word into four partials.
__device__ __forceinline__ void dot_word(uint32_t u, const XPairs& x, float& d0, float& d1, float& d2, float& d3) {
    const uint32_t t = u >> 8;
    const uint32_t magic = kMagic2;
    d0 = dot2(x.p[0], as_f16x2(and_or(u, 0x000F000Fu, magic)), d0);
    d1 = dot2(x.p[1], as_f16x2(and_or(u, 0x00F000F0u, magic)), d1);
    d2 = dot2(x.p[2], as_f16x2(and_or(t, 0x000F000Fu, magic)), d2);
    d3 = dot2(x.p[3], as_f16x2(and_or(t, 0x00F000F0u, magic)), d3);
}

__device__ __forceinline__ u32x4 ld_u32x4(const void* p) {
    return *reinterpret_cast<const u32x4*>(p);
}

// Streaming load for weights that are read exactly once (non-temporal hint
// unless QL_STREAM_NT is 0).
#ifndef QL_STREAM_NT
#define QL_STREAM_NT 1
#endif
__device__ __forceinline__ u32x4 ld_stream_u32x4(const void* p) {
#if QL_STREAM_NT
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
    return *reinterpret_cast<const u32x4*>(p);
#endif
}

// 64-bit selection keys: the unsigned order of logit_key(v, i) is "larger
// v first, then smaller index i".  The upper word is the bit pattern of v
// made monotone (negative values inverted, positive values with the sign
// bit set), the lower word 0xFFFFFFFF - i.  No finite v maps to key 0.
__device__ __forceinline__ uint64_t logit_key(float v, int e) {
    uint32_t u = __float_as_uint(v);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)e);
}

__device__ __forceinline__ float key_logit(uint64_t k) {
    uint32_t u = (uint32_t)(k >> 32);
    u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
    return __uint_as_float(u);
}

__device__ __forceinline__ int key_index(uint64_t k) {
    return (int)(0xFFFFFFFFu - (uint32_t)k);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, true);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, true);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int lane) {
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum over the 64 lanes of a wave (all lanes active), uniform result.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = umax64(v, dpp_u64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = umax64(v, dpp_u64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = umax64(v, dpp_u64<0x141>(v));  // row_half_mirror
    v = umax64(v, dpp_u64<0x140>(v));  // row_mirror
    return umax64(umax64(readlane_u64(v, 0), readlane_u64(v, 16)),
                  umax64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

__device__ __forceinline__ float silu(float z) {
    return z / (1.0f + __expf(-z));
}

}  // namespace ql
