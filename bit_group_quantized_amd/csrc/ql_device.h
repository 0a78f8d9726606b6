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

#include <type_traits>

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
// Byte m of the word holds codes 2m (low nibble) and 2m+1 (high nibble).  A
// byte permute puts byte m into bytes 0 and 2; under the 0x6400 exponent the
// low nibble of byte 0 and the high nibble of byte 2 give the fp16 pair
// (1024 + q_2m, 1024 + 16 q_2m+1), and one packed fma with (1, 1/16) and
// (-1024, -64) turns it into (q_2m, q_2m+1) exactly (64 + q - 64 for the
// high half).  The pair comes out already in output order, so no permute is
// needed after the scale-and-bias fma: 16 instructions per word.
__device__ __forceinline__ f16x8 dequant_word(uint32_t u, f16x2 s2, f16x2 b2) {
    const f16x2 unit = {(f16)1.0f, (f16)0.0625f};
    const f16x2 off = {(f16)-1024.0f, (f16)-64.0f};
    const uint32_t magic = kMagic2;
    uint32_t o[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t d = __builtin_amdgcn_perm(u, u, 0x0c000c00u | (uint32_t)m | ((uint32_t)m << 16));
        const f16x2 q = __builtin_elementwise_fma(as_f16x2(and_or(d, 0x00F0000Fu, magic)), unit, off);
        o[m] = as_u32(__builtin_elementwise_fma(q, s2, b2));
    }
    const u32x4 r = {o[0], o[1], o[2], o[3]};
    return __builtin_bit_cast(f16x8, r);
}

// ---- bf16 ------------------------------------------------------------------
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 pattern -> float (exact: a bf16 is the upper half of a float).
__device__ __forceinline__ float bf2f(uint16_t bits) { return __uint_as_float((uint32_t)bits << 16); }

// float -> bf16 pattern, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f2bf(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 p = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, p);
}

// Dequantize one word (codes k = 8w .. 8w+7) to 8 bf16 values in natural k
// order: bf16(s*q + b) from one fp32 fma per value (exact for the weights of
// this format, whose scale*code + bias needs far fewer than 24 bits) and one
// rounding to bf16.  The nibbles are split into bytes and converted with
// v_cvt_f32_ubyte.
__device__ __forceinline__ u32x4 dequant_word_bf16(uint32_t u, float s, float b) {
    const uint32_t lo = u & 0x0F0F0F0Fu;          // q0 q2 q4 q6 in bytes 0..3
    const uint32_t hi = (u >> 4) & 0x0F0F0F0Fu;   // q1 q3 q5 q7
    auto byte = [](uint32_t w, int k) { return (float)((w >> (8 * k)) & 0xFFu); };  // v_cvt_f32_ubyteN
    u32x4 o;
    o.x = pack_bf16x2(fmaf(byte(lo, 0), s, b), fmaf(byte(hi, 0), s, b));
    o.y = pack_bf16x2(fmaf(byte(lo, 1), s, b), fmaf(byte(hi, 1), s, b));
    o.z = pack_bf16x2(fmaf(byte(lo, 2), s, b), fmaf(byte(hi, 2), s, b));
    o.w = pack_bf16x2(fmaf(byte(lo, 3), s, b), fmaf(byte(hi, 3), s, b));
    return o;
}

// bf16 row GEMV: for one word u and activations x0..x7 (bf16 pairs (x0,x1)
// (x2,x3) (x4,x5) (x6,x7) in xw), code pairs come from the 0x4300 exponent
// (bf16 128 with unit 1 in the last place): ((u >> 4j) & 0x000F000F) | magic
// = (128 + q_j, 128 + q_{j+4}), paired with (x_j, x_{j+4}).  The products
// are exact in fp32; sum_k x_k (128 + q_k) = sum_k x_k q_k + 128 sum_k x_k.
struct XPairsBf {
    bf16x2 p[4];  // (x0,x4) (x1,x5) (x2,x6) (x3,x7)
};

__device__ __forceinline__ XPairsBf make_xpairs_bf(u32x4 xw) {
    XPairsBf r;
    r.p[0] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(xw.z, xw.x, 0x05040100u));
    r.p[1] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(xw.z, xw.x, 0x07060302u));
    r.p[2] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(xw.w, xw.y, 0x05040100u));
    r.p[3] = __builtin_bit_cast(bf16x2, __builtin_amdgcn_perm(xw.w, xw.y, 0x07060302u));
    return r;
}

__device__ __forceinline__ float dot2bf(bf16x2 a, bf16x2 b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

// Sum of the eight activations of one word (dot products with (1, 1)).
__device__ __forceinline__ float xsum_bf(const XPairsBf& r) {
    const bf16x2 one2 = {(__bf16)1.0f, (__bf16)1.0f};
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) s = dot2bf(r.p[i], one2, s);
    return s;
}

__device__ __forceinline__ void dot_word_bf(uint32_t u, const XPairsBf& x, float& d0, float& d1, float& d2,
                                            float& d3) {
    constexpr uint32_t magic = 0x43004300u;
    d0 = dot2bf(x.p[0], __builtin_bit_cast(bf16x2, and_or(u, 0x000F000Fu, magic)), d0);
    d1 = dot2bf(x.p[1], __builtin_bit_cast(bf16x2, and_or(u >> 4, 0x000F000Fu, magic)), d1);
    d2 = dot2bf(x.p[2], __builtin_bit_cast(bf16x2, and_or(u >> 8, 0x000F000Fu, magic)), d2);
    d3 = dot2bf(x.p[3], __builtin_bit_cast(bf16x2, and_or(u >> 12, 0x000F000Fu, magic)), d3);
}

// Activation pre-pairing for the dot-product form of the row GEMV.
// For one word u of codes q0..q7 (k = 8w .. 8w+7):
//   c0 = (u & 0x000F000F) | magic       = (1024 + q0,    1024 + q4)
//   c1 = (u & 0x00F000F0) | magic       = (1024 + 16 q1, 1024 + 16 q5)
//   c2 = ((u>>8) & 0x000F000F) | magic  = (1024 + q2,    1024 + q6)
//   c3 = ((u>>8) & 0x00F000F0) | magic  = (1024 + 16 q3, 1024 + 16 q7)
// The activations are paired unscaled, p0 = (x0, x4), p1 = (x1, x5),
// p2 = (x2, x6), p3 = (x3, x7), so every product x * c is exact in fp32 for
// any fp16 x (subnormal ones included).  With d_i = sum dot2(p_i, c_i):
//   (d0 + d2) + (d1 + d3) / 16 = sum_k x_k q_k + 1024 * (x0+x2+x4+x6)
//                                             + 64 * (x1+x3+x5+x7);
// the division by 16 is exact in fp32 and the constant is removed once per
// chunk of codes.
struct XPairs {
    f16x2 p[4];
};

__device__ __forceinline__ XPairs make_xpairs(u32x4 xw) {
    // xw holds x0..x7 as fp16 pairs (x0,x1) (x2,x3) (x4,x5) (x6,x7).
    XPairs r;
    r.p[0] = as_f16x2(__builtin_amdgcn_perm(xw.z, xw.x, 0x05040100u));  // (x0, x4)
    r.p[1] = as_f16x2(__builtin_amdgcn_perm(xw.z, xw.x, 0x07060302u));  // (x1, x5)
    r.p[2] = as_f16x2(__builtin_amdgcn_perm(xw.w, xw.y, 0x05040100u));  // (x2, x6)
    r.p[3] = as_f16x2(__builtin_amdgcn_perm(xw.w, xw.y, 0x07060302u));  // (x3, x7)
    return r;
}

// The constant of the dot-product form, 1024 * (sum of the even-k
// activations) + 64 * (sum of the odd-k ones), and the plain sum of the
// eight activations (for the bias term).  Sums of fp16 values as dot
// products with (1, 1): exact products, fp32 sums.
__device__ __forceinline__ void xpairs_consts(const XPairs& r, float& c, float& xs) {
    const f16x2 one2 = {(f16)1.0f, (f16)1.0f};
    const float ev = dot2(r.p[2], one2, dot2(r.p[0], one2, 0.f));
    const float od = dot2(r.p[3], one2, dot2(r.p[1], one2, 0.f));
    c = fmaf(1024.0f, ev, 64.0f * od);
    xs = ev + od;
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

// The four partials of dot_word combined: the odd-k codes entered as 16 q,
// so their partials are scaled by 1/16 (exact in fp32).
__device__ __forceinline__ float dot_sum(float d0, float d1, float d2, float d3) {
    return fmaf(d1 + d3, 0.0625f, d0 + d2);
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

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// v_permlane32_swap on (a, b): lanes 0-31 get a's two halves, lanes 32-63
// b's; their sum is a's cross-half total in the lower half of the wave and
// b's in the upper half.  v_permlane16_swap does the same for pairs of
// 16-lane rows (even rows end with a, odd rows with b).
__device__ __forceinline__ float swap_add32(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(unsigned, a),
                                                    __builtin_bit_cast(unsigned, b), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}
__device__ __forceinline__ float swap_add16(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__builtin_bit_cast(unsigned, a),
                                                    __builtin_bit_cast(unsigned, b), false, false);
    return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Whole-wave (64-lane team) row reduction: every lane holds partials of the
// same R rows; afterwards lane l holds the total of row l / (64 / R).  The
// halving steps across 32- and 16-lane rows exchange whole rows with the
// permlane swaps (no selects); inside 16-lane rows DPP pairs lane i with
// 15 - i, then 7 - i, then the quad permutations finish each group.
template <int R>
__device__ __forceinline__ float reduce_rows64(const float (&v)[R], int lane, int& row) {
    static_assert(R == 1 || R == 2 || R == 4 || R == 8, "1, 2, 4 or 8 rows");
    constexpr int R1 = (R > 1) ? R / 2 : 1;
    float a[R1];
#pragma unroll
    for (int i = 0; i < R1; ++i) a[i] = (R > 1) ? swap_add32(v[i], v[i + R1]) : swap_add32(v[0], v[0]);
    constexpr int R2 = (R1 > 1) ? R1 / 2 : 1;
    float b[R2];
#pragma unroll
    for (int i = 0; i < R2; ++i) b[i] = (R1 > 1) ? swap_add16(a[i], a[i + R2]) : swap_add16(a[0], a[0]);
    float t;
    if constexpr (R2 > 1) {
        const bool hi8 = (lane & 8) != 0;  // lanes 8-15 of a 16-lane row keep b[1]
        t = (hi8 ? b[1] : b[0]) + dpp_mov<0x140>(hi8 ? b[0] : b[1]);  // row_mirror
    } else {
        t = b[0] + dpp_mov<0x140>(b[0]);
    }
    t += dpp_mov<0x141>(t);  // row_half_mirror
    t += dpp_mov<0x4E>(t);   // quad_perm [2,3,0,1]
    t += dpp_mov<0xB1>(t);   // quad_perm [1,0,3,2]
    row = lane / (64 / R);
    return t;
}

// Team reduction over TPR consecutive lanes.
template <int TPR>
__device__ __forceinline__ float team_sum(float v) {
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

// Row reduction of a team of TPR lanes holding partials of the same R rows:
// afterwards the lanes with (lane % TPR) & (TPR / R - 1) == 0 hold one row
// total each, row = the returned index.
template <int TPR, int R>
__device__ __forceinline__ float reduce_rows(float (&v)[R], int lr, int& row) {
    static_assert(R <= TPR, "each row needs its own lane after the halving steps");
    if constexpr (TPR == 64 && (R == 1 || R == 2 || R == 4 || R == 8)) return reduce_rows64<R>(v, lr, row);
    int base = 0;
#pragma unroll
    for (int off = TPR / 2, cnt = R; off >= 1; off >>= 1) {
        if (cnt > 1) {
            const bool hi = (lr & off) != 0;
            const int h = cnt / 2;
#pragma unroll
            for (int i = 0; i < h; ++i) {
                const float send = hi ? v[i] : v[i + h];
                const float keep = hi ? v[i + h] : v[i];
                v[i] = keep + __shfl_xor(send, off, 64);
            }
            if (hi) base += h;
            cnt = h;
        } else {
            v[0] += __shfl_xor(v[0], off, 64);
        }
    }
    row = base;
    return v[0];
}

// Maximum over the 64 lanes of a wave (all lanes active), uniform result:
// DPP inside each 16-lane row, then the four row maxima through readlane.
__device__ __forceinline__ float wave_max_f32(float v) {
    v = fmaxf(v, dpp_mov<0xB1>(v));   // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp_mov<0x4E>(v));   // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp_mov<0x141>(v));  // row_half_mirror
    v = fmaxf(v, dpp_mov<0x140>(v));  // row_mirror
    const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const float c = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const float e = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    return fmaxf(fmaxf(a, b), fmaxf(c, e));
}

// Maximum of a 32-bit unsigned value over the 64 lanes of a wave, uniform.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    auto dpp = [](uint32_t x, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xF, 0xF, true);
    };
    v = max(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
    v = max(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
    v = max(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    v = max(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
    const uint32_t a = __builtin_amdgcn_readlane((int)v, 0), b = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = __builtin_amdgcn_readlane((int)v, 32), e = __builtin_amdgcn_readlane((int)v, 48);
    return max(max(a, b), max(c, e));
}

// Minimum of a 32-bit unsigned value over the 64 lanes of a wave, uniform.
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    auto dpp = [](uint32_t x, auto ctrl) {
        return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, decltype(ctrl)::value, 0xF, 0xF, true);
    };
    v = min(v, dpp(v, std::integral_constant<int, 0xB1>{}));   // quad_perm [1,0,3,2]
    v = min(v, dpp(v, std::integral_constant<int, 0x4E>{}));   // quad_perm [2,3,0,1]
    v = min(v, dpp(v, std::integral_constant<int, 0x141>{}));  // row_half_mirror
    v = min(v, dpp(v, std::integral_constant<int, 0x140>{}));  // row_mirror
    const uint32_t a = __builtin_amdgcn_readlane((int)v, 0), b = __builtin_amdgcn_readlane((int)v, 16);
    const uint32_t c = __builtin_amdgcn_readlane((int)v, 32), e = __builtin_amdgcn_readlane((int)v, 48);
    return min(min(a, b), min(c, e));
}

// Monotone 32-bit key of a float: unsigned order = numeric order (the sign
// bit flipped for positive values, all bits for negative ones); the key of
// -inf is 0x007FFFFF, so no float maps to 0.
__device__ __forceinline__ uint32_t mono32(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float unmono32(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
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

// fp16 bits of a * b with one rounding from the exact product
// (v_fma_mixlo_f16 with fp32 sources and a zero addend).  Left to itself the
// compiler picks this form in some kernels and an fp32 multiply followed by
// a conversion (two roundings) in others; the gated activations of every
// kernel go through this helper so that they round alike.
__device__ __forceinline__ uint16_t mul_to_f16(float a, float b) {
    uint32_t r;
    asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a), "v"(b));
    return (uint16_t)r;
}

}  // namespace ql
