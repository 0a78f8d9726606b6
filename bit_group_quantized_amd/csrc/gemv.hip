// Row-parallel w4 GEMV kernels (batch-1 decode) and their routed-expert
// variants for the decode MoE layer.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon":
//  * 优化单行权重路径 - single-row GEMV: groups of lanes cooperate on outputs
//    while reading different parts of the weight matrix in parallel; the
//    work is bound by weight reads, so it runs on the vector ALUs.
//  * 在矩阵乘法期间进行权重反量化 - w = scale*code + bias per 64-wide group;
//    here dequantization never leaves registers.
//  * 减少中间状态和流量 - decode fuses the expert gate and up projections with
//    the gated activation, and the down projection with the routing weights
//    and the shared expert.
//
// Mapping on gfx950 (wave64): a "row team" of TPR lanes owns one output row;
// lane l of a team owns quantization groups g = l, l + TPR, ... (GPL of
// them).  Per group a lane issues two 128-bit loads (64 codes) plus the
// group's scale and bias, so a team streams its row with fully coalesced
// loads.  The activation slice of a lane is loaded once, pre-paired for
// v_dot2_f32_f16, and kept in registers for every row the lane visits.
// The bias term uses sum_k x_k (s q_k + b) = s * sum_k x_k q_k + b * sum_k x_k
// with the per-group activation sum computed once.
#include <type_traits>

#include "ql_codecs.h"
#include "ql_device.h"
#include "ql_internal.h"
#include "ql_topk.h"

namespace ql {

namespace {


// Dot product of one group (8 words) with pre-paired activations.
__device__ __forceinline__ float group_dot(const u32x4& c0, const u32x4& c1, const XPairs* xp) {
    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
    dot_word(c0.x, xp[0], d0, d1, d2, d3);
    dot_word(c0.y, xp[1], d0, d1, d2, d3);
    dot_word(c0.z, xp[2], d0, d1, d2, d3);
    dot_word(c0.w, xp[3], d0, d1, d2, d3);
    dot_word(c1.x, xp[4], d0, d1, d2, d3);
    dot_word(c1.y, xp[5], d0, d1, d2, d3);
    dot_word(c1.z, xp[6], d0, d1, d2, d3);
    dot_word(c1.w, xp[7], d0, d1, d2, d3);
    return dot_sum(d0, d1, d2, d3);
}

// Load and pre-pair the 64 activations of group g.
__device__ __forceinline__ void load_group_x(const uint16_t* __restrict__ x, int g, XPairs* xp, float& c, float& xs) {
    c = 0.f;
    xs = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
        u32x4 xw = ld_u32x4(x + g * kGroup + w * 8);
        xp[w] = make_xpairs(xw);
        float cw, sw;
        xpairs_consts(xp[w], cw, sw);
        c += cw;
        xs += sw;
    }
}

// ---------------------------------------------------------------------------
// Dense GEMV: y[n] = sum_k x[k] W[k][n].
// GPL > 0: groups per lane fixed at compile time, activations in registers.
// GPL == 0: runtime group count, activations re-read (L1/L2) per row.
// ---------------------------------------------------------------------------
template <int TPR, int GPL, int UNROLL>
__global__ void __launch_bounds__(256)
gemv_w4_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
               const uint16_t* __restrict__ bi, const uint16_t* __restrict__ x,
               uint16_t* __restrict__ y, int K, int N) {
    constexpr int TEAMS = 64 / TPR;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int gwave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int nwaves = gridDim.x * (blockDim.x / 64);
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int stride = nwaves * TEAMS;

    if constexpr (GPL > 0) {
        XPairs xp[GPL][8];
        float xc[GPL], xsum[GPL];
#pragma unroll
        for (int i = 0; i < GPL; ++i) load_group_x(x, lr + i * TPR, xp[i], xc[i], xsum[i]);

        for (int r0 = gwave * TEAMS + team; r0 < N; r0 += stride * UNROLL) {
            u32x4 cw[UNROLL][GPL][2];
            uint16_t s[UNROLL][GPL], b[UNROLL][GPL];
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                const int rr = min(r0 + u * stride, N - 1);
#pragma unroll
                for (int i = 0; i < GPL; ++i) {
                    const int g = lr + i * TPR;
                    const uint32_t* p = qw + (size_t)rr * wpr + g * 8;
                    cw[u][i][0] = ld_stream_u32x4(p);
                    cw[u][i][1] = ld_stream_u32x4(p + 4);
                    s[u][i] = sc[(size_t)rr * G + g];
                    b[u][i] = bi[(size_t)rr * G + g];
                }
            }
#pragma unroll
            for (int u = 0; u < UNROLL; ++u) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i < GPL; ++i) {
                    const float d = group_dot(cw[u][i][0], cw[u][i][1], xp[i]);
                    acc += h2f(s[u][i]) * (d - xc[i]) + h2f(b[u][i]) * xsum[i];
                }
                acc = team_sum<TPR>(acc);
                const int row = r0 + u * stride;
                if (lr == 0 && row < N) y[row] = f2h(acc);
            }
        }
    } else {
        const int gpl = G / TPR;
        for (int r0 = gwave * TEAMS + team; r0 < N; r0 += stride) {
            float acc = 0.f;
            for (int i = 0; i < gpl; ++i) {
                const int g = lr + i * TPR;
                const uint32_t* p = qw + (size_t)r0 * wpr + g * 8;
                const u32x4 c0 = ld_stream_u32x4(p);
                const u32x4 c1 = ld_stream_u32x4(p + 4);
                const float s = h2f(sc[(size_t)r0 * G + g]);
                const float b = h2f(bi[(size_t)r0 * G + g]);
                XPairs xp[8];
                float c, xs;
                load_group_x(x, g, xp, c, xs);
                acc += s * (group_dot(c0, c1, xp) - c) + b * xs;
            }
            // r0 is uniform per team and teams of one wave may differ in trip
            // count only at the very end; every lane of a team reaches here.
            acc = team_sum<TPR>(acc);
            if (lr == 0) y[r0] = f2h(acc);
        }
    }
}

// ---------------------------------------------------------------------------
// Chunked dense GEMV: every lane owns 16-byte chunks of codes (32 codes, half
// a quantization group) at a fixed K position and visits R consecutive rows.
// One wave instruction then reads TPR*16 contiguous bytes of each of
// 64/TPR rows: with K = 2048 a whole 1 KB row per instruction.  All R rows'
// loads are issued before any arithmetic (R*V 128-bit loads in flight per
// lane), and the R partial sums are reduced across the team by halving: at
// each of the first log2(R) exchange steps a lane keeps half of its rows
// and adds the partner's copy of them, so R rows cost R-1 shuffles, not
// R*log2(TPR).
// ---------------------------------------------------------------------------

// Prologue and epilogue variants of the chunked GEMV (the decode steps on
// either side of a projection; Perplexity, "Optimizing on-device inference
// for Apple Silicon", sections 减少中间状态和流量 and 将 token 交接保留在 GPU 上):
//  * GV_RMSNORM: the activation row is RMS-normalized first.  A team of TPR
//    lanes holds all K activations, so the sum of squares is one team
//    reduction (pairwise exchanges, so every lane and every team gets the
//    same bits); each lane then scales its own chunks, x * r * gamma rounded
//    once to fp16, before pairing them for the dot products.
//  * GV_ARGMAX: instead of (or besides) the fp16 outputs, each block writes
//    the largest 64-bit selection key (fp32 output value, then lower row)
//    of its rows; argmax_finish_kernel reduces those keys to the token id.
enum { GV_PLAIN = 0, GV_RMSNORM = 1 };
enum { GV_STORE = 0, GV_ARGMAX = 1 };

// The work of block `blk` of the chunked GEMV (rows 4 * TEAMS * R * blk ..).
template <int TPR, int V, int R, int PRO, int EPI>
__device__ __forceinline__ void chunked_body(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                                             const uint16_t* __restrict__ bi, const uint16_t* __restrict__ x,
                                             uint16_t* __restrict__ y, int K, int N,
                                             const uint16_t* __restrict__ gamma, float eps,
                                             uint64_t* __restrict__ partials, int blk) {
    constexpr int TEAMS = 64 / TPR;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int gwave = blk * (blockDim.x / 64) + threadIdx.x / 64;
    const int row0 = (gwave * TEAMS + team) * R;

    // Activations of this lane's chunks (L2-resident after the first wave)
    // and then the codes, scales and biases of R rows: every load is issued
    // before any arithmetic, activations first so that work on row 0 can
    // start while later rows are still in flight.
    u32x4 xr[V][4];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) xr[v][w] = ld_u32x4(x + (lr + v * TPR) * 32 + w * 8);
    u32x4 gr[(PRO == GV_RMSNORM) ? V : 1][4];
    if constexpr (PRO == GV_RMSNORM) {
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int w = 0; w < 4; ++w) gr[v][w] = ld_u32x4(gamma + (lr + v * TPR) * 32 + w * 8);
    }
    u32x4 cw[R][V];
    uint16_t s[R][V], b[R][V];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int hg = lr + v * TPR;  // half-group index along K
            cw[r][v] = ld_stream_u32x4(qw + (size_t)row * wpr + hg * 4);
            s[r][v] = sc[(size_t)row * G + (hg >> 1)];
            b[r][v] = bi[(size_t)row * G + (hg >> 1)];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (PRO == GV_RMSNORM) {
        // Sum of squares: exact fp16 squares, fp32 sums (dot2 with itself).
        float ss = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                ss = dot2(as_f16x2(xr[v][w].x), as_f16x2(xr[v][w].x), ss);
                ss = dot2(as_f16x2(xr[v][w].y), as_f16x2(xr[v][w].y), ss);
                ss = dot2(as_f16x2(xr[v][w].z), as_f16x2(xr[v][w].z), ss);
                ss = dot2(as_f16x2(xr[v][w].w), as_f16x2(xr[v][w].w), ss);
            }
        if constexpr (TPR == 64) {
            // Whole-wave team: permlane swaps and DPP, every lane gets the total.
            const float one[1] = {ss};
            int unused;
            ss = reduce_rows64<1>(one, lane, unused);
        } else {
            ss = team_sum<TPR>(ss);
        }
        const float rinv = 1.0f / __builtin_sqrtf(ss / (float)K + eps);
        auto scale2 = [&](uint32_t xu, uint32_t gu) {
            const f16x2 xh = as_f16x2(xu), gh = as_f16x2(gu);
            const uint32_t lo = f2h(((float)xh[0] * rinv) * (float)gh[0]);
            const uint32_t hi = f2h(((float)xh[1] * rinv) * (float)gh[1]);
            return lo | (hi << 16);
        };
#pragma unroll
        for (int v = 0; v < V; ++v)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                xr[v][w].x = scale2(xr[v][w].x, gr[v][w].x);
                xr[v][w].y = scale2(xr[v][w].y, gr[v][w].y);
                xr[v][w].z = scale2(xr[v][w].z, gr[v][w].z);
                xr[v][w].w = scale2(xr[v][w].w, gr[v][w].w);
            }
    }
    XPairs xp[V][4];
    float xc[V], xs[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        xc[v] = 0.f;
        xs[v] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            xp[v][w] = make_xpairs(xr[v][w]);
            float cw_, sw_;
            xpairs_consts(xp[v][w], cw_, sw_);
            xc[v] += cw_;
            xs[v] += sw_;
        }
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
            dot_word(cw[r][v].x, xp[v][0], d0, d1, d2, d3);
            dot_word(cw[r][v].y, xp[v][1], d0, d1, d2, d3);
            dot_word(cw[r][v].z, xp[v][2], d0, d1, d2, d3);
            dot_word(cw[r][v].w, xp[v][3], d0, d1, d2, d3);
            const float d = dot_sum(d0, d1, d2, d3);
            acc[r] += h2f(s[r][v]) * (d - xc[v]) + h2f(b[r][v]) * xs[v];
        }
    }
    int rsel;
    const float tot = reduce_rows<TPR, R>(acc, lr, rsel);
    const bool owner = (lr & (TPR / R - 1)) == 0 && row0 + rsel < N;
    if constexpr (EPI == GV_STORE) {
        if (owner) y[row0 + rsel] = f2h(tot);
    } else {
        if (owner && y) y[row0 + rsel] = f2h(tot);
        // NaN outputs never win (key 0, the "nothing" key).
        uint64_t key = (owner && tot == tot) ? logit_key(tot, row0 + rsel) : 0;
        key = wave_max_u64(key);
        __shared__ uint64_t wkeys[4];
        if (lane == 0) wkeys[threadIdx.x >> 6] = key;
        __syncthreads();
        if (threadIdx.x == 0) partials[blk] = umax64(umax64(wkeys[0], wkeys[1]), umax64(wkeys[2], wkeys[3]));
    }
}

template <int TPR, int V, int R, int PRO, int EPI>
__global__ void __launch_bounds__(256)
gemv_w4_chunked_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                       const uint16_t* __restrict__ bi, const uint16_t* __restrict__ x,
                       uint16_t* __restrict__ y, int K, int N, const uint16_t* __restrict__ gamma,
                       float eps, uint64_t* __restrict__ partials) {
    chunked_body<TPR, V, R, PRO, EPI>(qw, sc, bi, x, y, K, N, gamma, eps, partials, blockIdx.x);
}

// Several matrices that share the activation row x (same K) in one launch:
// the grid is the concatenation of the matrices' own chunked-GEMV grids
// (matrix i owns blocks block0[i] .. block0[i+1]-1) and every matrix keeps
// the rows per wave (R or 2) its own launch would use, so each output has
// the bits of the separate call.  One launch instead of several saves the
// per-launch dispatch gap, which at K = 2048, N = 8192 is a third of the
// kernel's time.
struct GemvMulti {
    const uint32_t* qw[QL_GEMV_MULTI_MAX];
    const uint16_t* sc[QL_GEMV_MULTI_MAX];
    const uint16_t* bi[QL_GEMV_MULTI_MAX];
    uint16_t* y[QL_GEMV_MULTI_MAX];
    int N[QL_GEMV_MULTI_MAX];
    int small_r[QL_GEMV_MULTI_MAX];  // 1: two rows per wave
    int block0[QL_GEMV_MULTI_MAX + 1];
    int count;
};

template <int TPR, int V, int R>
__global__ void __launch_bounds__(256)
gemv_w4_multi_kernel(const GemvMulti m, const uint16_t* __restrict__ x, int K) {
    int i = 0;
    for (int j = 1; j < m.count; ++j)
        if ((int)blockIdx.x >= m.block0[j]) i = j;
    const int blk = blockIdx.x - m.block0[i];
    if constexpr (R > 2) {
        if (m.small_r[i]) {
            chunked_body<TPR, V, 2, GV_PLAIN, GV_STORE>(m.qw[i], m.sc[i], m.bi[i], x, m.y[i], K, m.N[i], nullptr,
                                                        0.f, nullptr, blk);
            return;
        }
    }
    chunked_body<TPR, V, R, GV_PLAIN, GV_STORE>(m.qw[i], m.sc[i], m.bi[i], x, m.y[i], K, m.N[i], nullptr, 0.f,
                                                nullptr, blk);
}

// bf16 variant of the chunked GEMV: bf16 activations, scales, biases and
// outputs ([PPLX] dequantization section: the page's checkpoint keeps scale
// and bias in bf16).  Same lane layout as above; the codes enter v_dot2 as
// bf16 128 + q (0x4300 exponent) against activation pairs (x_j, x_{j+4}),
// and 128 * sum(x) is removed per chunk.
template <int TPR, int V, int R>
__global__ void __launch_bounds__(256)
gemv_w4_bf16_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                    const uint16_t* __restrict__ bi, const uint16_t* __restrict__ x,
                    uint16_t* __restrict__ y, int K, int N) {
    constexpr int TEAMS = 64 / TPR;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int gwave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int row0 = (gwave * TEAMS + team) * R;
    u32x4 xr[V][4];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) xr[v][w] = ld_u32x4(x + (lr + v * TPR) * 32 + w * 8);
    u32x4 cw[R][V];
    uint16_t s[R][V], b[R][V];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int hg = lr + v * TPR;
            cw[r][v] = ld_stream_u32x4(qw + (size_t)row * wpr + hg * 4);
            s[r][v] = sc[(size_t)row * G + (hg >> 1)];
            b[r][v] = bi[(size_t)row * G + (hg >> 1)];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    XPairsBf xp[V][4];
    float xs[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
        xs[v] = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            xp[v][w] = make_xpairs_bf(xr[v][w]);
            xs[v] += xsum_bf(xp[v][w]);
        }
    }
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
            dot_word_bf(cw[r][v].x, xp[v][0], d0, d1, d2, d3);
            dot_word_bf(cw[r][v].y, xp[v][1], d0, d1, d2, d3);
            dot_word_bf(cw[r][v].z, xp[v][2], d0, d1, d2, d3);
            dot_word_bf(cw[r][v].w, xp[v][3], d0, d1, d2, d3);
            const float d = (d0 + d2) + (d1 + d3);
            acc[r] += bf2f(s[r][v]) * (d - 128.0f * xs[v]) + bf2f(b[r][v]) * xs[v];
        }
    }
    int rsel;
    const float tot = reduce_rows<TPR, R>(acc, lr, rsel);
    if ((lr & (TPR / R - 1)) == 0 && row0 + rsel < N) y[row0 + rsel] = f2bf(tot);
}

// Largest of n block keys -> token id (0 when no output was comparable).
__global__ void __launch_bounds__(1024)
argmax_finish_kernel(const uint64_t* __restrict__ partials, int n, int N, int32_t* __restrict__ token) {
    uint64_t best = 0;
    for (int i = threadIdx.x; i < n; i += 1024) best = umax64(best, partials[i]);
    best = wave_max_u64(best);
    __shared__ uint64_t wkeys[16];
    if ((threadIdx.x & 63) == 0) wkeys[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint64_t b = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) b = umax64(b, wkeys[i]);
        const int t = (b == 0) ? 0 : key_index(b);
        token[0] = min(max(t, 0), N - 1);
    }
}

// The input row of the token held in device memory: row `token` of a w4
// embedding table (N tokens, K = hidden width), dequantized to fp16 with one
// rounding, one 16-byte store per word of 8 codes.  An id outside [0, N)
// gives a row of zeros and reads no table memory.
__global__ void __launch_bounds__(256)
embed_w4_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                const uint16_t* __restrict__ bi, const int32_t* __restrict__ token,
                uint16_t* __restrict__ x, int K, int N) {
    const int w = blockIdx.x * 256 + threadIdx.x;
    if (w >= K / 8) return;
    const int t = token[0];
    u32x4 out = {0u, 0u, 0u, 0u};
    if (t >= 0 && t < N) {
        const int G = K / kGroup;
        const uint32_t u = qw[(size_t)t * (K / 8) + w];
        const f16 sv = __builtin_bit_cast(f16, sc[(size_t)t * G + (w >> 3)]);
        const f16 bv = __builtin_bit_cast(f16, bi[(size_t)t * G + (w >> 3)]);
        out = __builtin_bit_cast(u32x4, dequant_word(u, f16x2{sv, sv}, f16x2{bv, bv}));
    }
    *reinterpret_cast<u32x4*>(x + 8 * (size_t)w) = out;
}

// ---------------------------------------------------------------------------
// Routed-expert rows (decode MoE), chunked like the dense GEMV.  Row r <
// T*topk of the routed layout is (expert, token) = row_info[r], written by
// the dispatch step; rows T*topk .. T*topk+T-1 are the tokens multiplied by
// the shared expert.  One wave per block.
//
// MODE 0 (gate_up + SiLU): the wave's R weight rows are R/2 gate rows n and
//   the R/2 matching up rows n + N/2; after the halving reduction the lane
//   holding gate row n and the lane holding up row n differ only in the
//   first halving bit, so one more exchange brings them together.
// MODE 1 (down): R output rows.
// ---------------------------------------------------------------------------
// The lane's 16-byte chunks of activation row `xrow`.
template <int TPR, int V>
__device__ __forceinline__ void rows_load_x(const uint16_t* __restrict__ X, int xrow, int K, int lr,
                                            u32x4 (&xr)[V][4]) {
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) xr[v][w] = ld_u32x4(X + (size_t)xrow * K + (lr + v * TPR) * 32 + w * 8);
}

// Weight formats of the decode rows (WF): 0 = w4 (codes, fp16 scale and bias
// per 64); 1 = FP8-E4M3 codes [N][K] (bytes, through wq) with an fp16 scale
// per 64 (ws) and no bias; 2 = NVFP4: E2M1 codes in the w4 packing, E4M3
// block-scale bytes [N][K/16] (through ws) and the matrix's global scale.
// A lane's chunk is always 32 codes (k = 32c .. 32c+31) against the same 32
// activations; the codec chunks are dotted as the codec GEMVs do (exact
// fp16 code values in v_dot2_f32_f16, scales on fp32 partial sums).
template <int WF>
struct RowChunk {
    u32x4 c[(WF == 1) ? 2 : 1];  // codes: 16 bytes (w4, NVFP4) or 32 (FP8)
    uint16_t s, b;               // fp16 scale and bias (w4), scale (FP8), the two block-scale bytes (NVFP4)
};

template <int WF>
__device__ __forceinline__ RowChunk<WF> row_chunk_load(const uint32_t* __restrict__ wq,
                                                       const uint16_t* __restrict__ ws,
                                                       const uint16_t* __restrict__ wb, int row, int hg,
                                                       int K) {
    RowChunk<WF> ch;
    const int G = K / kGroup;
    if constexpr (WF == 1) {
        const uint8_t* c8 = reinterpret_cast<const uint8_t*>(wq) + (size_t)row * K + hg * 32;
        ch.c[0] = ld_stream_u32x4(c8);
        ch.c[1] = ld_stream_u32x4(c8 + 16);
        ch.s = ws[(size_t)row * G + (hg >> 1)];
        ch.b = 0;
    } else if constexpr (WF == 2) {
        ch.c[0] = ld_stream_u32x4(wq + (size_t)row * (K / 8) + hg * 4);
        ch.s = *reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(ws) + (size_t)row * (K / 16) +
                                                  2 * hg);
        ch.b = 0;
    } else {
        ch.c[0] = ld_stream_u32x4(wq + (size_t)row * (K / 8) + hg * 4);
        ch.s = ws[(size_t)row * G + (hg >> 1)];
        ch.b = wb[(size_t)row * G + (hg >> 1)];
    }
    return ch;
}

// Codec chunk dot product against the 32 raw activations xw (fp16 pairs in
// natural order): FP8 scale * sum, NVFP4 e4m3(block) * sum per block of 16
// (the global scale is applied by the caller).
template <int WF>
__device__ __forceinline__ float codec_chunk_dot(const RowChunk<WF>& ch, const u32x4 (&xw)[4]) {
    if constexpr (WF == 1) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {  // code word i: codes 4i .. 4i+3
            const uint32_t cwd = ch.c[i >> 2][i & 3];
            const u32x4 xq = xw[i >> 1];
            d0 = dot2(as_f16x2(xq[2 * (i & 1)]), e4m3x2_to_f16x2<false>(cwd), d0);
            d1 = dot2(as_f16x2(xq[2 * (i & 1) + 1]), e4m3x2_to_f16x2<true>(cwd), d1);
        }
        return h2f(ch.s) * (d0 + d1);
    } else {
        float d[2] = {0.f, 0.f};  // blocks 2c and 2c + 1 (words 0-1 and 2-3)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const u32x4 xq = xw[w];
            const uint32_t cwd = ch.c[0][w];
            float e = d[w >> 1];
            e = dot2(as_f16x2(xq.x), e2m1x2_to_f16x2<0>(cwd), e);
            e = dot2(as_f16x2(xq.y), e2m1x2_to_f16x2<1>(cwd), e);
            e = dot2(as_f16x2(xq.z), e2m1x2_to_f16x2<2>(cwd), e);
            e = dot2(as_f16x2(xq.w), e2m1x2_to_f16x2<3>(cwd), e);
            d[w >> 1] = e;
        }
        return e4m3_to_f32<0>(ch.s) * d[0] + e4m3_to_f32<1>(ch.s) * d[1];
    }
}

// One wave's outputs of row r: column block `xblock` of the expert matrix
// (wq, ws, wb; WF as above, gscale the NVFP4 global scale) applied to the
// activations xr.  BF16: activations, scales, biases and outputs are bf16
// patterns (codes enter v_dot2_f32_bf16 exactly, as in the bf16 GEMV).
template <int TPR, int V, int R, int MODE, bool BF16 = false, int WF = 0>
__device__ __forceinline__ void rows_body(const u32x4 (&xr)[V][4], const uint32_t* __restrict__ wq,
                                          const uint16_t* __restrict__ ws, const uint16_t* __restrict__ wb,
                                          float gscale, uint16_t* __restrict__ Y, int r, int xblock, int K,
                                          int N, int lane) {
    static_assert(WF == 0 || !BF16, "codec rows: fp16 activations");
    constexpr int TEAMS = 64 / TPR;
    constexpr int OUT = (MODE == 0) ? R / 2 : R;  // outputs per team
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int Nout = (MODE == 0) ? N / 2 : N;
    const int n0 = (xblock * TEAMS + team) * OUT;

    RowChunk<WF> chk[R][V];
#pragma unroll
    for (int q = 0; q < R; ++q) {
        const int nn = min(n0 + q % OUT, Nout - 1);
        const int row = nn + ((MODE == 0 && q >= OUT) ? Nout : 0);
#pragma unroll
        for (int v = 0; v < V; ++v) chk[q][v] = row_chunk_load<WF>(wq, ws, wb, row, lr + v * TPR, K);
    }
    (void)G;
    (void)wpr;
    __builtin_amdgcn_sched_barrier(0);
    float acc[R];
    if constexpr (WF != 0) {
#pragma unroll
        for (int q = 0; q < R; ++q) {
            acc[q] = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) acc[q] += codec_chunk_dot<WF>(chk[q][v], xr[v]);
        }
    } else if constexpr (BF16) {
        XPairsBf xp[V][4];
        float xs[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            xs[v] = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                xp[v][w] = make_xpairs_bf(xr[v][w]);
                xs[v] += xsum_bf(xp[v][w]);
            }
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {
            acc[q] = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
                const u32x4 cwv = chk[q][v].c[0];
                dot_word_bf(cwv.x, xp[v][0], d0, d1, d2, d3);
                dot_word_bf(cwv.y, xp[v][1], d0, d1, d2, d3);
                dot_word_bf(cwv.z, xp[v][2], d0, d1, d2, d3);
                dot_word_bf(cwv.w, xp[v][3], d0, d1, d2, d3);
                const float d = (d0 + d2) + (d1 + d3);
                acc[q] += bf2f(chk[q][v].s) * (d - 128.0f * xs[v]) + bf2f(chk[q][v].b) * xs[v];
            }
        }
    } else {
        XPairs xp[V][4];
        float xc[V], xs[V];
#pragma unroll
        for (int v = 0; v < V; ++v) {
            xc[v] = 0.f;
            xs[v] = 0.f;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                xp[v][w] = make_xpairs(xr[v][w]);
                float c_, s_;
                xpairs_consts(xp[v][w], c_, s_);
                xc[v] += c_;
                xs[v] += s_;
            }
        }
#pragma unroll
        for (int q = 0; q < R; ++q) {
            acc[q] = 0.f;
#pragma unroll
            for (int v = 0; v < V; ++v) {
                float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
                const u32x4 cwv = chk[q][v].c[0];
                dot_word(cwv.x, xp[v][0], d0, d1, d2, d3);
                dot_word(cwv.y, xp[v][1], d0, d1, d2, d3);
                dot_word(cwv.z, xp[v][2], d0, d1, d2, d3);
                dot_word(cwv.w, xp[v][3], d0, d1, d2, d3);
                acc[q] += h2f(chk[q][v].s) * (dot_sum(d0, d1, d2, d3) - xc[v]) + h2f(chk[q][v].b) * xs[v];
            }
        }
    }
    auto out16 = [](float v) -> uint16_t {
        if constexpr (BF16) return f2bf(v);
        else return f2h(v);
    };
    int sel;
    float tot = reduce_rows<TPR, R>(acc, lr, sel);
    if constexpr (WF == 2) tot *= gscale;  // both rows of a gate/up pair come from one expert
    const bool writer = (lr & (TPR / R - 1)) == 0;
    if constexpr (MODE == 0) {
        const float up = __shfl_xor(tot, TPR / 2, 64);  // row sel + R/2 of the same team
        if (writer && sel < OUT && n0 + sel < Nout)
            Y[(size_t)r * Nout + n0 + sel] = BF16 ? f2bf(silu(tot) * up) : mul_to_f16(silu(tot), up);
    } else {
        if (writer && n0 + sel < Nout) Y[(size_t)r * Nout + n0 + sel] = out16(tot);
    }
}

// Expert e's matrix within stacked experts of weight format WF (pointers
// as rows_body takes them).
template <int WF>
__device__ __forceinline__ void expert_ptrs(const uint32_t* qw, const uint16_t* sc, const uint16_t* bi,
                                            int e, int N, int K, const uint32_t*& wq, const uint16_t*& ws,
                                            const uint16_t*& wb) {
    const size_t n = (size_t)e * N;
    if constexpr (WF == 1) {
        wq = reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(qw) + n * K);
        ws = sc + n * (K / kGroup);
        wb = nullptr;
    } else if constexpr (WF == 2) {
        wq = qw + n * (K / 8);
        ws = reinterpret_cast<const uint16_t*>(reinterpret_cast<const uint8_t*>(sc) + n * (K / 16));
        wb = nullptr;
    } else {
        wq = qw + n * (K / 8);
        ws = sc + n * (K / kGroup);
        wb = bi + n * (K / kGroup);
    }
}

template <int TPR, int V, int R, int MODE, int WF = 0>
__global__ void __launch_bounds__(64)
moe_rows_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                const uint16_t* __restrict__ bi, const uint32_t* __restrict__ sqw,
                const uint16_t* __restrict__ ssc, const uint16_t* __restrict__ sbi,
                const float* __restrict__ gscales, float sgscale,
                const uint16_t* __restrict__ X, const int2* __restrict__ row_info,
                uint16_t* __restrict__ Y, int K, int N, int E, int T, int topk) {
    const int lane = threadIdx.x;
    const int r = blockIdx.y;
    const int routed = T * topk;
    const uint32_t* wq = sqw;
    const uint16_t* ws = ssc;
    const uint16_t* wb = sbi;
    float gscale = sgscale;
    int xrow;
    if (r < routed) {
        const int2 info = row_info[r];
        // Clamped so that a corrupted dispatch can never index out of bounds.
        const int e = min(max(info.x, 0), E - 1);
        expert_ptrs<WF>(qw, sc, bi, e, N, K, wq, ws, wb);
        if constexpr (WF == 2) gscale = gscales[e];
        xrow = (MODE == 0) ? min(max(info.y, 0), T - 1) : r;
    } else {
        xrow = (MODE == 0) ? r - routed : r;
    }
    u32x4 xr[V][4];
    rows_load_x<TPR, V>(X, xrow, K, lane % TPR, xr);
    rows_body<TPR, V, R, MODE, false, WF>(xr, wq, ws, wb, gscale, Y, r, blockIdx.x, K, N, lane);
}

// Decode gate/up projection fused with the token's routing: block (x, r)
// holds four waves, wave w computing column block 4x + w of row r (the
// rows of moe_rows_kernel's MODE 0, in assignment order: r = t*topk + j is
// the j-th expert chosen by token t, rows T*topk + t the shared expert).
// A routed block first sums the router partials of its token (the same
// fixed order as the dispatch-side router, so the choice is identical),
// takes the top-k (all four waves for E <= 256, else wave 0) and then
// reads only the j-th chosen expert's weights; its activation loads are
// issued before the routing.  Blocks with x = 0 also write the token's ids,
// gates, logits and the (expert, row) of their assignment for the down
// projection.
template <int TPR, int V, int R, int EPL, bool BF16, int WF = 0>
__global__ void __launch_bounds__(256)
moe_decode_gate_up_kernel(const float* __restrict__ partials, const float* __restrict__ bias,
                          const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                          const uint16_t* __restrict__ bi, const uint32_t* __restrict__ sqw,
                          const uint16_t* __restrict__ ssc, const uint16_t* __restrict__ sbi,
                          const float* __restrict__ gscales, float sgscale,
                          const uint16_t* __restrict__ X, uint16_t* __restrict__ Y, int K, int N,
                          int E, int T, int topk, int* __restrict__ ids, float* __restrict__ gates,
                          float* __restrict__ logits_out, int2* __restrict__ assign_info) {
    __shared__ float s_lg[64 * EPL];
    __shared__ int s_sel[QL_MAX_TOPK_DEV];
    __shared__ float s_gate[QL_MAX_TOPK_DEV];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int r = blockIdx.y;
    const int routed = T * topk;
    const int t = (r < routed) ? r / topk : r - routed;
    u32x4 xr[V][4];
    rows_load_x<TPR, V>(X, t, K, lane % TPR, xr);
    const uint32_t* wq = sqw;
    const uint16_t* ws = ssc;
    const uint16_t* wb = sbi;
    float gscale = sgscale;
    if (r < routed) {  // uniform over the block
        const int j = r - t * topk;
        for (int e = threadIdx.x; e < E; e += blockDim.x) {
            float part[kRouterSmallParts];
#pragma unroll
            for (int p = 0; p < kRouterSmallParts; ++p)
                part[p] = partials[((size_t)t * kRouterSmallParts + p) * E + e];
            float sum = 0.f;
#pragma unroll
            for (int p = 0; p < kRouterSmallParts; ++p) sum += part[p];
            if (bias) sum += bias[e];
            s_lg[e] = sum;
        }
        __syncthreads();
        if constexpr (EPL <= 4) {
            topk_block_small(s_lg, E, topk, s_sel, s_gate);  // all four waves; ends with a barrier
        } else {
            if (wave == 0) topk_one_token<EPL, 1>(s_lg, nullptr, s_lg, 0, E, topk, s_sel, s_gate);
            __syncthreads();
        }
        const int e = min(max(s_sel[j], 0), E - 1);
        expert_ptrs<WF>(qw, sc, bi, e, N, K, wq, ws, wb);
        if constexpr (WF == 2) gscale = gscales[e];
        if (blockIdx.x == 0) {
            if (threadIdx.x == 0) {
                ids[r] = e;
                gates[r] = s_gate[j];
                assign_info[r] = make_int2(e, r);
            }
            if (j == 0)
                for (int i = threadIdx.x; i < E; i += blockDim.x) logits_out[(size_t)t * E + i] = s_lg[i];
        }
    }
    rows_body<TPR, V, R, 0, BF16, WF>(xr, wq, ws, wb, gscale, Y, r, blockIdx.x * 4 + wave, K, N, lane);
}

// Decode down projection fused with the gate-weighted sum over the token's
// routed rows and its shared row.  A block of four waves owns TEAMS*R
// outputs of one token; the rows j = 0 .. J-1 (the shared row is j = topk)
// are dealt to the waves by j mod 4, so every SIMD of the CU works (one wave
// holding all rows left three idle and ran their work serially).  The
// (expert, row) of each assignment comes from assign_info.  The activation
// loads are issued first, then each wave's code loads; the activations are
// pre-paired into LDS while the codes are in flight.  Sums, in a fixed
// order: per lane over the wave's rows in ascending j, across the lanes of
// the row team, then the four wave sums in wave order.
// WF: weight format as in rows_body (codec rows keep the activation chunks
// raw in LDS; the NVFP4 global scale of each row joins its gate).
template <int TPR, int V, int R, int JC, bool BF16 = false, int WF = 0>
__global__ void __launch_bounds__(256)
moe_down_combine_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                        const uint16_t* __restrict__ bi, const uint32_t* __restrict__ sqw,
                        const uint16_t* __restrict__ ssc, const uint16_t* __restrict__ sbi,
                        const float* __restrict__ gscales, float sgscale,
                        const uint16_t* __restrict__ X, const float* __restrict__ gates,
                        const int2* __restrict__ assign_info, uint16_t* __restrict__ Y, int K,
                        int N, int E, int T, int topk, int has_shared) {
    static_assert(WF == 0 || !BF16, "codec rows: fp16 activations");
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_exp[QL_MAX_TOPK_DEV + 1];
    __shared__ int s_row[QL_MAX_TOPK_DEV + 1];
    __shared__ float s_gate[QL_MAX_TOPK_DEV + 1];
    constexpr int TEAMS = 64 / TPR;
    constexpr int NW = 4;  // waves per block
    __shared__ float s_red[NW][TEAMS * R];
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int CH = K / 32;  // 16-byte chunks of codes per row
    const int t = blockIdx.y;
    const int J = topk + has_shared;
    const int nrows = T * topk + (has_shared ? T : 0);
    XPairs* s_xp = reinterpret_cast<XPairs*>(smem);                   // [J][CH][4]
    float* s_c = reinterpret_cast<float*>(s_xp + (size_t)J * CH * 4);  // [J][CH]
    float* s_xs = s_c + J * CH;                                        // [J][CH]

    for (int j = threadIdx.x; j < J; j += blockDim.x) {
        if (j < topk) {
            const int2 info = assign_info[(size_t)t * topk + j];
            // Clamped so that a corrupted dispatch can never index out of bounds.
            s_exp[j] = min(max(info.x, 0), E - 1);
            s_row[j] = min(max(info.y, 0), nrows - 1);
            s_gate[j] = gates[(size_t)t * topk + j];
            if constexpr (WF == 2) s_gate[j] *= gscales[s_exp[j]];
        } else {
            s_exp[j] = -1;
            s_row[j] = T * topk + t;
            s_gate[j] = (WF == 2) ? sgscale : 1.0f;
        }
    }
    __syncthreads();

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int n0 = (blockIdx.x * TEAMS + team) * R;

    // Activation staging (whole block), loads of the first batch first.
    auto stage_load = [&](int idx0, u32x4 (&xw)[4]) {
        const int idx = min(idx0, J * CH - 1);
        const int j = idx / CH, c = idx % CH;
        const uint16_t* xrow = X + (size_t)s_row[j] * K + c * 32;
#pragma unroll
        for (int w = 0; w < 4; ++w) xw[w] = ld_u32x4(xrow + w * 8);
    };
    auto stage_store = [&](int idx, const u32x4 (&xw)[4]) {
        if (idx >= J * CH) return;
        const int j = idx / CH, c = idx % CH;
        float cc = 0.f, xx = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if constexpr (WF != 0) {
                s_xp[((size_t)j * CH + c) * 4 + w] = __builtin_bit_cast(XPairs, xw[w]);  // raw pairs
            } else if constexpr (BF16) {
                const XPairsBf xp = make_xpairs_bf(xw[w]);
                xx += xsum_bf(xp);
                s_xp[((size_t)j * CH + c) * 4 + w] = __builtin_bit_cast(XPairs, xp);
            } else {
                const XPairs xp = make_xpairs(xw[w]);
                float c_, s_;
                xpairs_consts(xp, c_, s_);
                cc += c_;
                xx += s_;
                s_xp[((size_t)j * CH + c) * 4 + w] = xp;
            }
        }
        s_c[j * CH + c] = cc;
        s_xs[j * CH + c] = xx;
    };
    u32x4 xw0[4];
    stage_load(threadIdx.x, xw0);

    float acc[R];
#pragma unroll
    for (int q = 0; q < R; ++q) acc[q] = 0.f;

    // This wave's rows: j = wave, wave + 4, ..., JC of them per round.
    RowChunk<WF> chk[JC][R][V];
    auto load_round = [&](int j0) {
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
            const int j = j0 + NW * jj;
            if (j >= J) break;  // uniform across the wave
            const int e = s_exp[j];
            const uint32_t* wq = sqw;
            const uint16_t* ws = ssc;
            const uint16_t* wb = sbi;
            if (e >= 0) expert_ptrs<WF>(qw, sc, bi, e, N, K, wq, ws, wb);
#pragma unroll
            for (int q = 0; q < R; ++q) {
                const int row = min(n0 + q, N - 1);
#pragma unroll
                for (int v = 0; v < V; ++v) chk[jj][q][v] = row_chunk_load<WF>(wq, ws, wb, row, lr + v * TPR, K);
            }
        }
    };
    (void)G;
    (void)wpr;
    auto compute_round = [&](int j0) {
#pragma unroll
        for (int jj = 0; jj < JC; ++jj) {
            const int j = j0 + NW * jj;
            if (j >= J) break;  // uniform across the wave
            const float g = s_gate[j];
#pragma unroll
            for (int v = 0; v < V; ++v) {
                const int hg = lr + v * TPR;
                XPairs xp[4];
#pragma unroll
                for (int w = 0; w < 4; ++w) xp[w] = s_xp[((size_t)j * CH + hg) * 4 + w];
                if constexpr (WF != 0) {
                    const u32x4 xw[4] = {__builtin_bit_cast(u32x4, xp[0]), __builtin_bit_cast(u32x4, xp[1]),
                                         __builtin_bit_cast(u32x4, xp[2]), __builtin_bit_cast(u32x4, xp[3])};
#pragma unroll
                    for (int q = 0; q < R; ++q) acc[q] += g * codec_chunk_dot<WF>(chk[jj][q][v], xw);
                    continue;
                }
                const float xc = s_c[j * CH + hg], xs = s_xs[j * CH + hg];
#pragma unroll
                for (int q = 0; q < R; ++q) {
                    float d0 = 0.f, d1 = 0.f, d2 = 0.f, d3 = 0.f;
                    const u32x4 cwv = chk[jj][q][v].c[0];
                    if constexpr (BF16) {
                        dot_word_bf(cwv.x, __builtin_bit_cast(XPairsBf, xp[0]), d0, d1, d2, d3);
                        dot_word_bf(cwv.y, __builtin_bit_cast(XPairsBf, xp[1]), d0, d1, d2, d3);
                        dot_word_bf(cwv.z, __builtin_bit_cast(XPairsBf, xp[2]), d0, d1, d2, d3);
                        dot_word_bf(cwv.w, __builtin_bit_cast(XPairsBf, xp[3]), d0, d1, d2, d3);
                        acc[q] += g * (bf2f(chk[jj][q][v].s) * (((d0 + d2) + (d1 + d3)) - 128.0f * xs) +
                                       bf2f(chk[jj][q][v].b) * xs);
                    } else {
                        dot_word(cwv.x, xp[0], d0, d1, d2, d3);
                        dot_word(cwv.y, xp[1], d0, d1, d2, d3);
                        dot_word(cwv.z, xp[2], d0, d1, d2, d3);
                        dot_word(cwv.w, xp[3], d0, d1, d2, d3);
                        acc[q] += g * (h2f(chk[jj][q][v].s) * (dot_sum(d0, d1, d2, d3) - xc) +
                                       h2f(chk[jj][q][v].b) * xs);
                    }
                }
            }
        }
    };
    load_round(wave);  // no loads for a wave without rows (wave >= J)
    stage_store(threadIdx.x, xw0);
    for (int idx = threadIdx.x + 256; idx < J * CH; idx += 256) {
        u32x4 xw[4];
        stage_load(idx, xw);
        stage_store(idx, xw);
    }
    __syncthreads();
    compute_round(wave);
    for (int j0 = wave + NW * JC; j0 < J; j0 += NW * JC) {
        load_round(j0);
        compute_round(j0);
    }
    int sel;
    const float tot = reduce_rows<TPR, R>(acc, lr, sel);
    if ((lr & (TPR / R - 1)) == 0) s_red[wave][team * R + sel] = tot;
    __syncthreads();
    if (threadIdx.x < TEAMS * R) {
        const int n = blockIdx.x * TEAMS * R + threadIdx.x;
        const float y = ((s_red[0][threadIdx.x] + s_red[1][threadIdx.x]) + s_red[2][threadIdx.x]) +
                        s_red[3][threadIdx.x];
        if (n < N) Y[(size_t)t * N + n] = BF16 ? f2bf(y) : f2h(y);
    }
}

constexpr int kMaxGemvBlocks = 2048;

template <int TPR, int GPL, int UNROLL>
int launch_gemv_t(const GemvArgs& a, hipStream_t st) {
    constexpr int TEAMS = 64 / TPR;
    const long rows_per_block_iter = 4L * TEAMS * UNROLL;
    const long work = (a.N + rows_per_block_iter - 1) / rows_per_block_iter;
    const long iters = (work + kMaxGemvBlocks - 1) / kMaxGemvBlocks;
    const int blocks = (int)((work + iters - 1) / iters);
    hipLaunchKernelGGL((gemv_w4_kernel<TPR, GPL, UNROLL>), dim3(blocks), dim3(256), 0, st,
                       a.qweight, a.scales, a.biases, a.x, a.y, a.K, a.N);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

// Largest power of two (at most 64) dividing G.
inline int pow2_divisor(int G) {
    int t = 1;
    while (t < 64 && G % (2 * t) == 0) t *= 2;
    return t;
}

template <int TPR, int V, bool BF16 = false, int WF = 0>
void launch_down_combine_t(const GroupedArgs& a, const int2* assign_info, hipStream_t st) {
    constexpr int TEAMS = 64 / TPR;
    constexpr int R = (TPR < 2) ? TPR : 2;
    const int has_shared = a.sqw != nullptr;
    const int J = a.topk + has_shared;
    const size_t smem = (size_t)J * (a.K / 32) * (4 * sizeof(XPairs) + 2 * sizeof(float));
    dim3 grid((a.N + TEAMS * R - 1) / (TEAMS * R), a.T);
    // four waves; each takes the rows j = wave, wave + 4, ... (3 per round)
    hipLaunchKernelGGL((moe_down_combine_kernel<TPR, V, R, 3, BF16, WF>), grid, dim3(256), smem, st, a.qw,
                       a.sc, a.bi, a.sqw, a.ssc, a.sbi, a.gscales, a.sgscale, a.X, a.gates, assign_info, a.Y,
                       a.K, a.N, a.E, a.T, a.topk, has_shared);
}

template <int TPR, int V>
void launch_down_combine_wf(const GroupedArgs& a, const int2* assign_info, hipStream_t st) {
    if (a.wf == 1) launch_down_combine_t<TPR, V, false, 1>(a, assign_info, st);
    else if (a.wf == 2) launch_down_combine_t<TPR, V, false, 2>(a, assign_info, st);
    else if (a.bf16) launch_down_combine_t<TPR, V, true>(a, assign_info, st);
    else launch_down_combine_t<TPR, V, false>(a, assign_info, st);
}

template <int TPR, int V>
int launch_rows_t(const GroupedArgs& a, hipStream_t st) {
    constexpr int TEAMS = 64 / TPR;
    const MoeWorkspace L = moe_workspace_layout(a.T, a.E, a.topk);
    const int has_shared = a.sqw != nullptr;
    if (a.op == QL_OP_DOWN_COMBINE) {
        launch_down_combine_wf<TPR, V>(a, reinterpret_cast<const int2*>(a.ws + L.assign_info), st);
    } else {
        constexpr int R = (TPR < 8) ? TPR : 8;
        const int rows = a.T * a.topk + (has_shared ? a.T : 0);
        const int2* rinfo = reinterpret_cast<const int2*>(a.ws + L.row_info);
        auto go = [&](auto mode, auto wf) {
            constexpr int MODE = decltype(mode)::value, WF = decltype(wf)::value;
            const int outs = (MODE == 0) ? a.N / 2 : a.N;
            const int per = (MODE == 0) ? TEAMS * (R / 2) : TEAMS * R;
            dim3 grid((outs + per - 1) / per, rows);
            hipLaunchKernelGGL((moe_rows_kernel<TPR, V, R, MODE, WF>), grid, dim3(64), 0, st, a.qw, a.sc,
                               a.bi, a.sqw, a.ssc, a.sbi, a.gscales, a.sgscale, a.X, rinfo, a.Y, a.K, a.N,
                               a.E, a.T, a.topk);
        };
        static_assert(R % 2 == 0, "gate/up pairing needs an even row count");
        using M0 = std::integral_constant<int, 0>;
        using M1 = std::integral_constant<int, 1>;
        using W0 = std::integral_constant<int, 0>;
        using W1 = std::integral_constant<int, 1>;
        using W2 = std::integral_constant<int, 2>;
        const bool gu = a.op == QL_OP_GATE_UP_SILU;
        if (a.wf == 1) gu ? go(M0{}, W1{}) : go(M1{}, W1{});
        else if (a.wf == 2) gu ? go(M0{}, W2{}) : go(M1{}, W2{});
        else gu ? go(M0{}, W0{}) : go(M1{}, W0{});
    }
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

}  // namespace

template <int TPR, int V, int R, int PRO, int EPI>
int launch_chunked_t(const GemvArgs& a, hipStream_t st) {
    constexpr int ROWS_PER_BLOCK = 4 * (64 / TPR) * R;
    static_assert(ROWS_PER_BLOCK >= 8, "at most ceil(N / 8) argmax block keys");
    const int blocks = (a.N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    hipLaunchKernelGGL((gemv_w4_chunked_kernel<TPR, V, R, PRO, EPI>), dim3(blocks), dim3(256), 0, st,
                       a.qweight, a.scales, a.biases, a.x, a.y, a.K, a.N, a.gamma, a.eps, a.partials);
    if (hipGetLastError() != hipSuccess) return QL_ERR_HIP;
    if constexpr (EPI == GV_ARGMAX) {
        hipLaunchKernelGGL(argmax_finish_kernel, dim3(1), dim3(1024), 0, st, a.partials, blocks, a.N, a.token);
        if (hipGetLastError() != hipSuccess) return QL_ERR_HIP;
    }
    return QL_OK;
}

// Rows per team of the chunked GEMV: 8 rows in flight per wave for large N;
// fewer for small N so that the grid still spreads over every CU.
#ifndef QL_GEMV_ROWS
#define QL_GEMV_ROWS 8
#endif
constexpr int kGemvRows = QL_GEMV_ROWS;
constexpr int kGemvMinBlocks = 1024;

template <int TPR, int V, int PRO, int EPI>
int launch_chunked_r(const GemvArgs& a, hipStream_t st) {
    constexpr int R = (kGemvRows < TPR) ? kGemvRows : TPR;
    const long blocks_big = (a.N + 4L * (64 / TPR) * R - 1) / (4L * (64 / TPR) * R);
    // The RMSNorm prologue is the same work in every wave, so that variant
    // keeps the full R rows per lane (measured at K 2048, N 8192: 5.2 us
    // with 2 rows, 3.8 us with 8, as fast as the plain GEMV).
    if (PRO == GV_RMSNORM || blocks_big >= kGemvMinBlocks || R <= 2)
        return launch_chunked_t<TPR, V, R, PRO, EPI>(a, st);
    return launch_chunked_t<TPR, V, 2, PRO, EPI>(a, st);
}

// Chunked kernel: K/32 chunks per row spread over TPR lanes, V per lane.
// QL_ERR_UNSUPPORTED_SHAPE for other K.
template <int PRO, int EPI>
int launch_chunked(const GemvArgs& a, hipStream_t st) {
    switch (a.K) {
        case 256: return launch_chunked_r<8, 1, PRO, EPI>(a, st);
        case 512: return launch_chunked_r<16, 1, PRO, EPI>(a, st);
        case 1024: return launch_chunked_r<32, 1, PRO, EPI>(a, st);
        case 2048: return launch_chunked_r<64, 1, PRO, EPI>(a, st);
        case 4096: return launch_chunked_r<64, 2, PRO, EPI>(a, st);
        case 8192: return launch_chunked_t<64, 4, 4, PRO, EPI>(a, st);
        case 16384: return launch_chunked_t<64, 8, 2, PRO, EPI>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

bool gemv_fused_supported(int K) {
    switch (K) {
        case 256: case 512: case 1024: case 2048: case 4096: case 8192: case 16384: return true;
        default: return false;
    }
}

template <int TPR, int V, int R>
int launch_bf16_t(const GemvArgs& a, hipStream_t st) {
    constexpr int ROWS_PER_BLOCK = 4 * (64 / TPR) * R;
    const int blocks = (a.N + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK;
    hipLaunchKernelGGL((gemv_w4_bf16_kernel<TPR, V, R>), dim3(blocks), dim3(256), 0, st, a.qweight,
                       a.scales, a.biases, a.x, a.y, a.K, a.N);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

template <int TPR, int V>
int launch_bf16_r(const GemvArgs& a, hipStream_t st) {
    constexpr int R = (kGemvRows < TPR) ? kGemvRows : TPR;
    const long blocks_big = (a.N + 4L * (64 / TPR) * R - 1) / (4L * (64 / TPR) * R);
    if (blocks_big >= kGemvMinBlocks || R <= 2) return launch_bf16_t<TPR, V, R>(a, st);
    return launch_bf16_t<TPR, V, 2>(a, st);
}

int launch_gemv_bf16(const GemvArgs& a, hipStream_t st) {
    switch (a.K) {
        case 256: return launch_bf16_r<8, 1>(a, st);
        case 512: return launch_bf16_r<16, 1>(a, st);
        case 1024: return launch_bf16_r<32, 1>(a, st);
        case 2048: return launch_bf16_r<64, 1>(a, st);
        case 4096: return launch_bf16_r<64, 2>(a, st);
        case 8192: return launch_bf16_t<64, 4, 4>(a, st);
        case 16384: return launch_bf16_t<64, 8, 2>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

// FALLBACK: the matrix's own launch drops to two rows per wave when it has
// few blocks (launch_chunked_r); K = 8192 and 16384 keep fixed rows.
template <int TPR, int V, int R, bool FALLBACK = true>
int launch_multi_t(const GemvMultiArgs& a, hipStream_t st) {
    GemvMulti m{};
    m.count = a.count;
    long blocks = 0;
    for (int i = 0; i < a.count; ++i) {
        m.qw[i] = a.qweight[i];
        m.sc[i] = a.scales[i];
        m.bi[i] = a.biases[i];
        m.y[i] = a.y[i];
        m.N[i] = a.N[i];
        // The rows per wave of the matrix's own launch (launch_chunked_r).
        const long big = (a.N[i] + 4L * (64 / TPR) * R - 1) / (4L * (64 / TPR) * R);
        m.small_r[i] = (FALLBACK && R > 2 && big < kGemvMinBlocks) ? 1 : 0;
        const int rpb = 4 * (64 / TPR) * (m.small_r[i] ? 2 : R);
        m.block0[i] = (int)blocks;
        blocks += (a.N[i] + rpb - 1) / rpb;
        if (blocks > 0x7fffffffL) return QL_ERR_UNSUPPORTED_SHAPE;
    }
    m.block0[a.count] = (int)blocks;
    if (blocks == 0) return QL_OK;
    hipLaunchKernelGGL((gemv_w4_multi_kernel<TPR, V, R>), dim3((unsigned)blocks), dim3(256), 0, st, m, a.x, a.K);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

int launch_gemv_multi(const GemvMultiArgs& a, hipStream_t st) {
    constexpr int R = kGemvRows;
    switch (a.K) {
        case 256: return launch_multi_t<8, 1, (R < 8 ? R : 8)>(a, st);
        case 512: return launch_multi_t<16, 1, (R < 16 ? R : 16)>(a, st);
        case 1024: return launch_multi_t<32, 1, R>(a, st);
        case 2048: return launch_multi_t<64, 1, R>(a, st);
        case 4096: return launch_multi_t<64, 2, R>(a, st);
        case 8192: return launch_multi_t<64, 4, 4, false>(a, st);  // the fixed rows of launch_chunked
        case 16384: return launch_multi_t<64, 8, 2, false>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

int launch_gemv_rmsnorm(const GemvArgs& a, hipStream_t st) { return launch_chunked<GV_RMSNORM, GV_STORE>(a, st); }

int launch_gemv_argmax(const GemvArgs& a, hipStream_t st) { return launch_chunked<GV_PLAIN, GV_ARGMAX>(a, st); }

int launch_embed(const GemvArgs& a, hipStream_t st) {
    const int words = a.K / 8;
    hipLaunchKernelGGL(embed_w4_kernel, dim3((words + 255) / 256), dim3(256), 0, st, a.qweight, a.scales,
                       a.biases, a.token, a.y, a.K, a.N);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

int launch_gemv(const GemvArgs& a, hipStream_t st) {
    if (gemv_fused_supported(a.K)) return launch_chunked<GV_PLAIN, GV_STORE>(a, st);
    const int G = a.K / kGroup;
    switch (G) {
        case 8: return launch_gemv_t<8, 1, 2>(a, st);
        case 16: return launch_gemv_t<16, 1, 2>(a, st);
        case 32: return launch_gemv_t<32, 1, 2>(a, st);
        case 64: return launch_gemv_t<64, 1, 2>(a, st);
        case 128: return launch_gemv_t<64, 2, 2>(a, st);
        case 256: return launch_gemv_t<64, 4, 1>(a, st);
        default: break;
    }
    switch (pow2_divisor(G)) {
        case 1: return launch_gemv_t<1, 0, 1>(a, st);
        case 2: return launch_gemv_t<2, 0, 1>(a, st);
        case 4: return launch_gemv_t<4, 0, 1>(a, st);
        case 8: return launch_gemv_t<8, 0, 1>(a, st);
        case 16: return launch_gemv_t<16, 0, 1>(a, st);
        case 32: return launch_gemv_t<32, 0, 1>(a, st);
        default: return launch_gemv_t<64, 0, 1>(a, st);
    }
}

}  // namespace ql

namespace ql {

bool moe_rows_supported(int K) {
    // K/32 chunks of codes spread over TPR <= 64 lanes, V = 1, 2, 4 or 8 per lane.
    switch (K) {
        case 64: case 128: case 256: case 512: case 1024: case 2048: case 4096: case 8192:
        case 16384: return true;
        default: return false;
    }
}

namespace {

template <int TPR, int V, int EPL, bool BF16, int WF = 0>
void launch_decode_gate_up_t(const DecodeArgs& a, const DecodeLayout& L, hipStream_t st) {
    constexpr int TEAMS = 64 / TPR;
    // Rows per team: 8, or 4 where each row's decode costs more (bf16
    // activations, FP8 codes), which spreads the launch over twice the
    // workgroups (measured faster for those two, no change for w4 fp16).
    constexpr int RMAX = (BF16 || WF == 1) ? 4 : 8;
    constexpr int R = (TPR < RMAX) ? TPR : RMAX;
    static_assert(R % 2 == 0, "gate/up pairing needs an even row count");
    constexpr int COLS = 4 * TEAMS * (R / 2);  // act columns per block
    const int has_shared = a.sgu_qw != nullptr;
    const int rows = a.T * a.topk + (has_shared ? a.T : 0);
    dim3 grid((a.I + COLS - 1) / COLS, rows);
    hipLaunchKernelGGL((moe_decode_gate_up_kernel<TPR, V, R, EPL, BF16, WF>), grid, dim3(256), 0, st,
                       reinterpret_cast<const float*>(a.ws + L.partials), a.bias, a.gu_qw, a.gu_sc,
                       a.gu_bi, a.sgu_qw, a.sgu_sc, a.sgu_bi, a.gu_gscales, a.sgu_gscale, a.H,
                       reinterpret_cast<uint16_t*>(a.ws + L.act), a.D, 2 * a.I, a.E, a.T, a.topk, a.ids,
                       a.gates, reinterpret_cast<float*>(a.ws + L.logits),
                       reinterpret_cast<int2*>(a.ws + L.assign_info));
}

template <int TPR, int V>
void launch_decode_gate_up_v(const DecodeArgs& a, const DecodeLayout& L, hipStream_t st) {
    if (a.wf == 1) {
        if (a.E <= 256) launch_decode_gate_up_t<TPR, V, 4, false, 1>(a, L, st);
        else launch_decode_gate_up_t<TPR, V, 16, false, 1>(a, L, st);
    } else if (a.wf == 2) {
        if (a.E <= 256) launch_decode_gate_up_t<TPR, V, 4, false, 2>(a, L, st);
        else launch_decode_gate_up_t<TPR, V, 16, false, 2>(a, L, st);
    } else if (a.bf16) {
        if (a.E <= 256) launch_decode_gate_up_t<TPR, V, 4, true>(a, L, st);
        else launch_decode_gate_up_t<TPR, V, 16, true>(a, L, st);
    } else {
        if (a.E <= 256) launch_decode_gate_up_t<TPR, V, 4, false>(a, L, st);
        else launch_decode_gate_up_t<TPR, V, 16, false>(a, L, st);
    }
}

template <int TPR, int V>
void launch_decode_down_v(const DecodeArgs& a, const DecodeLayout& L, hipStream_t st) {
    GroupedArgs g{a.dn_qw, a.dn_sc, a.dn_bi, a.sdn_qw, a.sdn_sc, a.sdn_bi,
                  reinterpret_cast<const uint16_t*>(a.ws + L.act), nullptr, nullptr, a.gates,
                  nullptr, a.ws, a.out, a.I, a.D, a.E, a.T, a.topk, QL_OP_DOWN_COMBINE};
    g.bf16 = a.bf16;
    g.wf = a.wf;
    g.gscales = a.dn_gscales;
    g.sgscale = a.sdn_gscale;
    launch_down_combine_wf<TPR, V>(g, reinterpret_cast<const int2*>(a.ws + L.assign_info), st);
}

}  // namespace

size_t align_up256(size_t v) { return (v + 255) & ~(size_t)255; }

DecodeLayout moe_decode_layout(int T, int E, int topk, int I) {
    DecodeLayout L;
    size_t off = 0;
    L.partials = off;
    off = align_up256(off + (size_t)T * kRouterSmallParts * E * sizeof(float));
    L.logits = off;
    off = align_up256(off + (size_t)T * E * sizeof(float));
    L.assign_info = off;
    off = align_up256(off + (size_t)T * topk * 2 * sizeof(int));
    L.act = off;
    off = align_up256(off + (size_t)T * (topk + 1) * I * sizeof(uint16_t));
    L.total = off;
    return L;
}

int launch_moe_decode(const DecodeArgs& a, hipStream_t st) {
    const DecodeLayout L = moe_decode_layout(a.T, a.E, a.topk, a.I);
    int rc = launch_router_partials_small(a.H, a.Wr, reinterpret_cast<float*>(a.ws + L.partials), a.T,
                                          a.D, a.E, st, a.bf16);
    if (rc != QL_OK) return rc;
    switch (a.D) {
        case 64: launch_decode_gate_up_v<2, 1>(a, L, st); break;
        case 128: launch_decode_gate_up_v<4, 1>(a, L, st); break;
        case 256: launch_decode_gate_up_v<8, 1>(a, L, st); break;
        case 512: launch_decode_gate_up_v<16, 1>(a, L, st); break;
        case 1024: launch_decode_gate_up_v<32, 1>(a, L, st); break;
        case 2048: launch_decode_gate_up_v<64, 1>(a, L, st); break;
        case 4096: launch_decode_gate_up_v<64, 2>(a, L, st); break;
        case 8192: launch_decode_gate_up_v<64, 4>(a, L, st); break;
        case 16384: launch_decode_gate_up_v<64, 8>(a, L, st); break;
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
    if (hipGetLastError() != hipSuccess) return QL_ERR_HIP;
    switch (a.I) {
        case 64: launch_decode_down_v<2, 1>(a, L, st); break;
        case 128: launch_decode_down_v<4, 1>(a, L, st); break;
        case 256: launch_decode_down_v<8, 1>(a, L, st); break;
        case 512: launch_decode_down_v<16, 1>(a, L, st); break;
        case 1024: launch_decode_down_v<32, 1>(a, L, st); break;
        case 2048: launch_decode_down_v<64, 1>(a, L, st); break;
        case 4096: launch_decode_down_v<64, 2>(a, L, st); break;
        case 8192: launch_decode_down_v<64, 4>(a, L, st); break;
        case 16384: launch_decode_down_v<64, 8>(a, L, st); break;
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

int launch_moe_rows(const GroupedArgs& a, hipStream_t st) {
    switch (a.K) {
        case 64: return launch_rows_t<2, 1>(a, st);
        case 128: return launch_rows_t<4, 1>(a, st);
        case 256: return launch_rows_t<8, 1>(a, st);
        case 512: return launch_rows_t<16, 1>(a, st);
        case 1024: return launch_rows_t<32, 1>(a, st);
        case 2048: return launch_rows_t<64, 1>(a, st);
        case 4096: return launch_rows_t<64, 2>(a, st);
        case 8192: return launch_rows_t<64, 4>(a, st);
        case 16384: return launch_rows_t<64, 8>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

}  // namespace ql
