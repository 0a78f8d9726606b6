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
#include "ql_device.h"
#include "ql_internal.h"

namespace ql {

namespace {

// Team reduction over TPR consecutive lanes.
template <int TPR>
__device__ __forceinline__ float team_sum(float v) {
#pragma unroll
    for (int off = TPR / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}

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
    return (d0 + d2) + (d1 + d3);
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
        xpairs_consts(xp[w], xw, cw, sw);
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
// Routed-expert rows (decode MoE).  Row r < T*topk is the assignment
// sorted_assign[r], multiplied by the expert e with offsets[e] <= r <
// offsets[e+1]; rows T*topk .. T*topk+T-1 are the tokens multiplied by the
// shared expert.
// ---------------------------------------------------------------------------
// Expert of routed row r from offsets staged in LDS (upper bound search).
__device__ __forceinline__ int expert_of_row(const int* s_off, int E, int r) {
    int lo = 0, hi = E;  // find largest e with s_off[e] <= r
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_off[mid] <= r) lo = mid; else hi = mid;
    }
    return lo;
}

__device__ __forceinline__ void stage_offsets(const int* __restrict__ offsets, int E, int* s_off) {
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_off[i] = offsets[i];
    __syncthreads();
}

// MODE 0: gate_up with SiLU(gate) * up   (output width N/2, x = X[token])
// MODE 1: down                            (output width N,   x = X[row])
template <int TPR, int GPL, int MODE>
__global__ void __launch_bounds__(256)
moe_rows_gemv_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                     const uint16_t* __restrict__ bi,
                     const uint32_t* __restrict__ sqw, const uint16_t* __restrict__ ssc,
                     const uint16_t* __restrict__ sbi,
                     const uint16_t* __restrict__ X, const int* __restrict__ offsets,
                     const int* __restrict__ sorted_assign, uint16_t* __restrict__ Y,
                     int K, int N, int E, int T, int topk) {
    __shared__ int s_off[QL_MAX_EXPERTS_DEV + 1];
    constexpr int TEAMS = 64 / TPR;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int wave = threadIdx.x / 64;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int r = blockIdx.y;
    const int routed = T * topk;

    stage_offsets(offsets, E, s_off);
    const uint32_t* wq;
    const uint16_t* ws;
    const uint16_t* wb;
    int xrow;
    if (r < routed) {
        const int e = expert_of_row(s_off, E, r);
        wq = qw + (size_t)e * N * wpr;
        ws = sc + (size_t)e * N * G;
        wb = bi + (size_t)e * N * G;
        // Clamped so that a corrupted dispatch can never index outside X.
        xrow = (MODE == 0) ? min(max(sorted_assign[r] / topk, 0), T - 1) : r;
    } else {
        wq = sqw;
        ws = ssc;
        wb = sbi;
        xrow = (MODE == 0) ? r - routed : r;
    }
    const int Nout = (MODE == 0) ? N / 2 : N;
    const int n = (blockIdx.x * (blockDim.x / 64) + wave) * TEAMS + team;
    const int nn = min(n, Nout - 1);

    // Issue the weight loads first: they do not depend on the activations.
    constexpr int NR = (MODE == 0) ? 2 : 1;
    u32x4 cw[NR][GPL][2];
    uint16_t s[NR][GPL], b[NR][GPL];
#pragma unroll
    for (int q = 0; q < NR; ++q) {
        const int row = nn + q * Nout;
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            const int g = lr + i * TPR;
            const uint32_t* p = wq + (size_t)row * wpr + g * 8;
            cw[q][i][0] = ld_stream_u32x4(p);
            cw[q][i][1] = ld_stream_u32x4(p + 4);
            s[q][i] = ws[(size_t)row * G + g];
            b[q][i] = wb[(size_t)row * G + g];
        }
    }
    const uint16_t* x = X + (size_t)xrow * K;
    float acc[NR];
#pragma unroll
    for (int q = 0; q < NR; ++q) acc[q] = 0.f;
#pragma unroll
    for (int i = 0; i < GPL; ++i) {
        XPairs xp[8];
        float c, xs;
        load_group_x(x, lr + i * TPR, xp, c, xs);
#pragma unroll
        for (int q = 0; q < NR; ++q) {
            const float d = group_dot(cw[q][i][0], cw[q][i][1], xp);
            acc[q] += h2f(s[q][i]) * (d - c) + h2f(b[q][i]) * xs;
        }
    }
#pragma unroll
    for (int q = 0; q < NR; ++q) acc[q] = team_sum<TPR>(acc[q]);
    if (lr == 0 && n < Nout) {
        const float v = (MODE == 0) ? silu(acc[0]) * acc[1] : acc[0];
        Y[(size_t)r * Nout + n] = f2h(v);
    }
}

// Decode down projection fused with the gate-weighted sum over the token's
// routed rows and the shared row.  One block column per token.  The rows'
// activations are pre-paired once per block into LDS.
template <int TPR, int GPL>
__global__ void __launch_bounds__(256)
moe_down_combine_kernel(const uint32_t* __restrict__ qw, const uint16_t* __restrict__ sc,
                        const uint16_t* __restrict__ bi,
                        const uint32_t* __restrict__ sqw, const uint16_t* __restrict__ ssc,
                        const uint16_t* __restrict__ sbi,
                        const uint16_t* __restrict__ X, const int* __restrict__ offsets,
                        const float* __restrict__ gates, const int* __restrict__ assign_pos,
                        uint16_t* __restrict__ Y, int K, int N, int E, int T, int topk,
                        int has_shared) {
    extern __shared__ __align__(16) unsigned char smem[];
    __shared__ int s_off[QL_MAX_EXPERTS_DEV + 1];
    __shared__ int s_exp[QL_MAX_TOPK_DEV + 1];
    __shared__ float s_gate[QL_MAX_TOPK_DEV + 1];
    constexpr int TEAMS = 64 / TPR;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int t = blockIdx.y;
    const int J = topk + (has_shared ? 1 : 0);
    XPairs* s_xp = reinterpret_cast<XPairs*>(smem);                 // [J][G][8]
    float* s_c = reinterpret_cast<float*>(s_xp + (size_t)J * G * 8);  // [J][G]
    float* s_xs = s_c + J * G;                                       // [J][G]

    stage_offsets(offsets, E, s_off);
    if (threadIdx.x < J) {
        const int j = threadIdx.x;
        if (j < topk) {
            s_exp[j] = expert_of_row(s_off, E, min(max(assign_pos[t * topk + j], 0), T * topk - 1));
            s_gate[j] = gates[t * topk + j];
        } else {
            s_exp[j] = -1;  // shared expert, weight 1
            s_gate[j] = 1.0f;
        }
    }
    // Stage pre-paired activations: one (row j, group g) per thread iteration.
    for (int idx = threadIdx.x; idx < J * G; idx += blockDim.x) {
        const int j = idx / G, g = idx % G;
        const int nrows = T * topk + (has_shared ? T : 0);
        const int row = (j < topk) ? min(max(assign_pos[t * topk + j], 0), nrows - 1) : T * topk + t;
        XPairs xp[8];
        float c, xs;
        load_group_x(X + (size_t)row * K, g, xp, c, xs);
#pragma unroll
        for (int w = 0; w < 8; ++w) s_xp[((size_t)j * G + g) * 8 + w] = xp[w];
        s_c[j * G + g] = c;
        s_xs[j * G + g] = xs;
    }
    __syncthreads();

    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int n = (blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64) * TEAMS + team;
    const int nn = min(n, N - 1);
    float acc = 0.f;
    for (int j = 0; j < J; ++j) {
        const int e = s_exp[j];
        const uint32_t* wq = (e >= 0) ? qw + (size_t)e * N * wpr : sqw;
        const uint16_t* ws = (e >= 0) ? sc + (size_t)e * N * G : ssc;
        const uint16_t* wb = (e >= 0) ? bi + (size_t)e * N * G : sbi;
        float part = 0.f;
#pragma unroll
        for (int i = 0; i < GPL; ++i) {
            const int g = lr + i * TPR;
            const uint32_t* p = wq + (size_t)nn * wpr + g * 8;
            const u32x4 c0 = ld_stream_u32x4(p);
            const u32x4 c1 = ld_stream_u32x4(p + 4);
            const float s = h2f(ws[(size_t)nn * G + g]);
            const float b = h2f(wb[(size_t)nn * G + g]);
            const XPairs* xp = s_xp + ((size_t)j * G + g) * 8;
            XPairs xr[8];
#pragma unroll
            for (int w = 0; w < 8; ++w) xr[w] = xp[w];
            part += s * (group_dot(c0, c1, xr) - s_c[j * G + g]) + b * s_xs[j * G + g];
        }
        acc += s_gate[j] * part;
    }
    acc = team_sum<TPR>(acc);
    if (lr == 0 && n < N) Y[(size_t)t * N + n] = f2h(acc);
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

template <int TPR, int GPL>
int launch_rows_t(const GroupedArgs& a, hipStream_t st) {
    constexpr int TEAMS = 64 / TPR;
    constexpr int OUT_PER_BLOCK = 4 * TEAMS;
    const int G = a.K / kGroup;
    if (a.op == QL_OP_DOWN_COMBINE) {
        const int has_shared = a.sqw != nullptr;
        const int J = a.topk + has_shared;
        const size_t smem = (size_t)J * G * (8 * sizeof(XPairs) + 2 * sizeof(float));
        dim3 grid((a.N + OUT_PER_BLOCK - 1) / OUT_PER_BLOCK, a.T);
        hipLaunchKernelGGL((moe_down_combine_kernel<TPR, GPL>), grid, dim3(256), smem, st,
                           a.qw, a.sc, a.bi, a.sqw, a.ssc, a.sbi, a.X, a.offsets, a.gates, a.pos,
                           a.Y, a.K, a.N, a.E, a.T, a.topk, has_shared);
    } else {
        const int R = a.T * a.topk + (a.sqw ? a.T : 0);
        const int Nout = (a.op == QL_OP_GATE_UP_SILU) ? a.N / 2 : a.N;
        dim3 grid((Nout + OUT_PER_BLOCK - 1) / OUT_PER_BLOCK, R);
        if (a.op == QL_OP_GATE_UP_SILU)
            hipLaunchKernelGGL((moe_rows_gemv_kernel<TPR, GPL, 0>), grid, dim3(256), 0, st,
                               a.qw, a.sc, a.bi, a.sqw, a.ssc, a.sbi, a.X, a.offsets,
                               a.sorted_assign, a.Y, a.K, a.N, a.E, a.T, a.topk);
        else
            hipLaunchKernelGGL((moe_rows_gemv_kernel<TPR, GPL, 1>), grid, dim3(256), 0, st,
                               a.qw, a.sc, a.bi, a.sqw, a.ssc, a.sbi, a.X, a.offsets,
                               a.sorted_assign, a.Y, a.K, a.N, a.E, a.T, a.topk);
    }
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

}  // namespace

int launch_gemv(const GemvArgs& a, hipStream_t st) {
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
    const int G = K / kGroup;
    return K % kGroup == 0 && G >= 1 && G <= 256 && (G & (G - 1)) == 0;
}

int launch_moe_rows(const GroupedArgs& a, hipStream_t st) {
    switch (a.K / kGroup) {
        case 1: return launch_rows_t<1, 1>(a, st);
        case 2: return launch_rows_t<2, 1>(a, st);
        case 4: return launch_rows_t<4, 1>(a, st);
        case 8: return launch_rows_t<8, 1>(a, st);
        case 16: return launch_rows_t<16, 1>(a, st);
        case 32: return launch_rows_t<32, 1>(a, st);
        case 64: return launch_rows_t<64, 1>(a, st);
        case 128: return launch_rows_t<64, 2>(a, st);
        case 256: return launch_rows_t<64, 4>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

}  // namespace ql
