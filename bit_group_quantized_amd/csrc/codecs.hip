// Row-parallel GEMV for the second weight codecs: FP8-E4M3 weights with an
// fp16 scale per 64 along K, and NVFP4 (E2M1 codes with an E4M3 scale per 16
// along K and one fp32 scale).
//
// "待验证｜lithos-metal补Apple推理内核", section "一分钟内合并了什么": the
// project decodes FP8 E4M3 weights two codes per half2 and serves an NVFP4
// checkpoint.  Here one gfx950 conversion turns two codes into an fp16 pair
// holding their exact values (NaN codes become NaN), so the products in
// v_dot2_f32_f16 are exact and only the fp32 sums round, as in the w4 GEMV;
// group and block scales are applied to fp32 partial sums.
//
// Lane layout as the chunked w4 GEMV: a team of TPR lanes owns a row, each
// lane 16-byte chunks at a fixed K position, R consecutive rows per team;
// every load of a lane is issued before any arithmetic.
#include "ql_device.h"
#include "ql_codecs.h"
#include "ql_internal.h"

namespace ql {

namespace {

template <int TPR, int V, int R>
__global__ void __launch_bounds__(256)
gemv_fp8_kernel(const uint8_t* __restrict__ codes, const uint16_t* __restrict__ sc,
                const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int K, int N) {
    constexpr int TEAMS = 64 / TPR;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int G = K / 64;
    const int gwave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int row0 = (gwave * TEAMS + team) * R;
    // Chunk c = lr + v * TPR covers codes k = 16c .. 16c + 15.
    u32x4 xr[V][2];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int h = 0; h < 2; ++h) xr[v][h] = ld_u32x4(x + (lr + v * TPR) * 16 + h * 8);
    u32x4 cw[R][V];
    uint16_t s[R][V];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int c = lr + v * TPR;
            cw[r][v] = ld_stream_u32x4(codes + (size_t)row * K + c * 16);
            s[r][v] = sc[(size_t)row * G + (c >> 2)];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            float d0 = 0.f, d1 = 0.f;
            const uint32_t wv[4] = {cw[r][v].x, cw[r][v].y, cw[r][v].z, cw[r][v].w};
            const uint32_t xv[8] = {xr[v][0].x, xr[v][0].y, xr[v][0].z, xr[v][0].w,
                                    xr[v][1].x, xr[v][1].y, xr[v][1].z, xr[v][1].w};
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                // codes (b0, b1) and (b2, b3) of the word, in natural order
                d0 = dot2(as_f16x2(xv[2 * w]), e4m3x2_to_f16x2<false>(wv[w]), d0);
                d1 = dot2(as_f16x2(xv[2 * w + 1]), e4m3x2_to_f16x2<true>(wv[w]), d1);
            }
            acc[r] += h2f(s[r][v]) * (d0 + d1);
        }
    }
    int rsel;
    const float tot = reduce_rows<TPR, R>(acc, lr, rsel);
    if ((lr & (TPR / R - 1)) == 0 && row0 + rsel < N) y[row0 + rsel] = f2h(tot);
}

template <int TPR, int V, int R>
__global__ void __launch_bounds__(256)
gemv_nvfp4_kernel(const uint32_t* __restrict__ qw, const uint8_t* __restrict__ bsc, float gscale,
                  const uint16_t* __restrict__ x, uint16_t* __restrict__ y, int K, int N) {
    constexpr int TEAMS = 64 / TPR;
    const int lane = threadIdx.x & 63;
    const int lr = lane % TPR;
    const int team = lane / TPR;
    const int wpr = K / 8;
    const int NB = K / 16;  // block scales per row
    const int gwave = blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
    const int row0 = (gwave * TEAMS + team) * R;
    // Chunk c = lr + v * TPR covers codes k = 32c .. 32c + 31 (blocks 2c, 2c + 1).
    u32x4 xr[V][4];
#pragma unroll
    for (int v = 0; v < V; ++v)
#pragma unroll
        for (int w = 0; w < 4; ++w) xr[v][w] = ld_u32x4(x + (lr + v * TPR) * 32 + w * 8);
    u32x4 cw[R][V];
    uint16_t bs[R][V];  // the chunk's two block-scale bytes
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int row = min(row0 + r, N - 1);
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const int c = lr + v * TPR;
            cw[r][v] = ld_stream_u32x4(qw + (size_t)row * wpr + c * 4);
            bs[r][v] = *reinterpret_cast<const uint16_t*>(bsc + (size_t)row * NB + 2 * c);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        acc[r] = 0.f;
#pragma unroll
        for (int v = 0; v < V; ++v) {
            const uint32_t wv[4] = {cw[r][v].x, cw[r][v].y, cw[r][v].z, cw[r][v].w};
            float d[2] = {0.f, 0.f};  // blocks 2c and 2c + 1 (words 0-1 and 2-3)
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                const u32x4 xq = xr[v][w];  // x pairs (x0,x1) (x2,x3) (x4,x5) (x6,x7)
                float e = d[w >> 1];
                e = dot2(as_f16x2(xq.x), e2m1x2_to_f16x2<0>(wv[w]), e);
                e = dot2(as_f16x2(xq.y), e2m1x2_to_f16x2<1>(wv[w]), e);
                e = dot2(as_f16x2(xq.z), e2m1x2_to_f16x2<2>(wv[w]), e);
                e = dot2(as_f16x2(xq.w), e2m1x2_to_f16x2<3>(wv[w]), e);
                d[w >> 1] = e;
            }
            const uint32_t b2 = bs[r][v];
            acc[r] += e4m3_to_f32<0>(b2) * d[0] + e4m3_to_f32<1>(b2) * d[1];
        }
    }
    int rsel;
    const float tot = reduce_rows<TPR, R>(acc, lr, rsel);
    if ((lr & (TPR / R - 1)) == 0 && row0 + rsel < N) y[row0 + rsel] = f2h(tot * gscale);
}

constexpr int kCodecRows = 8;
constexpr int kCodecMinBlocks = 1024;

template <int TPR, int V, int R>
int launch_fp8_t(const CodecArgs& a, hipStream_t st) {
    constexpr int RPB = 4 * (64 / TPR) * R;
    const int blocks = (a.N + RPB - 1) / RPB;
    hipLaunchKernelGGL((gemv_fp8_kernel<TPR, V, R>), dim3(blocks), dim3(256), 0, st, a.codes8, a.scales,
                       a.x, a.y, a.K, a.N);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

template <int TPR, int V, int R>
int launch_nvfp4_t(const CodecArgs& a, hipStream_t st) {
    constexpr int RPB = 4 * (64 / TPR) * R;
    const int blocks = (a.N + RPB - 1) / RPB;
    hipLaunchKernelGGL((gemv_nvfp4_kernel<TPR, V, R>), dim3(blocks), dim3(256), 0, st, a.codes4,
                       a.block_scales, a.global_scale, a.x, a.y, a.K, a.N);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

// 8 rows per team, or 2 when that leaves too few blocks to fill the chip.
template <int TPR, int V, bool FP8>
int launch_codec_r(const CodecArgs& a, hipStream_t st) {
    constexpr int R = (kCodecRows < TPR) ? kCodecRows : TPR;
    const long blocks_big = (a.N + 4L * (64 / TPR) * R - 1) / (4L * (64 / TPR) * R);
    const bool big = blocks_big >= kCodecMinBlocks || R <= 2;
    if constexpr (FP8)
        return big ? launch_fp8_t<TPR, V, R>(a, st) : launch_fp8_t<TPR, V, 2>(a, st);
    else
        return big ? launch_nvfp4_t<TPR, V, R>(a, st) : launch_nvfp4_t<TPR, V, 2>(a, st);
}

}  // namespace

bool gemv_fp8_supported(int K) {
    switch (K) {
        case 256: case 512: case 1024: case 2048: case 4096: case 8192: return true;
        default: return false;
    }
}

bool gemv_nvfp4_supported(int K) { return gemv_fused_supported(K); }

int launch_gemv_fp8(const CodecArgs& a, hipStream_t st) {
    // K/16 chunks of 16 codes per row.
    switch (a.K) {
        case 256: return launch_codec_r<16, 1, true>(a, st);
        case 512: return launch_codec_r<32, 1, true>(a, st);
        case 1024: return launch_codec_r<64, 1, true>(a, st);
        case 2048: return launch_codec_r<64, 2, true>(a, st);
        case 4096: return launch_codec_r<64, 4, true>(a, st);
        case 8192: return launch_fp8_t<64, 8, 4>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

int launch_gemv_nvfp4(const CodecArgs& a, hipStream_t st) {
    // K/32 chunks of 32 codes per row.
    switch (a.K) {
        case 256: return launch_codec_r<8, 1, false>(a, st);
        case 512: return launch_codec_r<16, 1, false>(a, st);
        case 1024: return launch_codec_r<32, 1, false>(a, st);
        case 2048: return launch_codec_r<64, 1, false>(a, st);
        case 4096: return launch_codec_r<64, 2, false>(a, st);
        case 8192: return launch_nvfp4_t<64, 4, 4>(a, st);
        case 16384: return launch_nvfp4_t<64, 8, 2>(a, st);
        default: return QL_ERR_UNSUPPORTED_SHAPE;
    }
}

}  // namespace ql
