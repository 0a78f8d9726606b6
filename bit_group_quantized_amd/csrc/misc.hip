// Pack step of the w4 format and the deterministic MoE combine.
//
// Pack: Perplexity, "Optimizing on-device inference for Apple Silicon",
// section 在矩阵乘法期间进行权重反量化 - each weight is stored as a 4-bit code;
// here 8 codes of one output, consecutive along K, fill one uint32, least
// significant nibble first.
//
// Combine: same page, section 减少中间状态和流量 - the expert outputs are
// weighted by the routing scores and the shared expert's result is added
// (fp16 rows, or bf16 rows for the bf16 variant of the layer).
// One workgroup per token sums its rows in a fixed order, so the result
// does not depend on scheduling (no atomics).
#include "ql_device.h"
#include "ql_internal.h"

namespace ql {

namespace {

__global__ void __launch_bounds__(256)
pack_kernel(const uint8_t* __restrict__ codes, int64_t nwords, uint32_t* __restrict__ qw) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= nwords) return;
    const uint2 v = *reinterpret_cast<const uint2*>(codes + i * 8);
    uint32_t w = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= ((v.x >> (8 * j)) & 0xFu) << (4 * j);
#pragma unroll
    for (int j = 0; j < 4; ++j) w |= ((v.y >> (8 * j)) & 0xFu) << (4 * (j + 4));
    qw[i] = w;
}

// out[t][n] = sum_j gates[t][j] * Yd[pos[t*topk+j]][n] (+ Yd[T*topk+t][n]).
// BF16: rows and output hold bf16 patterns instead of fp16.
template <bool VEC, bool BF16>
__global__ void __launch_bounds__(256)
combine_kernel(const uint16_t* __restrict__ Yd, const float* __restrict__ gates,
               const int* __restrict__ pos, int T, int topk, int N, int has_shared,
               int64_t nrows, uint16_t* __restrict__ out) {
    __shared__ int s_row[QL_MAX_TOPK_DEV + 1];
    __shared__ float s_g[QL_MAX_TOPK_DEV + 1];
    const int t = blockIdx.y;
    const int J = topk + has_shared;
    if (threadIdx.x < J) {
        const int j = threadIdx.x;
        int row;
        float g;
        if (j < topk) {
            row = pos[(size_t)t * topk + j];
            g = gates[(size_t)t * topk + j];
        } else {
            row = T * topk + t;
            g = 1.0f;
        }
        // Rows outside [0, nrows) can only come from an invalid dispatch;
        // they are skipped so that every read stays in bounds.
        s_row[j] = (row >= 0 && row < nrows) ? row : -1;
        s_g[j] = g;
    }
    __syncthreads();
    if constexpr (VEC) {
        const int n8 = blockIdx.x * blockDim.x + threadIdx.x;
        if (n8 * 8 >= N) return;
        float acc[8];
#pragma unroll
        for (int v = 0; v < 8; ++v) acc[v] = 0.f;
        for (int j = 0; j < J; ++j) {
            const int row = s_row[j];
            if (row < 0) continue;
            const u32x4 w = ld_u32x4(Yd + (size_t)row * N + n8 * 8);
            const float g = s_g[j];
            if constexpr (BF16) {
                const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    acc[2 * v] += g * bf2f((uint16_t)(ww[v] & 0xFFFFu));
                    acc[2 * v + 1] += g * bf2f((uint16_t)(ww[v] >> 16));
                }
            } else {
                const f16x8 h = __builtin_bit_cast(f16x8, w);
#pragma unroll
                for (int v = 0; v < 8; ++v) acc[v] += g * (float)h[v];
            }
        }
        if constexpr (BF16) {
            u32x4 o;
            o.x = pack_bf16x2(acc[0], acc[1]);
            o.y = pack_bf16x2(acc[2], acc[3]);
            o.z = pack_bf16x2(acc[4], acc[5]);
            o.w = pack_bf16x2(acc[6], acc[7]);
            *reinterpret_cast<u32x4*>(out + (size_t)t * N + n8 * 8) = o;
        } else {
            f16x8 o;
#pragma unroll
            for (int v = 0; v < 8; ++v) o[v] = (f16)acc[v];
            *reinterpret_cast<f16x8*>(out + (size_t)t * N + n8 * 8) = o;
        }
    } else {
        const int n = blockIdx.x * blockDim.x + threadIdx.x;
        if (n >= N) return;
        float acc = 0.f;
        for (int j = 0; j < J; ++j) {
            const int row = s_row[j];
            if (row < 0) continue;
            const uint16_t y = Yd[(size_t)row * N + n];
            acc += s_g[j] * (BF16 ? bf2f(y) : h2f(y));
        }
        out[(size_t)t * N + n] = BF16 ? f2bf(acc) : f2h(acc);
    }
}

}  // namespace

int launch_pack(const uint8_t* codes, int N, int K, uint32_t* qweight, hipStream_t st) {
    const int64_t nwords = (int64_t)N * (K / 8);
    const int64_t blocks = (nwords + 255) / 256;
    hipLaunchKernelGGL(pack_kernel, dim3((unsigned)blocks), dim3(256), 0, st, codes, nwords, qweight);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

namespace {

template <bool BF16>
void launch_combine_t(const uint16_t* Yd, const float* gates, const int32_t* pos, int T, int topk,
                      int N, int has_shared, uint16_t* out, hipStream_t st) {
    const int64_t nrows = (int64_t)T * topk + (has_shared ? T : 0);
    if (N % 8 == 0) {
        dim3 grid((N / 8 + 255) / 256, T);
        hipLaunchKernelGGL((combine_kernel<true, BF16>), grid, dim3(256), 0, st, Yd, gates, pos, T,
                           topk, N, has_shared, nrows, out);
    } else {
        dim3 grid((N + 255) / 256, T);
        hipLaunchKernelGGL((combine_kernel<false, BF16>), grid, dim3(256), 0, st, Yd, gates, pos, T,
                           topk, N, has_shared, nrows, out);
    }
}

}  // namespace

int launch_combine(const uint16_t* Yd, const float* gates, const int32_t* pos, int T, int topk,
                   int N, int has_shared, uint16_t* out, hipStream_t st, bool bf16) {
    if (bf16) launch_combine_t<true>(Yd, gates, pos, T, topk, N, has_shared, out, st);
    else launch_combine_t<false>(Yd, gates, pos, T, topk, N, has_shared, out, st);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

}  // namespace ql
