// Measurement kernels for the benchmark (libqlprobe), not part of the
// qlinear interface.
//
// Also an LDS throughput probe and the latency probes further down.
//
// HBM read-bandwidth probe for the benchmark's calibration leg:
// the fastest sustained read rate of this chip for the weight-read pattern
// of the row GEMV, and for a plain streaming read, so that the GEMV's
// achieved bandwidth can be reported beside a measured ceiling as well as
// beside the 8 TB/s specification.  Not part of the qlinear interface.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// 进一步优化的局限性: kernels there are graded against the fastest sustained
// weight-read rate for their access pattern.
//
// Pattern "rows": the buffer is cut into 1 KB rows (the codes of one K = 2048
// output of the w4 GEMV); a block of four waves owns 8 consecutive rows per
// wave; each lane issues one 16-byte non-temporal load per row (one wave
// instruction reads a whole row), all eight before using any, exactly as
// gemv_w4_chunked_kernel<64, 1, 8> loads its codes.  Pattern "stream": every
// thread walks the buffer in 16-byte steps with a grid-wide stride.  Each
// block XOR-folds what it read into one word, so no load can be dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t fold(u32x4 v) { return v.x ^ v.y ^ v.z ^ v.w; }

__device__ __forceinline__ void block_out(uint32_t acc, uint32_t* out) {
    __shared__ uint32_t s[4];
    for (int off = 32; off >= 1; off >>= 1) acc ^= __shfl_xor(acc, off, 64);
    if ((threadIdx.x & 63) == 0) s[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[blockIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

__global__ void __launch_bounds__(256) read_rows_kernel(const u32x4* __restrict__ buf, size_t rows,
                                                        uint32_t* __restrict__ out) {
    constexpr int R = 8;
    const int lane = threadIdx.x & 63;
    const size_t wave = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const size_t row0 = wave * R;
    u32x4 v[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const size_t row = min(row0 + r, rows - 1);
        v[r] = __builtin_nontemporal_load(buf + row * 64 + lane);
    }
    uint32_t acc = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) acc ^= fold(v[r]);
    block_out(acc, out);
}

__global__ void __launch_bounds__(256) read_stream_kernel(const u32x4* __restrict__ buf, size_t n16,
                                                          uint32_t* __restrict__ out) {
    constexpr int U = 4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    uint32_t acc = 0;
    for (; i + (U - 1) * stride < n16; i += U * stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(buf + i + u * stride);
#pragma unroll
        for (int u = 0; u < U; ++u) acc ^= fold(v[u]);
    }
    for (; i < n16; i += stride) acc ^= fold(__builtin_nontemporal_load(buf + i));
    block_out(acc, out);
}

// Latency probes: an empty kernel (the cost of a launch, or of one node of
// a HIP graph, with no work in it), and one thread following a chain of
// dependent loads through a buffer (the round trip of one load from
// wherever the buffer lives: L2, the Infinity Cache or HBM).
__global__ void empty_kernel() {}

__global__ void chase_kernel(const uint32_t* __restrict__ next, uint32_t mask, uint32_t start, int steps,
                             uint32_t* __restrict__ out) {
    // The index mixes in threadIdx.x (0 here: one thread) so that the loads
    // are vector-memory loads, not scalar ones.
    uint32_t i = (start ^ threadIdx.x) & mask;
    for (int s = 0; s < steps; ++s) i = (next[i] ^ threadIdx.x) & mask;  // the mask keeps every load in bounds
    out[0] = i;
}

// LDS throughput probe: eight waves of one workgroup (one per CU: 96 KB of
// LDS each) issue groups of eight 16-byte (or 8-byte) LDS accesses back to
// back, and thread 0 records the shader clocks (s_memtime) the loop took, so
// bytes / cycles is the CU's LDS rate for that access form.  The accesses
// are written as instructions so that no address or data arithmetic sits
// between them.  Mode 0: ds_read_b128, 64 lanes reading 1 KB contiguous;
// mode 1: ds_read_b128 in the matrix-fragment pattern of the GEMM tiles
// (lane l reads row l % 32 of a 144-byte-stride tile, 64-byte half l / 32);
// mode 2: ds_write_b128 in the activation staging pattern (8 lanes per
// 144-byte row); mode 3: ds_write_b64, 64 lanes writing 512 B contiguous.
// Every address is below 40 KB of the 64 KB the kernel initializes.
constexpr int kLdsProbeWaves = 8;
constexpr int kLdsProbeBlocks = 256;
constexpr size_t kLdsProbeBytes = 96 * 1024;

template <int MODE>
__global__ void __launch_bounds__(64 * kLdsProbeWaves)
lds_probe_kernel(int iters, long long* __restrict__ cycles, uint32_t* __restrict__ out) {
    extern __shared__ __align__(16) u32x4 lds_buf[];
    for (int i = threadIdx.x; i < 4096; i += blockDim.x)
        lds_buf[i] = u32x4{(uint32_t)i, (uint32_t)i * 3u, (uint32_t)i * 5u, (uint32_t)i * 7u};
    __syncthreads();
    const uint32_t lane = threadIdx.x & 63;
    uint32_t a0;
    if (MODE == 0) a0 = lane * 16u;
    else if (MODE == 1) a0 = (lane & 31u) * 144u + (lane >> 5) * 64u;
    else if (MODE == 2) a0 = (lane >> 3) * 144u + (lane & 7u) * 16u;
    else a0 = lane * 8u;
    a0 += (uint32_t)(uintptr_t)lds_buf;
    uint32_t acc = 0;
    __syncthreads();
    const long long t0 = clock64();
    for (int it = 0; it < iters; ++it) {
        const uint32_t a = a0 + (uint32_t)(it & 1) * 16u;
        if constexpr (MODE <= 1) {
            u32x4 v0, v1, v2, v3, v4, v5, v6, v7;
            asm volatile(
                "ds_read_b128 %0, %8 offset:0\n ds_read_b128 %1, %8 offset:4608\n"
                "ds_read_b128 %2, %8 offset:9216\n ds_read_b128 %3, %8 offset:13824\n"
                "ds_read_b128 %4, %8 offset:18432\n ds_read_b128 %5, %8 offset:23040\n"
                "ds_read_b128 %6, %8 offset:27648\n ds_read_b128 %7, %8 offset:32256\n"
                "s_waitcnt lgkmcnt(0)"
                : "=v"(v0), "=v"(v1), "=v"(v2), "=v"(v3), "=v"(v4), "=v"(v5), "=v"(v6), "=v"(v7)
                : "v"(a)
                : "memory");
            acc ^= v0.x ^ v7.w;
        } else if constexpr (MODE == 2) {
            const u32x4 w = {(uint32_t)it, lane, 0u, 0u};
            asm volatile(
                "ds_write_b128 %0, %1 offset:0\n ds_write_b128 %0, %1 offset:4608\n"
                "ds_write_b128 %0, %1 offset:9216\n ds_write_b128 %0, %1 offset:13824\n"
                "ds_write_b128 %0, %1 offset:18432\n ds_write_b128 %0, %1 offset:23040\n"
                "ds_write_b128 %0, %1 offset:27648\n ds_write_b128 %0, %1 offset:32256\n"
                "s_waitcnt lgkmcnt(0)" ::"v"(a),
                "v"(w)
                : "memory");
        } else {
            const uint64_t w = ((uint64_t)lane << 32) | (uint32_t)it;
            asm volatile(
                "ds_write_b64 %0, %1 offset:0\n ds_write_b64 %0, %1 offset:4608\n"
                "ds_write_b64 %0, %1 offset:9216\n ds_write_b64 %0, %1 offset:13824\n"
                "ds_write_b64 %0, %1 offset:18432\n ds_write_b64 %0, %1 offset:23040\n"
                "ds_write_b64 %0, %1 offset:27648\n ds_write_b64 %0, %1 offset:32256\n"
                "s_waitcnt lgkmcnt(0)" ::"v"(a),
                "v"(w)
                : "memory");
        }
    }
    __syncthreads();
    const long long t1 = clock64();
    if (threadIdx.x == 0) cycles[blockIdx.x] = t1 - t0;
    out[blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

template <int MODE>
int launch_lds_probe(int iters, long long* cycles, uint32_t* out, hipStream_t st) {
    if (hipFuncSetAttribute((const void*)lds_probe_kernel<MODE>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            (int)kLdsProbeBytes) != hipSuccess)
        return 5;
    hipLaunchKernelGGL((lds_probe_kernel<MODE>), dim3(kLdsProbeBlocks), dim3(64 * kLdsProbeWaves), kLdsProbeBytes,
                       st, iters, cycles, out);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // namespace

extern "C" {

// LDS probe (modes 0-3 above): `cycles` holds ql_probe_lds_blocks() int64,
// `out` ql_probe_lds_blocks() * 512 uint32.  Each workgroup moves
// ql_probe_lds_bytes(mode, iters) bytes.  Returns 0, 1 on a bad argument,
// 5 on a launch error.
int ql_probe_lds_blocks(void) { return kLdsProbeBlocks; }

double ql_probe_lds_bytes(int mode, int iters) {
    return (double)kLdsProbeWaves * iters * 8 * (mode == 3 ? 512.0 : 1024.0);
}

int ql_probe_lds(int mode, int iters, long long* cycles, uint32_t* out, void* stream) {
    if (!cycles || !out || iters < 1) return 1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    switch (mode) {
        case 0: return launch_lds_probe<0>(iters, cycles, out, st);
        case 1: return launch_lds_probe<1>(iters, cycles, out, st);
        case 2: return launch_lds_probe<2>(iters, cycles, out, st);
        case 3: return launch_lds_probe<3>(iters, cycles, out, st);
        default: return 1;
    }
}

int ql_probe_empty(void* stream) {
    hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, reinterpret_cast<hipStream_t>(stream));
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

// next: n uint32 indices, n a power of two (values are masked to n - 1);
// out: one uint32.  One thread follows `steps` dependent loads from `start`.
int ql_probe_chase(const uint32_t* next, uint32_t n, uint32_t start, int steps, uint32_t* out,
                   void* stream) {
    if (!next || !out || n == 0 || (n & (n - 1)) != 0 || steps < 0) return 1;
    hipLaunchKernelGGL(chase_kernel, dim3(1), dim3(1), 0, reinterpret_cast<hipStream_t>(stream), next, n - 1,
                       start, steps, out);
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

// Blocks a probe launch writes one word each to `out` (uint32).
size_t ql_probe_out_words(int pattern, size_t bytes) {
    if (pattern == 0) return (bytes / 1024 + 31) / 32;  // rows: 8 rows per wave, 4 waves per block
    return 4096;                                        // stream: a fixed grid
}

// Reads `bytes` (a positive multiple of 1024, 16-byte aligned) of `buf` once
// with pattern 0 ("rows") or 1 ("stream"); `out` holds
// ql_probe_out_words(pattern, bytes) words.  Returns 0, or 1 on a bad
// argument, 5 on a launch error.
int ql_read_probe(int pattern, const void* buf, size_t bytes, uint32_t* out, void* stream) {
    if (!buf || !out || bytes == 0 || bytes % 1024 != 0 || (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
        return 1;
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const u32x4* b = static_cast<const u32x4*>(buf);
    if (pattern == 0) {
        const size_t rows = bytes / 1024;
        const size_t blocks = (rows + 31) / 32;
        if (blocks > 0x7fffffffu) return 1;
        hipLaunchKernelGGL(read_rows_kernel, dim3((unsigned)blocks), dim3(256), 0, st, b, rows, out);
    } else if (pattern == 1) {
        hipLaunchKernelGGL(read_stream_kernel, dim3(4096), dim3(256), 0, st, b, bytes / 16, out);
    } else {
        return 1;
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
