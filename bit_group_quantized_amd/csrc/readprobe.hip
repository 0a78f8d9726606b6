// Measurement kernels for the benchmark (libqlprobe), not part of the
// qlinear interface.
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

}  // namespace

extern "C" {

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
