// Internal interface between the C-ABI layer (capi.cpp) and the kernel
// translation units.  Not installed; callers use include/qlinear.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

#include "../../include/qlinear.h"

#define QL_MAX_EXPERTS_DEV QL_MAX_EXPERTS
#define QL_MAX_TOPK_DEV QL_MAX_TOPK

namespace ql {

// Raises a kernel's dynamic LDS limit on the current device, once per device
// (bit d of `done` records device d; devices past 31 set it on every call).
// Safe to call from several host threads.
inline int set_max_dynamic_lds(const void* kernel, size_t bytes, std::atomic<uint32_t>& done) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return QL_ERR_HIP;
    const uint32_t bit = (dev >= 0 && dev < 32) ? (1u << dev) : 0u;
    if (bit && (done.load(std::memory_order_acquire) & bit)) return QL_OK;
    if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes) != hipSuccess)
        return QL_ERR_HIP;
    if (bit) done.fetch_or(bit, std::memory_order_release);
    return QL_OK;
}

struct GemvArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint16_t* biases;
    const uint16_t* x;
    uint16_t* y;
    int K, N;
    const uint16_t* gamma = nullptr;  // RMSNorm prologue
    float eps = 0.f;
    uint64_t* partials = nullptr;     // argmax epilogue: one key per block
    int32_t* token = nullptr;         // argmax result / embedding row id
};
int launch_gemv(const GemvArgs& a, hipStream_t st);
// K with the chunked kernel (powers of two 256 .. 16384): the fused variants.
bool gemv_fused_supported(int K);
int launch_gemv_rmsnorm(const GemvArgs& a, hipStream_t st);
// Up to QL_GEMV_MULTI_MAX matrices sharing x (same K, a chunked-kernel K).
struct GemvMultiArgs {
    const uint32_t* qweight[QL_GEMV_MULTI_MAX];
    const uint16_t* scales[QL_GEMV_MULTI_MAX];
    const uint16_t* biases[QL_GEMV_MULTI_MAX];
    uint16_t* y[QL_GEMV_MULTI_MAX];
    int N[QL_GEMV_MULTI_MAX];
    int count;
    int K;
    const uint16_t* x;
};
int launch_gemv_multi(const GemvMultiArgs& a, hipStream_t st);
// Second weight codecs, single-row GEMV with fp16 x and y.
struct CodecArgs {
    const uint8_t* codes8 = nullptr;        // FP8: E4M3 codes [N][K]
    const uint16_t* scales = nullptr;       // FP8: fp16 scale [N][K/64]
    const uint32_t* codes4 = nullptr;       // NVFP4: E2M1 codes [N][K/8] (w4 packing)
    const uint8_t* block_scales = nullptr;  // NVFP4: E4M3 scale [N][K/16]
    float global_scale = 1.f;               // NVFP4
    const uint16_t* x = nullptr;
    uint16_t* y = nullptr;
    int K = 0, N = 0;
};
bool gemv_fp8_supported(int K);    // 256 .. 8192, powers of two
bool gemv_nvfp4_supported(int K);  // 256 .. 16384, powers of two
int launch_gemv_fp8(const CodecArgs& a, hipStream_t st);
int launch_gemv_nvfp4(const CodecArgs& a, hipStream_t st);
// bf16 activations, scales, biases and outputs; the chunked K set.
int launch_gemv_bf16(const GemvArgs& a, hipStream_t st);
// Writes a.y if non-null, the block keys to a.partials (at most
// ceil(N / 8) of them) and the token id to a.token.
int launch_gemv_argmax(const GemvArgs& a, hipStream_t st);
// a.y = fp16 row *a.token of the w4 table (a.K wide, a.N rows).
int launch_embed(const GemvArgs& a, hipStream_t st);

struct GemmArgs {
    const uint32_t* qweight;
    const uint16_t* scales;
    const uint16_t* biases;
    const uint16_t* X;
    uint16_t* Y;
    int64_t M;
    int K, N;
    float gscale = 1.f;  // NVFP4 weights: global scale
};
int launch_gemm(const GemmArgs& a, hipStream_t st);
// bf16 activations, scales, biases and outputs (same tile table).
int launch_gemm_bf16(const GemmArgs& a, hipStream_t st);
// FP8-E4M3 weights: qweight points at the uint8 codes [N][K], scales fp16
// [N][K/64], biases unused.
int launch_gemm_fp8(const GemmArgs& a, hipStream_t st);
// NVFP4 weights: qweight the E2M1 codes [N][K/8], scales points at the E4M3
// block scales (bytes) [N][K/16], gscale the global scale.
int launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st);
// K split in two halves inside each workgroup (K a multiple of 128).
bool gemm_ksplit_supported(int K);
int launch_gemm_ksplit(const GemmArgs& a, hipStream_t st);
bool gemm_ws_supported(int K);                          // few-row GEMM shapes
int launch_gemm_ws(const GemmArgs& a, hipStream_t st);  // few-row GEMM (weight-stationary)

int launch_pack(const uint8_t* codes, int N, int K, uint32_t* qweight, hipStream_t st);

// Workspace carving shared by the routing and grouped-GEMM launchers.
struct MoeWorkspace {
    size_t header;        // int32[4]: num_tiles, tile_rows, error, reserved
    size_t tiles;         // int32[max_tiles][4]
    size_t logits;        // float[T][E]
    size_t partials;      // float[T][nparts][E]   router partial sums
    size_t chunk_counts;  // int32[nchunks][E]
    size_t chunk_err;     // int32[nchunks]
    size_t chunk_masks;   // uint32[nchunks][E][8]   which tokens of each 256-token chunk chose each expert
    size_t row_info;      // int32[T*topk][2]: (expert, token) of each routed row
    size_t assign_info;   // int32[T*topk][2]: (expert, row) of each assignment
    size_t short_order;   // int32[max_tiles]: the short tiles by cost (see dispatch_scan_kernel)
    size_t total;
    int max_tiles, nchunks, nparts;
};

constexpr int kRouteChunkTokens = 256;  // tokens per dispatch chunk
constexpr int kTinyTileRows = 32;       // short tiles of at most this many rows take the register-streamed tile
constexpr int kRouterPartRows = 64;     // D rows per small-T router partial
constexpr int kRouterSmallT = 16;       // T at or below: row-parallel router
constexpr int kRouterMfmaSplit = 4;     // K splits of the MFMA router (partials per logit)
constexpr int kRouterSmallParts = 8;    // small-T router: D split in 8 slices, one partial each

struct RouteArgs {
    const uint16_t* H;
    const uint16_t* Wr;
    const float* bias;
    int T, D, E, topk;
    int32_t* ids;
    float* gates;
    int32_t* counts;
    int32_t* offsets;
    int32_t* sorted_assign;
    int32_t* pos;
    unsigned char* ws;
    bool bf16 = false;  // H and Wr hold bf16 patterns
};
int launch_router_logits_mfma(const uint16_t* H, const uint16_t* Wr, float* partials, int T, int D,
                              int E, hipStream_t st, bool bf16 = false);
bool router_uses_mfma(int T, int E);
// Small-T router partials: [T][kRouterSmallParts][E] fp32; their sum over the
// slices in ascending order (plus the bias) is the logit.
int launch_router_partials_small(const uint16_t* H, const uint16_t* Wr, float* partials, int T,
                                 int D, int E, hipStream_t st, bool bf16 = false);
int launch_route(const RouteArgs& a, hipStream_t st);
MoeWorkspace moe_workspace_layout(int T, int E, int topk);     // logits + top-k + dispatch
int launch_dispatch(const RouteArgs& a, hipStream_t st);  // dispatch only (ids given)

struct GroupedArgs {
    const uint32_t* qw;
    const uint16_t* sc;
    const uint16_t* bi;
    const uint32_t* sqw;  // shared expert or null
    const uint16_t* ssc;
    const uint16_t* sbi;
    const uint16_t* X;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    const float* gates;
    const int32_t* pos;
    const unsigned char* ws;
    uint16_t* Y;
    int K, N, E, T, topk, op;
    bool bf16 = false;  // X, scales, biases and Y hold bf16 patterns
    int wf = 0;         // 1: FP8 experts (qw = codes as bytes, sc = fp16 scales, no biases)
                        // 2: NVFP4 experts (qw = codes, sc = E4M3 block-scale bytes, no biases)
    const float* gscales = nullptr;  // NVFP4: per-expert global scales (device, [E])
    float sgscale = 0.f;             // NVFP4: the shared expert's global scale
    bool shared_only = false;        // the shared expert's rows only (no routing inputs read)
};
bool moe_rows_supported(int K);
int launch_moe_rows(const GroupedArgs& a, hipStream_t st);    // small T, row-parallel
int launch_moe_grouped(const GroupedArgs& a, hipStream_t st); // any T, MFMA tiles

// Whole decode layer (T <= QL_DECODE_MAX_T) in three launches: router
// partials; routing fused into the gate/up rows; down rows fused with the
// gate-weighted sum.
struct DecodeLayout {
    size_t partials;     // fp32 [T][kRouterSmallParts][E]
    size_t logits;       // fp32 [T][E]
    size_t assign_info;  // int32 [T*topk][2]: (expert, row) of each assignment
    size_t act;          // fp16 [T*topk + T][I], assignment order, then shared rows
    size_t total;
};
DecodeLayout moe_decode_layout(int T, int E, int topk, int I);
struct DecodeArgs {
    const uint16_t* H;
    const uint16_t* Wr;
    const float* bias;
    int T, D, E, topk, I;
    const uint32_t* gu_qw;  // routed experts, gate/up [E][2I][D/8]
    const uint16_t* gu_sc;
    const uint16_t* gu_bi;
    const uint32_t* dn_qw;  // routed experts, down [E][D][I/8]
    const uint16_t* dn_sc;
    const uint16_t* dn_bi;
    const uint32_t* sgu_qw;  // shared expert (all null or all set)
    const uint16_t* sgu_sc;
    const uint16_t* sgu_bi;
    const uint32_t* sdn_qw;
    const uint16_t* sdn_sc;
    const uint16_t* sdn_bi;
    int32_t* ids;
    float* gates;
    unsigned char* ws;
    uint16_t* out;
    bool bf16 = false;  // H, Wr, scales, biases, act and out hold bf16 patterns
    int wf = 0;         // expert weight format: 0 w4, 1 FP8 (codes as bytes, fp16 scales, no biases),
                        // 2 NVFP4 (codes, E4M3 block-scale bytes through the scale pointers)
    const float* gu_gscales = nullptr;  // NVFP4: per-expert global scales (device, [E])
    const float* dn_gscales = nullptr;
    float sgu_gscale = 0.f;             // NVFP4: the shared expert's global scales
    float sdn_gscale = 0.f;
};
int launch_moe_decode(const DecodeArgs& a, hipStream_t st);
// This device's copy of the library's decode scratch array
// (QL_DECODE_SCRATCH_BYTES), resolved on the first call on each device.
int decode_scratch(unsigned char** ptr);

int launch_combine(const uint16_t* Yd, const float* gates, const int32_t* pos, int T, int topk,
                   int N, int has_shared, uint16_t* out, hipStream_t st, bool bf16 = false);

}  // namespace ql
