/*
 * qlinear.h - C ABI of the group-affine 4-bit linear-layer and routed-expert
 * MoE library for AMD Instinct MI355X (gfx950).
 *
 * Sources of the operations (page title, then section):
 *   [PPLX] Perplexity, "Optimizing on-device inference for Apple Silicon":
 *     "在矩阵乘法期间进行权重反量化"  dequantizing weights inside the matmul
 *     "将专家路由保留在 GPU 上"        keeping expert routing on the GPU
 *     "使瓦片大小与专家负载相匹配"    matching tile size to expert load
 *     "Qwen 创建了三种不同的工作负载形状" the three workload shapes (top-8 of
 *                                      256 experts plus one shared expert)
 *     "优化单行权重路径"              the row-parallel single-row GEMV
 *     "减少中间状态和流量"            the fused decode expert chains
 *     "将 token 交接保留在 GPU 上"    the token hand-off kept on the GPU
 *   [LITHOS] "待验证｜lithos-metal补Apple推理内核", "一分钟内合并了什么":
 *     FP8 E4M3 decode and the NVFP4 checkpoint (second codecs)
 *   [LAYA] laya-mlx, "工程调查：这个 MLX 端口还能再快 10× 吗？",
 *     "选择性量化": affine quantization with group size 64.
 *
 * ---------------------------------------------------------------------------
 * Packed-weight layout (version QL_LAYOUT_VERSION)
 * ---------------------------------------------------------------------------
 * A logical weight matrix W has K inputs and N outputs; a linear layer
 * computes y[n] = sum_k x[k] * W[k][n].  Each weight is a 4-bit code
 * q in 0..15; each group of 64 consecutive k of one output n shares an fp16
 * scale and an fp16 bias, and W[k][n] = scale[n][k/64] * q(n,k) +
 * bias[n][k/64]  ([PPLX] dequantization section; the bias form and fp16
 * scale/bias are this library's reading of it).
 *
 *   qweight  uint32 [N][K/8], row-major.  Word w of row n holds codes
 *            k = 8w .. 8w+7; code k sits in bits [4*(k%8), 4*(k%8)+4)
 *            (least significant nibble first).
 *   scales   fp16 bit patterns [N][K/64], row-major.
 *   biases   fp16 bit patterns [N][K/64], row-major.
 *   K must be a positive multiple of 64 (group_size must be 64); N >= 0.
 *   Stacked experts: [E][N][K/8] and [E][N][K/64], expert after expert.
 *   Expert gate_up matrices: columns [0, I) are the gate projection and
 *   [I, 2I) the up projection of the same expert.
 *
 * Activations and outputs are fp16 bit patterns, row-major.  Accumulation
 * is in fp32; outputs are rounded to fp16 to nearest even.
 *
 * ---------------------------------------------------------------------------
 * Conventions for every entry point
 * ---------------------------------------------------------------------------
 * - All pointers except those documented as host values are device
 *   pointers.  The caller owns every buffer; the library never allocates,
 *   frees or synchronizes, and keeps no state between calls.
 * - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL means
 *   the default stream).  Calls are re-entrant.
 * - Arguments are validated on the host before anything is enqueued; a
 *   failing check returns an error and enqueues nothing.  Sizes of zero
 *   (M, N or T) are valid and enqueue nothing.
 * - Device pointers to packed weights, activations and outputs must be
 *   16-byte aligned; scales/biases 2-byte; int32/float arrays 4-byte.
 * - A launch failure reported by the runtime returns QL_ERR_HIP.  Faults in
 *   kernels surface at the caller's next synchronization of the stream.
 */
#ifndef QLINEAR_H
#define QLINEAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define QL_LAYOUT_VERSION 1
#define QL_GROUP_SIZE 64

/* Rows per tile of the routed tile map written by moe_route/moe_dispatch. */
#define QL_MOE_TILE_ROWS 128

/* Status codes. */
#define QL_OK 0
#define QL_ERR_INVALID_ARG 1      /* null pointer, negative size, topk > E ... */
#define QL_ERR_UNSUPPORTED_SHAPE 2 /* K % 64 != 0, group_size != 64, limits   */
#define QL_ERR_MISALIGNED 3       /* a pointer violates its alignment rule    */
#define QL_ERR_WORKSPACE 4        /* workspace null or smaller than required  */
#define QL_ERR_HIP 5              /* the HIP runtime rejected a launch        */

/* Operations of moe_grouped_gemm. */
#define QL_OP_GATE_UP_SILU 1
#define QL_OP_DOWN 2
#define QL_OP_DOWN_COMBINE 3
/* Flag or'ed into the op of the grouped GEMMs (with QL_OP_GATE_UP_SILU or
 * QL_OP_DOWN): compute only the shared expert's rows. */
#define QL_OP_SHARED_ONLY 0x100

/* Limits. */
#define QL_MAX_EXPERTS 1024
#define QL_MAX_TOPK 32
#define QL_MAX_K 32768
#define QL_DECODE_MAX_T 4 /* largest T served by the row-parallel expert path */
#define QL_DECODE_SCRATCH_BYTES (1u << 20) /* device scratch of moe_decode_noalloc */
#define QL_GEMV_MULTI_MAX 8 /* matrices of one qlinear_gemv_multi call */

/* One w4 matrix (host struct holding device pointers). */
typedef struct ql_w4 {
    const uint32_t* qweight; /* [N][K/8]  */
    const uint16_t* scales;  /* [N][K/64] */
    const uint16_t* biases;  /* [N][K/64] */
    int32_t K;
    int32_t N;
    int32_t group_size; /* must be 64 */
} ql_w4;

/* num_experts w4 matrices of the same shape stacked contiguously. */
typedef struct ql_w4_experts {
    const uint32_t* qweight; /* [E][N][K/8]  */
    const uint16_t* scales;  /* [E][N][K/64] */
    const uint16_t* biases;  /* [E][N][K/64] */
    int32_t K;
    int32_t N;
    int32_t group_size; /* must be 64 */
    int32_t num_experts;
} ql_w4_experts;

/* Version of the packed layout above. */
int ql_layout_version(void);

/* Static description of a status code (never NULL). */
const char* ql_status_string(int status);

/*
 * qlinear_pack - build packed words from one code per byte.
 * Offline format step of [PPLX] dequantization section: 4-bit codes packed
 * 8 per uint32 along K as described in the layout above.
 *   codes    uint8 [N][K], each 0..15 (higher bits are ignored).
 *   qweight  uint32 [N][K/8] output.
 * K must be a positive multiple of 8.  Errors: INVALID_ARG, MISALIGNED
 * (codes and qweight 16-byte aligned), UNSUPPORTED_SHAPE.
 */
int qlinear_pack(const uint8_t* codes, int32_t N, int32_t K, uint32_t* qweight, void* stream);

/*
 * qlinear_gemv - y = x . dequant(W) for one activation row (batch-1 decode).
 * [PPLX] "优化单行权重路径" (row-parallel GEMV) with the dequantization of
 * the same page's dequantization section done in registers.
 *   W  a K x N w4 matrix;  x  fp16 [K];  y  fp16 [N] output.
 * Errors: INVALID_ARG (null W/x/y with N > 0), UNSUPPORTED_SHAPE (K % 64,
 * K > QL_MAX_K, group_size != 64), MISALIGNED, HIP.
 */
int qlinear_gemv(const ql_w4* W, const uint16_t* x, uint16_t* y, void* stream);

/*
 * qlinear_gemv_multi - y_i = x . dequant(W_i) for `count` matrices that
 * share one activation row (a decode step's projections of the same
 * input), in one launch.  [PPLX] "优化单行权重路径" as qlinear_gemv; the
 * single launch removes the per-launch dispatch gap of the separate calls.
 *   Ws     host array of count K x N_i w4 matrices, all with the same K, K
 *          one of 256, 512, 1024, 2048, 4096, 8192, 16384;
 *   x      fp16 [K];  ys  host array of count device pointers, fp16 [N_i].
 * Every output has the bits qlinear_gemv gives for its matrix.
 * 1 <= count <= QL_GEMV_MULTI_MAX; matrices with N_i = 0 are skipped.
 * Errors: INVALID_ARG (null Ws/ys/x/ys[i], count out of range, K differs),
 * UNSUPPORTED_SHAPE (K not in the list, or as qlinear_gemv), MISALIGNED, HIP.
 */
int qlinear_gemv_multi(const ql_w4* Ws, int32_t count, const uint16_t* x, uint16_t* const* ys,
                       void* stream);

/*
 * qlinear_gemm - Y = X . dequant(W) for M activation rows (prefill).
 * [PPLX] dequantization section: small weight tiles are dequantized into
 * on-chip memory just long enough to be multiplied; fp32 accumulation,
 * 16-bit output; the full dequantized matrix never exists in memory.
 *   X  fp16 [M][K];  Y  fp16 [M][N] output.  Row m of Y depends only on row
 *   m of X and is bit-identical whatever M is (no split over K).
 * Errors: as qlinear_gemv, plus INVALID_ARG for M < 0.
 */
int qlinear_gemm(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/*
 * qlinear_gemm_few_rows - Y = X . dequant(W) for few activation rows: the
 * verify-sized groups and small expert batches the pages discuss between
 * the single-row and the many-row path ([PPLX] "使瓦片大小与专家负载相匹配",
 * tile choice against row count; "优化单行权重路径").  Weight-stationary:
 * every weight is read and dequantized once and kept in registers while all
 * M rows stream past it, so the cost grows slowly with M.  Measured on
 * MI355X it is 2-3x faster than qlinear_gemm for 2 to 64 rows, equal near
 * 128 and slower beyond (the activations are re-read once per 32 columns).
 *   X fp16 [M][K], Y fp16 [M][N]; fp16 dequantized weights, fp32 accumulation
 *   split over 8 K slices summed in a fixed order: deterministic, but its
 *   rounding differs from qlinear_gemm's (which does not split K).
 * Limits: K in {512, 1024, 2048}.
 * Errors: as qlinear_gemm; UNSUPPORTED_SHAPE for other K.
 */
int qlinear_gemm_few_rows(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y,
                          void* stream);

/*
 * qlinear_gemm_ksplit - Y = X . dequant(W) for a few hundred rows ([PPLX]
 * dequantization section, as qlinear_gemm; "使瓦片大小与专家负载相匹配", tile
 * choice against row count).  At such M qlinear_gemm gives each CU a single
 * workgroup whose K steps form one dependent chain; here every workgroup
 * holds two copies of its tile's waves that take the two halves of K side
 * by side, and adds the halves' fp32 sums at the end.  For the caller to
 * pick (like qlinear_gemm_few_rows): up to about 10% faster than
 * qlinear_gemm for a few hundred rows (the gain varies with the board and
 * can vanish), slower for a thousand rows and more.
 *   X fp16 [M][K], Y fp16 [M][N]; fp16 dequantized weights; each output is
 *   (fp32 sum over the first K/2) + (fp32 sum over the second K/2), rounded
 *   once to fp16: deterministic, and row m of Y is bit-identical whatever M
 *   is, but its rounding differs from qlinear_gemm's (which does not split K).
 * Limits: K a multiple of 128.
 * Errors: as qlinear_gemm; UNSUPPORTED_SHAPE for other K.
 */
int qlinear_gemm_ksplit(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/*
 * qlinear_gemv_bf16, qlinear_gemm_bf16 - the same two layers with bf16
 * activations, scales, biases and outputs ([PPLX] dequantization section:
 * the page's checkpoint keeps scale and bias in bf16 and its matrix path
 * multiplies bf16 operands).  W's scales and biases hold bf16 bit patterns
 * (same [N][K/64] layout); x / X and y / Y are bf16, row-major.
 * Accumulation is in fp32; outputs are rounded to bf16, nearest even.  The
 * GEMV multiplies the exact codes (v_dot2 on bf16 pairs); the GEMM rounds
 * each dequantized weight scale*code + bias once to bf16 for the MFMA.
 * qlinear_gemm_bf16 keeps qlinear_gemm's tile table and its row invariance.
 * Limits: qlinear_gemv_bf16 takes K a power of two from 256 to 16384.
 * Errors: as qlinear_gemv / qlinear_gemm; UNSUPPORTED_SHAPE for another K
 * in qlinear_gemv_bf16.
 */
int qlinear_gemv_bf16(const ql_w4* W, const uint16_t* x, uint16_t* y, void* stream);
int qlinear_gemm_bf16(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/*
 * Second weight codecs ("待验证｜lithos-metal补Apple推理内核", section
 * "一分钟内合并了什么": FP8 E4M3 decode, two codes per half2, and an NVFP4
 * checkpoint).  The formats are this library's reading of that page:
 *
 *   ql_fp8:   codes  uint8 [N][K], E4M3FN (bias 7, S.1111.111 = NaN, max 448)
 *             scales fp16 [N][K/64];  W[k][n] = e4m3(code[n][k]) * scale[n][k/64]
 *   ql_nvfp4: qweight uint32 [N][K/8], E2M1 codes packed as the w4 codes
 *             (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6, sign in bit 3)
 *             block_scales uint8 [N][K/16], E4M3;  global_scale fp32
 *             W[k][n] = e2m1(code) * e4m3(block_scale[n][k/16]) * global_scale
 */
typedef struct ql_fp8 {
    const uint8_t* codes;    /* [N][K], 16-byte aligned */
    const uint16_t* scales;  /* [N][K/64] fp16 */
    int32_t K;
    int32_t N;
} ql_fp8;

/* num_experts FP8 matrices of the same shape stacked contiguously. */
typedef struct ql_fp8_experts {
    const uint8_t* codes;    /* [E][N][K], 16-byte aligned */
    const uint16_t* scales;  /* [E][N][K/64] fp16 */
    int32_t K;
    int32_t N;
    int32_t num_experts;
} ql_fp8_experts;

typedef struct ql_nvfp4 {
    const uint32_t* qweight;      /* [N][K/8], 16-byte aligned */
    const uint8_t* block_scales;  /* [N][K/16] E4M3, 2-byte aligned */
    float global_scale;
    int32_t K;
    int32_t N;
} ql_nvfp4;

/* num_experts NVFP4 matrices of the same shape stacked contiguously, each
 * with a global scale of its own. */
typedef struct ql_nvfp4_experts {
    const uint32_t* qweight;       /* [E][N][K/8], 16-byte aligned */
    const uint8_t* block_scales;   /* [E][N][K/16] E4M3, 4-byte aligned */
    const float* global_scales;    /* [E] fp32 in device memory, finite */
    int32_t K;
    int32_t N;
    int32_t num_experts;
} ql_nvfp4_experts;

/*
 * qlinear_gemv_fp8, qlinear_gemv_nvfp4 - y fp16 [N] = x fp16 [K] . W for
 * one activation row.  Two codes at a time are converted to an fp16 pair of
 * their exact values (the FP8 "two codes per half2"), multiplied in fp32
 * with v_dot2, scaled per group / block in fp32 and rounded once to fp16.
 * An E4M3 code S.1111.111 (weight code or NVFP4 block scale) is NaN, as the
 * format defines, and makes the outputs of its row NaN.
 * Limits: K a power of two, 256 .. 8192 (FP8) or 256 .. 16384 (NVFP4).
 * Errors: INVALID_ARG (null W/x/y with N > 0, N < 0), UNSUPPORTED_SHAPE,
 * MISALIGNED (codes/qweight and x 16-byte, scales, block_scales and y
 * 2-byte aligned), HIP.
 */
int qlinear_gemv_fp8(const ql_fp8* W, const uint16_t* x, uint16_t* y, void* stream);
int qlinear_gemv_nvfp4(const ql_nvfp4* W, const uint16_t* x, uint16_t* y, void* stream);

/*
 * qlinear_gemm_fp8 - Y fp16 [M][N] = X fp16 [M][K] . W for FP8-E4M3 weights,
 * the prefill counterpart of qlinear_gemv_fp8 ([PPLX] dequantization section:
 * small weight tiles dequantized into on-chip memory for the matrix path).
 * The MFMA tiles of qlinear_gemm (same shape table, same row invariance:
 * row m's bits do not depend on M) with each staged weight
 * fp16(e4m3(code) * scale): the code converts exactly to fp16 and one fp16
 * multiply rounds the product once (any finite fp16 scale; a NaN code gives a
 * NaN weight).  Staged weights are fp16: a product above 65504 in magnitude
 * becomes infinite and one below 2^-14 is held on fp16's subnormal grid.
 * fp32 accumulation, fp16 output.
 * Limits: K a positive multiple of 64, K <= QL_MAX_K.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, MISALIGNED (codes and X 16-byte,
 * scales and Y 2-byte aligned), HIP.
 */
int qlinear_gemm_fp8(const ql_fp8* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/*
 * qlinear_gemm_nvfp4 - Y fp16 [M][N] = X fp16 [M][K] . W for NVFP4 weights,
 * the prefill counterpart of qlinear_gemv_nvfp4: the MFMA tiles of
 * qlinear_gemm (same shape table and row invariance) with each staged weight
 * fp16(e2m1 * (e4m3(block scale) * global_scale)): the block scale and the
 * product are formed in fp32 (the e2m1 and e4m3 values are exact) and
 * rounded once to fp16, with the fp16 range of qlinear_gemm_fp8's staged
 * weights; a NaN block scale gives NaN weights.  fp32 accumulation, fp16
 * output.
 * Limits: K a positive multiple of 64, K <= QL_MAX_K; global_scale finite.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, MISALIGNED (qweight and X 16-byte,
 * block_scales 4-byte, Y 2-byte aligned), HIP.
 */
int qlinear_gemm_nvfp4(const ql_nvfp4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream);

/*
 * qlinear_gemv_rmsnorm - y = fp16(rmsnorm(x)) . dequant(W): a decode
 * projection with its normalization fused in front ([PPLX] "减少中间状态和流量":
 * the decode chains keep intermediates in registers, normalization among
 * the fused steps).  u[k] = x[k] / sqrt(mean(x^2) + eps) * gamma[k] is
 * computed in fp32 inside the GEMV (every block derives the same sum of
 * squares) and rounded to fp16 once, where an unfused path would store it;
 * the projection then reads that row.  The norm's RMS form is this
 * library's reading of the page.
 *   W  K x N w4;  x, gamma  fp16 [K];  eps  >= 0, finite;  y  fp16 [N].
 * Limits: K a power of two from 256 to 16384.
 * Errors: as qlinear_gemv; INVALID_ARG for a null gamma or a bad eps;
 * UNSUPPORTED_SHAPE for other K; MISALIGNED (x, gamma 16-byte aligned).
 */
int qlinear_gemv_rmsnorm(const ql_w4* W, const uint16_t* x, const uint16_t* gamma, float eps,
                         uint16_t* y, void* stream);

/*
 * qlinear_gemv_argmax_workspace_bytes - device workspace of
 * qlinear_gemv_argmax for N outputs: 8 * ceil(N / 8) bytes (0 for N <= 0).
 */
size_t qlinear_gemv_argmax_workspace_bytes(int64_t N);

/*
 * qlinear_gemv_argmax - the vocabulary head with the token choice on the
 * GPU ([PPLX] "将 token 交接保留在 GPU 上": the step ends by picking the
 * highest-scoring token and the GPU writes its id straight into the next
 * step's input slot, with no round trip through the host).
 *   logits = x . dequant(W) as in qlinear_gemv; *token = the index of the
 *   largest fp32 logit (before rounding to fp16), the smallest index among
 *   equal largest values.  NaN logits are never chosen; if no logit is
 *   comparable the token is 0.  The result is always in [0, N).
 *   W  K x N w4 (N >= 1);  x  fp16 [K];  logits  fp16 [N] output or NULL;
 *   token  int32 device slot (4-byte aligned), written by the GPU;
 *   workspace  device memory of qlinear_gemv_argmax_workspace_bytes(N)
 *   bytes, 8-byte aligned, no initialization needed, must not be shared by
 *   calls that may run concurrently.  Two launches on the stream.
 * Limits: K a power of two from 256 to 16384.
 * Errors: INVALID_ARG (null W, x or token, N < 1), UNSUPPORTED_SHAPE,
 * MISALIGNED, WORKSPACE, HIP.
 */
int qlinear_gemv_argmax(const ql_w4* W, const uint16_t* x, uint16_t* logits, int32_t* token,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * qlinear_embed_token - the next step's input row from the token slot:
 * x = fp16(dequant(E)[*token]), row *token of a w4 embedding table read on
 * the GPU ([PPLX] token hand-off section: the next step starts from the
 * chosen token; the table in the w4 layout above, one output per token, is
 * this library's reading).  Each value is rounded once (scale*code + bias).
 *   E  w4 table with K = hidden width, N = number of tokens;  token  int32
 *   device slot;  x  fp16 [K] output (16-byte aligned).  An id outside
 *   [0, N) yields a row of zeros and reads no table memory.
 * Errors: INVALID_ARG (null E, token or x with K > 0, N < 1),
 * UNSUPPORTED_SHAPE (as qlinear_gemv), MISALIGNED, HIP.
 */
int qlinear_embed_token(const ql_w4* E, const int32_t* token, uint16_t* x, void* stream);

/*
 * moe_workspace_bytes - bytes of device workspace that moe_route and
 * moe_dispatch need for T tokens, E experts, top-k; 0 on invalid input.
 *
 * The workspace needs no initialization; it may be reused by any sequence
 * of calls and sizes that fit it.
 *
 * Workspace layout (offsets in bytes; readable by the caller after the
 * stream has completed):
 *   [0, 4)     int32 num_tiles   number of valid entries of the tile map
 *   [4, 8)     int32 tile_rows   = QL_MOE_TILE_ROWS (height of a short tile)
 *   [8, 12)    int32 error flag  nonzero if the ids violated the contract of
 *                                 moe_dispatch (out of range or repeated)
 *   [12, 16)   int32 num_tall    tall tiles, listed first in the map
 *   [16, 32)   reserved
 *   [32, ...)  int32 tiles[max_tiles][4] = {expert, first row, rows, height},
 *              max_tiles = (T*topk)/QL_MOE_TILE_ROWS + E.
 *              Load-matched map ([PPLX] "使瓦片大小与专家负载相匹配"): an
 *              expert's rows are cut into tall tiles of 2*QL_MOE_TILE_ROWS
 *              rows while a full one remains, the rest into short tiles of
 *              at most QL_MOE_TILE_ROWS rows; all tall tiles come first
 *              (experts ascending), then all short tiles.  height is the
 *              tile height (rows <= height).
 *   then, at ql_moe_logits_offset(T, E, topk): float logits[T][E] (router
 *   logits incl. bias, written by moe_route only)
 *   then internal scratch.
 */
size_t moe_workspace_bytes(int32_t T, int32_t E, int32_t topk);
size_t ql_moe_logits_offset(int32_t T, int32_t E, int32_t topk);

/*
 * moe_route - on-GPU router and dispatch with no host round trip.
 * [PPLX] "Qwen 创建了三种不同的工作负载形状": score E experts per token and keep
 * topk; reading taken: softmax over all E logits, keep the topk largest
 * (ties toward the lower expert index), renormalize them to sum 1; an
 * optional per-expert logit bias is added to the logits.  Then [PPLX]
 * "将专家路由保留在 GPU 上": histogram, prefix scan, stable scatter of the
 * assignments a = t*topk + j into expert groups, and the tile map.
 *   H            fp16 [T][D] tokens
 *   Wr           fp16 [D][E] router weight
 *   logit_bias   fp32 [E] or NULL
 *   topk_ids     int32 [T][topk] out: chosen experts, by descending gate
 *   topk_gates   fp32  [T][topk] out: renormalized gates (descending)
 *   counts       int32 [E] out: assignments per expert
 *   offsets      int32 [E+1] out: exclusive prefix sum of counts
 *   sorted_assign int32 [T*topk] out: assignments grouped by expert,
 *                ascending a inside each expert
 *   assign_pos   int32 [T*topk] out: inverse of sorted_assign
 *   workspace    device buffer of ws_bytes >= moe_workspace_bytes(T,E,topk)
 * Logits are accumulated in fp32.  Limits: 1 <= topk <= min(E,
 * QL_MAX_TOPK), E <= QL_MAX_EXPERTS, D a positive multiple of 64.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, MISALIGNED, WORKSPACE, HIP.
 */
int moe_route(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
              int32_t T, int32_t D, int32_t E, int32_t topk,
              int32_t* topk_ids, float* topk_gates,
              int32_t* counts, int32_t* offsets,
              int32_t* sorted_assign, int32_t* assign_pos,
              void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_dispatch - the dispatch half of moe_route for ids chosen elsewhere:
 * histogram, prefix scan, stable scatter and tile map ([PPLX]
 * "将专家路由保留在 GPU 上").  topk_ids int32 [T][topk]: the ids of one token
 * must be distinct and in [0, E).  Ids that break this are skipped and set
 * the workspace error flag; the outputs are then unspecified but every
 * write stays in bounds.  Other arguments as moe_route.
 */
int moe_dispatch(const int32_t* topk_ids, int32_t T, int32_t E, int32_t topk,
                 int32_t* counts, int32_t* offsets,
                 int32_t* sorted_assign, int32_t* assign_pos,
                 void* workspace, size_t ws_bytes, void* stream);

/*
 * moe_grouped_gemm - the expert projections over routed rows, ragged per
 * expert, fed by the dispatch outputs on the device.
 * [PPLX] dequantization section (fused-dequant grouped GEMM), "使瓦片大小与专
 * 家负载相匹配" (tiles over each expert's rows) and "减少中间状态和流量"
 * (gate+up fused with the gated activation; down fused with the routing
 * weights and the shared expert).
 *
 * Rows: routed row r in [0, T*topk) is assignment sorted_assign[r] of
 * token sorted_assign[r] / topk, multiplied by expert e with offsets[e] <=
 * r < offsets[e+1]; if `shared` is not NULL, rows [T*topk, T*topk + T)
 * are the T tokens in order, multiplied by the shared expert.
 *
 *   op = QL_OP_GATE_UP_SILU: W is [E] x (K = D, N = 2I), X = H fp16 [T][D];
 *        Y fp16 [rows][I] = SiLU(u[:, :I]) * u[:, I:], u = X[token] . W_e.
 *   op = QL_OP_DOWN: W is [E] x (K = I, N = D), X = act fp16 [rows][I] in
 *        row order; Y fp16 [rows][D].
 *   op = QL_OP_DOWN_COMBINE (T <= QL_DECODE_MAX_T): as QL_OP_DOWN, but
 *        Y fp16 [T][D] = sum_j topk_gates[t][j] * (row assign_pos[t*topk+j])
 *        (+ the shared row of t), accumulated in fp32 in a fixed order, so
 *        repeated calls give identical bits: the rows j = 0..topk-1 and the
 *        shared row (j = topk) are dealt to four groups by j mod 4; within a
 *        group, for each K slice over its rows in ascending j, then across
 *        K slices; then the four group sums in group order.
 * topk_gates and assign_pos are read only by QL_OP_DOWN_COMBINE (may be
 * NULL otherwise).  `workspace` is the one filled by moe_route or
 * moe_dispatch for the same T, E, topk.
 *
 * Splitting the layer across two streams: the shared expert does not
 * depend on the routing, so it can run beside it.  A call with shared =
 * NULL computes the routed rows only; a call with op | QL_OP_SHARED_ONLY
 * (QL_OP_GATE_UP_SILU or QL_OP_DOWN, shared not NULL) computes the shared
 * rows [T*topk, T*topk + T) of Y only and reads neither the experts of W
 * (W still gives K, N and E), nor offsets, sorted_assign or the workspace,
 * which may then be NULL / 0.  The two calls together write exactly the
 * rows, and the bits, of the one call with both; they touch disjoint rows
 * of X and Y, so they may run concurrently on different streams.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, MISALIGNED, WORKSPACE, HIP.
 */
int moe_grouped_gemm(const ql_w4_experts* W, const ql_w4* shared,
                     const uint16_t* X, int32_t T, int32_t topk, int32_t op,
                     const int32_t* offsets, const int32_t* sorted_assign,
                     const float* topk_gates, const int32_t* assign_pos,
                     const void* workspace, size_t ws_bytes,
                     uint16_t* Y, void* stream);

/*
 * moe_combine - out[t] = sum_j topk_gates[t][j] * Ydown[assign_pos[t*topk+j]]
 * (+ Ydown[T*topk + t] if has_shared), fp32 in the order j = 0..topk-1 then
 * shared, rounded to fp16.  [PPLX] "减少中间状态和流量" (routing scores and the
 * shared expert's result applied to the expert outputs).  Deterministic: no
 * atomics.
 *   Ydown fp16 [T*topk (+T)][N];  out fp16 [T][N].
 * Errors: INVALID_ARG, MISALIGNED, HIP.
 */
int moe_combine(const uint16_t* Ydown, const float* topk_gates, const int32_t* assign_pos,
                int32_t T, int32_t topk, int32_t N, int32_t has_shared,
                uint16_t* out, void* stream);

/*
 * bf16 variant of the routed-expert layer (prefill and any T): [PPLX]
 * dequantization section - the page's checkpoint keeps scales and biases in
 * bf16 and its matrix path multiplies bf16 operands.  Same layouts, rows,
 * workspace and determinism as the fp16 calls above, with every 16-bit
 * array holding bf16 patterns: H and the router weight Wr (moe_route_bf16;
 * logits still accumulated in fp32), X, the experts' scales and biases and
 * Y (moe_grouped_gemm_bf16: W and shared point at bf16 scales/biases; the
 * dequantized weight is bf16(s*q + b), one rounding, and the products run
 * on v_mfma_f32_32x32x16_bf16 with fp32 accumulation; act = SiLU(gate) * up
 * rounded to bf16), Ydown and out (moe_combine_bf16).  moe_grouped_gemm_bf16
 * serves QL_OP_GATE_UP_SILU and QL_OP_DOWN for every T on the tiled path;
 * QL_OP_DOWN_COMBINE returns UNSUPPORTED_SHAPE.
 * Errors: as the fp16 calls.
 */
int moe_route_bf16(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
                   int32_t T, int32_t D, int32_t E, int32_t topk,
                   int32_t* topk_ids, float* topk_gates,
                   int32_t* counts, int32_t* offsets,
                   int32_t* sorted_assign, int32_t* assign_pos,
                   void* workspace, size_t ws_bytes, void* stream);
int moe_grouped_gemm_bf16(const ql_w4_experts* W, const ql_w4* shared,
                          const uint16_t* X, int32_t T, int32_t topk, int32_t op,
                          const int32_t* offsets, const int32_t* sorted_assign,
                          const void* workspace, size_t ws_bytes,
                          uint16_t* Y, void* stream);
int moe_combine_bf16(const uint16_t* Ydown, const float* topk_gates, const int32_t* assign_pos,
                     int32_t T, int32_t topk, int32_t N, int32_t has_shared,
                     uint16_t* out, void* stream);

/*
 * moe_grouped_gemm_fp8 - moe_grouped_gemm with FP8-E4M3 experts (the
 * ql_fp8 format of qlinear_gemm_fp8, stacked over experts; "待验证｜lithos-
 * metal补Apple推理内核", section "一分钟内合并了什么": FP8 weight decode).
 * Same rows, workspace, tile map and fp16 X / Y as moe_grouped_gemm; each
 * staged weight is fp16(e4m3(code) * scale), one rounding (as in
 * qlinear_gemm_fp8, with its fp16 range), fp32 accumulation on the MFMA tiles, act = SiLU(gate) * up rounded
 * to fp16.  Ops, rows, QL_OP_SHARED_ONLY and the arguments as
 * moe_grouped_gemm.  For T <= QL_DECODE_MAX_T and K a power of two in
 * 64 .. 16384 the rows run on the row-parallel decode kernels, which dot
 * exact fp16 code values with the activations in fp32 (v_dot2) and apply
 * each scale to its group's fp32 partial sum, as qlinear_gemv_fp8 does;
 * QL_OP_DOWN_COMBINE (the gate-weighted sum of moe_grouped_gemm) needs that
 * path.  `shared` (may be NULL) has the shape of one expert.  Limits: K a
 * positive multiple of 64, K <= QL_MAX_K.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, MISALIGNED (codes and X 16-byte,
 * scales and Y 2-byte aligned), WORKSPACE, HIP.
 */
int moe_grouped_gemm_fp8(const ql_fp8_experts* W, const ql_fp8* shared,
                         const uint16_t* X, int32_t T, int32_t topk, int32_t op,
                         const int32_t* offsets, const int32_t* sorted_assign,
                         const float* topk_gates, const int32_t* assign_pos,
                         const void* workspace, size_t ws_bytes,
                         uint16_t* Y, void* stream);

/*
 * moe_grouped_gemm_nvfp4 - moe_grouped_gemm with NVFP4 experts (the
 * ql_nvfp4 format of qlinear_gemm_nvfp4, stacked over experts, a global
 * scale per expert read from device memory; the same page and section as
 * the FP8 call).  Same rows, workspace, tile map, fp16 X / Y and ops as
 * moe_grouped_gemm_fp8; each staged weight is fp16(e2m1 * (e4m3(block
 * scale) * global scale)), formed in fp32 and rounded once, as in
 * qlinear_gemm_nvfp4; on the row-parallel decode path (as for the FP8
 * call) the block scales multiply fp32 partial sums of 16 codes and the
 * global scale the row's total, as in qlinear_gemv_nvfp4.  `shared` (may be
 * NULL; host global_scale, finite) has the shape of one expert.
 * Limits: K a positive multiple of 64, K <= QL_MAX_K.
 * Errors: INVALID_ARG (incl. a non-finite shared global scale),
 * UNSUPPORTED_SHAPE, MISALIGNED (qweight and X 16-byte, block_scales and
 * global_scales 4-byte, Y 2-byte aligned), WORKSPACE, HIP.
 */
int moe_grouped_gemm_nvfp4(const ql_nvfp4_experts* W, const ql_nvfp4* shared,
                           const uint16_t* X, int32_t T, int32_t topk, int32_t op,
                           const int32_t* offsets, const int32_t* sorted_assign,
                           const float* topk_gates, const int32_t* assign_pos,
                           const void* workspace, size_t ws_bytes,
                           uint16_t* Y, void* stream);

/*
 * moe_decode - the whole routed-expert layer for a few decode tokens in
 * three launches: router partial sums; the token's top-k fused into the
 * gate/up rows (each routed workgroup finishes its token's logits, takes
 * the top-k and then reads only its chosen expert's weights); the down rows
 * fused with the gate-weighted sum and the shared expert.
 * [PPLX] "减少中间状态和流量" (the decode step fuses routing scores and the
 * shared expert into the expert projections) and section "解码：最小化每个 token 移动的字节数" (decode
 * reads only the chosen experts' weights).
 *   H            fp16 [T][D] tokens, 1 <= T <= QL_DECODE_MAX_T
 *   Wr           fp16 [D][E] router weight;  logit_bias fp32 [E] or NULL
 *   gate_up      [E] x (K = D, N = 2I) experts (gate columns [0, I), up [I, 2I))
 *   down         [E] x (K = I, N = D) experts
 *   shared_gate_up, shared_down: the shared expert, both or neither (NULL)
 *   topk_ids     int32 [T][topk] out;  topk_gates fp32 [T][topk] out
 *   out          fp16 [T][D] out
 *   workspace    device buffer of ws_bytes >= moe_decode_workspace_bytes(T, E, topk, I)
 * Routing is bit-identical to moe_route on the same inputs (same partial
 * sums in the same order, same selection); the layer output is the one of
 * moe_route + moe_grouped_gemm(QL_OP_GATE_UP_SILU) +
 * moe_grouped_gemm(QL_OP_DOWN_COMBINE), bit for bit.  The workspace holds,
 * at moe_decode_logits_offset(T, E, topk), the fp32 logits [T][E].
 * Limits: D and I powers of two in 64 .. 16384, D a multiple of 64,
 * (topk + 1) * I * 2 <= 49152, 1 <= topk <= min(E, QL_MAX_TOPK),
 * E <= QL_MAX_EXPERTS.
 * Errors: INVALID_ARG, UNSUPPORTED_SHAPE, MISALIGNED, WORKSPACE, HIP.
 */
size_t moe_decode_workspace_bytes(int32_t T, int32_t E, int32_t topk, int32_t I);
size_t moe_decode_logits_offset(int32_t T, int32_t E, int32_t topk);
int moe_decode(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
               int32_t T, int32_t D, int32_t E, int32_t topk,
               const ql_w4_experts* gate_up, const ql_w4_experts* down,
               const ql_w4* shared_gate_up, const ql_w4* shared_down,
               int32_t* topk_ids, float* topk_gates,
               void* workspace, size_t ws_bytes, uint16_t* out, void* stream);
/*
 * moe_decode_bf16 - moe_decode with bf16 H, Wr, expert scales and biases and
 * out (the bf16 layer of moe_route_bf16 and friends): codes enter the row
 * dot products exactly (v_dot2_f32_bf16 against bf16 128 + q), scale and
 * bias are applied in fp32, act is rounded to bf16.  Same limits, workspace
 * and errors as moe_decode.
 */
int moe_decode_bf16(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
                    int32_t T, int32_t D, int32_t E, int32_t topk,
                    const ql_w4_experts* gate_up, const ql_w4_experts* down,
                    const ql_w4* shared_gate_up, const ql_w4* shared_down,
                    int32_t* topk_ids, float* topk_gates,
                    void* workspace, size_t ws_bytes, uint16_t* out, void* stream);

/*
 * moe_decode_fp8, moe_decode_nvfp4 - moe_decode with FP8-E4M3 or NVFP4
 * experts (the ql_fp8 / ql_nvfp4 formats, stacked; "待验证｜lithos-metal补
 * Apple推理内核", section "一分钟内合并了什么") and fp16 H, Wr, out.  The same
 * three launches, routing and fixed summation orders as moe_decode; the
 * rows dot exact fp16 code values with the activations in fp32 (v_dot2) and
 * apply the FP8 group scale, or the NVFP4 block scale and then the
 * expert's global scale, to fp32 partial sums (qlinear_gemv_fp8 /
 * qlinear_gemv_nvfp4); act = SiLU(gate) * up rounded once to fp16.  The
 * output is that of moe_route + moe_grouped_gemm_fp8 / _nvfp4
 * (QL_OP_GATE_UP_SILU, then QL_OP_DOWN_COMBINE), bit for bit.  Same
 * limits, workspace and errors as moe_decode (MISALIGNED also for the
 * codec alignment rules of moe_grouped_gemm_fp8 / _nvfp4).
 */
int moe_decode_fp8(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
                   int32_t T, int32_t D, int32_t E, int32_t topk,
                   const ql_fp8_experts* gate_up, const ql_fp8_experts* down,
                   const ql_fp8* shared_gate_up, const ql_fp8* shared_down,
                   int32_t* topk_ids, float* topk_gates,
                   void* workspace, size_t ws_bytes, uint16_t* out, void* stream);
int moe_decode_nvfp4(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
                     int32_t T, int32_t D, int32_t E, int32_t topk,
                     const ql_nvfp4_experts* gate_up, const ql_nvfp4_experts* down,
                     const ql_nvfp4* shared_gate_up, const ql_nvfp4* shared_down,
                     int32_t* topk_ids, float* topk_gates,
                     void* workspace, size_t ws_bytes, uint16_t* out, void* stream);

/*
 * moe_decode_noalloc - moe_decode for callers that cannot allocate device
 * memory or pass a workspace (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The same three launches, the
 * same kernels and the same results, bit for bit, as moe_decode; instead
 * of the caller's workspace they use a device array of
 * QL_DECODE_SCRATCH_BYTES that the library owns (one copy per GPU, held
 * until the process ends).  It allocates nothing: the first call on a
 * device only looks up that device's copy of the array.
 *   Arguments as moe_decode without workspace and ws_bytes.  The scratch
 *   needs no initialization.  Calls that may overlap on one GPU (several
 *   streams or threads) race on the shared scratch and must be serialized
 *   by the caller; calls on different GPUs do not interact.  The logits of
 *   the last call stay in the scratch and are not exposed.
 * Limits: as moe_decode, and moe_decode_workspace_bytes(T, E, topk, I) <=
 * QL_DECODE_SCRATCH_BYTES (every shape within moe_decode's limits fits).
 * Errors: as moe_decode; WORKSPACE if the scratch is too small; HIP if the
 * array cannot be resolved on the current device.
 */
int moe_decode_noalloc(const uint16_t* H, const uint16_t* Wr, const float* logit_bias,
                       int32_t T, int32_t D, int32_t E, int32_t topk,
                       const ql_w4_experts* gate_up, const ql_w4_experts* down,
                       const ql_w4* shared_gate_up, const ql_w4* shared_down,
                       int32_t* topk_ids, float* topk_gates, uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QLINEAR_H */
