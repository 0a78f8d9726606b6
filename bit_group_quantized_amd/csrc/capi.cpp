// C ABI of the library: argument validation on the host, then asynchronous
// launches on the caller's stream.  See include/qlinear.h for the contract
// of every entry point.
#include <cmath>
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "ql_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Shape and pointer checks of one w4 matrix; N == 0 is allowed.
int check_w4(const uint32_t* qw, const uint16_t* sc, const uint16_t* bi, int32_t K, int32_t N,
             int32_t gs) {
    if (N < 0 || K < 0) return QL_ERR_INVALID_ARG;
    if (gs != QL_GROUP_SIZE) return QL_ERR_UNSUPPORTED_SHAPE;
    if (K == 0 || K % QL_GROUP_SIZE != 0 || K > QL_MAX_K) return QL_ERR_UNSUPPORTED_SHAPE;
    if (N == 0) return QL_OK;
    if (!qw || !sc || !bi) return QL_ERR_INVALID_ARG;
    if (!aligned(qw, 16) || !aligned(sc, 2) || !aligned(bi, 2)) return QL_ERR_MISALIGNED;
    return QL_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

}  // namespace

extern "C" {

int ql_layout_version(void) { return QL_LAYOUT_VERSION; }

const char* ql_status_string(int status) {
    switch (status) {
        case QL_OK: return "ok";
        case QL_ERR_INVALID_ARG: return "invalid argument";
        case QL_ERR_UNSUPPORTED_SHAPE: return "unsupported shape";
        case QL_ERR_MISALIGNED: return "misaligned pointer";
        case QL_ERR_WORKSPACE: return "workspace missing or too small";
        case QL_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

int qlinear_pack(const uint8_t* codes, int32_t N, int32_t K, uint32_t* qweight, void* stream) {
    if (N < 0 || K < 0) return QL_ERR_INVALID_ARG;
    if (K % 8 != 0) return QL_ERR_UNSUPPORTED_SHAPE;
    if (N == 0 || K == 0) return QL_OK;
    if (!codes || !qweight) return QL_ERR_INVALID_ARG;
    if (!aligned(codes, 16) || !aligned(qweight, 16)) return QL_ERR_MISALIGNED;
    return ql::launch_pack(codes, N, K, qweight, as_stream(stream));
}

int qlinear_gemv(const ql_w4* W, const uint16_t* x, uint16_t* y, void* stream) {
    if (!W) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (W->N == 0) return QL_OK;
    if (!x || !y) return QL_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 2)) return QL_ERR_MISALIGNED;
    ql::GemvArgs a{W->qweight, W->scales, W->biases, x, y, W->K, W->N};
    return ql::launch_gemv(a, as_stream(stream));
}

int qlinear_gemv_multi(const ql_w4* Ws, int32_t count, const uint16_t* x, uint16_t* const* ys,
                       void* stream) {
    if (!Ws || !ys || count < 1 || count > QL_GEMV_MULTI_MAX) return QL_ERR_INVALID_ARG;
    ql::GemvMultiArgs a{};
    a.count = count;
    a.K = Ws[0].K;
    a.x = x;
    bool any = false;
    for (int i = 0; i < count; ++i) {
        const ql_w4& W = Ws[i];
        const int rc = check_w4(W.qweight, W.scales, W.biases, W.K, W.N, W.group_size);
        if (rc != QL_OK) return rc;
        if (W.K != a.K) return QL_ERR_INVALID_ARG;
        if (W.N > 0) {
            if (!ys[i]) return QL_ERR_INVALID_ARG;
            if (!aligned(ys[i], 2)) return QL_ERR_MISALIGNED;
            any = true;
        }
        a.qweight[i] = W.qweight;
        a.scales[i] = W.scales;
        a.biases[i] = W.biases;
        a.y[i] = ys[i];
        a.N[i] = W.N;
    }
    if (!ql::gemv_fused_supported(a.K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!any) return QL_OK;
    if (!x) return QL_ERR_INVALID_ARG;
    if (!aligned(x, 16)) return QL_ERR_MISALIGNED;
    return ql::launch_gemv_multi(a, as_stream(stream));
}

int qlinear_gemm(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream) {
    if (!W || M < 0) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (W->N == 0 || M == 0) return QL_OK;
    if (M > (int64_t)0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 2)) return QL_ERR_MISALIGNED;
    ql::GemmArgs a{W->qweight, W->scales, W->biases, X, Y, M, W->K, W->N};
    return ql::launch_gemm(a, as_stream(stream));
}

int qlinear_gemm_few_rows(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y,
                          void* stream) {
    if (!W || M < 0) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (!ql::gemm_ws_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N == 0 || M == 0) return QL_OK;
    if (M > (int64_t)0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 2)) return QL_ERR_MISALIGNED;
    ql::GemmArgs a{W->qweight, W->scales, W->biases, X, Y, M, W->K, W->N};
    return ql::launch_gemm_ws(a, as_stream(stream));
}

int qlinear_gemm_ksplit(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream) {
    if (!W || M < 0) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (!ql::gemm_ksplit_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N == 0 || M == 0) return QL_OK;
    if (M > (int64_t)0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 2)) return QL_ERR_MISALIGNED;
    ql::GemmArgs a{W->qweight, W->scales, W->biases, X, Y, M, W->K, W->N};
    return ql::launch_gemm_ksplit(a, as_stream(stream));
}

int qlinear_gemv_rmsnorm(const ql_w4* W, const uint16_t* x, const uint16_t* gamma, float eps,
                         uint16_t* y, void* stream) {
    if (!W) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (!ql::gemv_fused_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!(eps >= 0.f) || !std::isfinite(eps)) return QL_ERR_INVALID_ARG;
    if (W->N == 0) return QL_OK;
    if (!x || !gamma || !y) return QL_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(y, 2)) return QL_ERR_MISALIGNED;
    ql::GemvArgs a{W->qweight, W->scales, W->biases, x, y, W->K, W->N};
    a.gamma = gamma;
    a.eps = eps;
    return ql::launch_gemv_rmsnorm(a, as_stream(stream));
}

size_t qlinear_gemv_argmax_workspace_bytes(int64_t N) {
    if (N <= 0 || N > 0x7fffffff) return 0;
    return (size_t)((N + 7) / 8) * 8;
}

int qlinear_gemv_argmax(const ql_w4* W, const uint16_t* x, uint16_t* logits, int32_t* token,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (!W) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (!ql::gemv_fused_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N < 1 || !x || !token) return QL_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(token, 4) || (logits && !aligned(logits, 2)))
        return QL_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < qlinear_gemv_argmax_workspace_bytes(W->N))
        return QL_ERR_WORKSPACE;
    if (!aligned(workspace, 8)) return QL_ERR_MISALIGNED;
    ql::GemvArgs a{W->qweight, W->scales, W->biases, x, logits, W->K, W->N};
    a.partials = static_cast<uint64_t*>(workspace);
    a.token = token;
    return ql::launch_gemv_argmax(a, as_stream(stream));
}

int qlinear_embed_token(const ql_w4* E, const int32_t* token, uint16_t* x, void* stream) {
    if (!E) return QL_ERR_INVALID_ARG;
    int rc = check_w4(E->qweight, E->scales, E->biases, E->K, E->N, E->group_size);
    if (rc != QL_OK) return rc;
    if (E->N < 1 || !token || !x) return QL_ERR_INVALID_ARG;
    if (!aligned(token, 4) || !aligned(x, 16)) return QL_ERR_MISALIGNED;
    ql::GemvArgs a{E->qweight, E->scales, E->biases, nullptr, x, E->K, E->N};
    a.token = const_cast<int32_t*>(token);
    return ql::launch_embed(a, as_stream(stream));
}

int qlinear_gemv_bf16(const ql_w4* W, const uint16_t* x, uint16_t* y, void* stream) {
    if (!W) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (!ql::gemv_fused_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N == 0) return QL_OK;
    if (!x || !y) return QL_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(y, 2)) return QL_ERR_MISALIGNED;
    ql::GemvArgs a{W->qweight, W->scales, W->biases, x, y, W->K, W->N};
    return ql::launch_gemv_bf16(a, as_stream(stream));
}

int qlinear_gemm_bf16(const ql_w4* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream) {
    if (!W || M < 0) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (W->N == 0 || M == 0) return QL_OK;
    if (M > (int64_t)0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 2)) return QL_ERR_MISALIGNED;
    ql::GemmArgs a{W->qweight, W->scales, W->biases, X, Y, M, W->K, W->N};
    return ql::launch_gemm_bf16(a, as_stream(stream));
}

int qlinear_gemv_fp8(const ql_fp8* W, const uint16_t* x, uint16_t* y, void* stream) {
    if (!W || W->N < 0 || W->K < 0) return QL_ERR_INVALID_ARG;
    if (!ql::gemv_fp8_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N == 0) return QL_OK;
    if (!W->codes || !W->scales || !x || !y) return QL_ERR_INVALID_ARG;
    if (!aligned(W->codes, 16) || !aligned(W->scales, 2) || !aligned(x, 16) || !aligned(y, 2))
        return QL_ERR_MISALIGNED;
    ql::CodecArgs a;
    a.codes8 = W->codes;
    a.scales = W->scales;
    a.x = x;
    a.y = y;
    a.K = W->K;
    a.N = W->N;
    return ql::launch_gemv_fp8(a, as_stream(stream));
}

int qlinear_gemm_fp8(const ql_fp8* W, const uint16_t* X, int64_t M, uint16_t* Y, void* stream) {
    if (!W || W->N < 0 || W->K < 0 || M < 0) return QL_ERR_INVALID_ARG;
    if (W->K == 0 || W->K % QL_GROUP_SIZE != 0 || W->K > QL_MAX_K) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N == 0 || M == 0) return QL_OK;
    if (M > (int64_t)0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!W->codes || !W->scales || !X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(W->codes, 16) || !aligned(W->scales, 2) || !aligned(X, 16) || !aligned(Y, 2))
        return QL_ERR_MISALIGNED;
    ql::GemmArgs a{reinterpret_cast<const uint32_t*>(W->codes), W->scales, nullptr, X, Y, M, W->K,
                   W->N};
    return ql::launch_gemm_fp8(a, as_stream(stream));
}

int qlinear_gemm_nvfp4(const ql_nvfp4* W, const uint16_t* X, int64_t M, uint16_t* Y,
                       void* stream) {
    if (!W || W->N < 0 || W->K < 0 || M < 0) return QL_ERR_INVALID_ARG;
    if (W->K == 0 || W->K % QL_GROUP_SIZE != 0 || W->K > QL_MAX_K) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!std::isfinite(W->global_scale)) return QL_ERR_INVALID_ARG;
    if (W->N == 0 || M == 0) return QL_OK;
    if (M > (int64_t)0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!W->qweight || !W->block_scales || !X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(W->qweight, 16) || !aligned(W->block_scales, 4) || !aligned(X, 16) || !aligned(Y, 2))
        return QL_ERR_MISALIGNED;
    ql::GemmArgs a{W->qweight, reinterpret_cast<const uint16_t*>(W->block_scales), nullptr, X, Y, M,
                   W->K, W->N, W->global_scale};
    return ql::launch_gemm_nvfp4(a, as_stream(stream));
}

int qlinear_gemv_nvfp4(const ql_nvfp4* W, const uint16_t* x, uint16_t* y, void* stream) {
    if (!W || W->N < 0 || W->K < 0) return QL_ERR_INVALID_ARG;
    if (!ql::gemv_nvfp4_supported(W->K)) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N == 0) return QL_OK;
    if (!W->qweight || !W->block_scales || !x || !y) return QL_ERR_INVALID_ARG;
    if (!aligned(W->qweight, 16) || !aligned(W->block_scales, 2) || !aligned(x, 16) || !aligned(y, 2))
        return QL_ERR_MISALIGNED;
    ql::CodecArgs a;
    a.codes4 = W->qweight;
    a.block_scales = W->block_scales;
    a.global_scale = W->global_scale;
    a.x = x;
    a.y = y;
    a.K = W->K;
    a.N = W->N;
    return ql::launch_gemv_nvfp4(a, as_stream(stream));
}

size_t moe_workspace_bytes(int32_t T, int32_t E, int32_t topk) {
    if (T < 0 || E <= 0 || E > QL_MAX_EXPERTS || topk <= 0 || topk > E || topk > QL_MAX_TOPK)
        return 0;
    return ql::moe_workspace_layout(T, E, topk).total;
}

size_t ql_moe_logits_offset(int32_t T, int32_t E, int32_t topk) {
    if (moe_workspace_bytes(T, E, topk) == 0) return 0;
    return ql::moe_workspace_layout(T, E, topk).logits;
}

static int check_route_common(int32_t T, int32_t E, int32_t topk, const int32_t* counts,
                              const int32_t* offsets, const int32_t* sorted_assign,
                              const int32_t* assign_pos, const void* workspace, size_t ws_bytes) {
    if (T < 0 || E <= 0 || topk <= 0) return QL_ERR_INVALID_ARG;
    if (topk > E) return QL_ERR_INVALID_ARG;
    if (E > QL_MAX_EXPERTS || topk > QL_MAX_TOPK) return QL_ERR_UNSUPPORTED_SHAPE;
    if ((int64_t)T * topk > 0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!counts || !offsets) return QL_ERR_INVALID_ARG;
    if (T > 0 && (!sorted_assign || !assign_pos)) return QL_ERR_INVALID_ARG;
    if (!aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_assign, 4) ||
        !aligned(assign_pos, 4))
        return QL_ERR_MISALIGNED;
    if (!workspace || ws_bytes < moe_workspace_bytes(T, E, topk)) return QL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QL_ERR_MISALIGNED;
    return QL_OK;
}

static int route_impl(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T,
                      int32_t D, int32_t E, int32_t topk, int32_t* topk_ids, float* topk_gates,
                      int32_t* counts, int32_t* offsets, int32_t* sorted_assign,
                      int32_t* assign_pos, void* workspace, size_t ws_bytes, void* stream, bool bf16) {
    int rc = check_route_common(T, E, topk, counts, offsets, sorted_assign, assign_pos, workspace,
                                ws_bytes);
    if (rc != QL_OK) return rc;
    if (D <= 0) return QL_ERR_INVALID_ARG;
    if (D % QL_GROUP_SIZE != 0 || D > QL_MAX_K) return QL_ERR_UNSUPPORTED_SHAPE;
    if (T > 0 && (!H || !Wr || !topk_ids || !topk_gates)) return QL_ERR_INVALID_ARG;
    if (!aligned(H, 16) || !aligned(Wr, 16) || !aligned(logit_bias, 4) || !aligned(topk_ids, 4) ||
        !aligned(topk_gates, 4))
        return QL_ERR_MISALIGNED;
    ql::RouteArgs a{H, Wr, logit_bias, T, D, E, topk, topk_ids, topk_gates, counts, offsets,
                    sorted_assign, assign_pos, static_cast<unsigned char*>(workspace), bf16};
    if (T == 0) return ql::launch_dispatch(a, as_stream(stream));  // counts = 0, offsets = 0
    return ql::launch_route(a, as_stream(stream));
}

int moe_route(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T, int32_t D,
              int32_t E, int32_t topk, int32_t* topk_ids, float* topk_gates, int32_t* counts,
              int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, void* workspace,
              size_t ws_bytes, void* stream) {
    return route_impl(H, Wr, logit_bias, T, D, E, topk, topk_ids, topk_gates, counts, offsets,
                      sorted_assign, assign_pos, workspace, ws_bytes, stream, false);
}

int moe_route_bf16(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T,
                   int32_t D, int32_t E, int32_t topk, int32_t* topk_ids, float* topk_gates,
                   int32_t* counts, int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos,
                   void* workspace, size_t ws_bytes, void* stream) {
    return route_impl(H, Wr, logit_bias, T, D, E, topk, topk_ids, topk_gates, counts, offsets,
                      sorted_assign, assign_pos, workspace, ws_bytes, stream, true);
}

int moe_dispatch(const int32_t* topk_ids, int32_t T, int32_t E, int32_t topk, int32_t* counts,
                 int32_t* offsets, int32_t* sorted_assign, int32_t* assign_pos, void* workspace,
                 size_t ws_bytes, void* stream) {
    int rc = check_route_common(T, E, topk, counts, offsets, sorted_assign, assign_pos, workspace,
                                ws_bytes);
    if (rc != QL_OK) return rc;
    if (T > 0 && !topk_ids) return QL_ERR_INVALID_ARG;
    if (!aligned(topk_ids, 4)) return QL_ERR_MISALIGNED;
    ql::RouteArgs a{nullptr, nullptr, nullptr, T, 0, E, topk, const_cast<int32_t*>(topk_ids),
                    nullptr, counts, offsets, sorted_assign, assign_pos,
                    static_cast<unsigned char*>(workspace)};
    return ql::launch_dispatch(a, as_stream(stream));
}

// Expert weights of a grouped call, already checked for format and layout.
struct ExpertView {
    const uint32_t* qw;
    const uint16_t* sc;
    const uint16_t* bi;
    const uint32_t* sqw;  // shared expert or null
    const uint16_t* ssc;
    const uint16_t* sbi;
    int32_t K, N, E;
    bool bf16;
    int wf;  // 0 = w4, 1 = FP8, 2 = NVFP4
    const float* gscales = nullptr;  // NVFP4: per-expert global scales (device)
    float sgscale = 0.f;             // NVFP4: the shared expert's global scale
};

static int w4_view(const ql_w4_experts* W, const ql_w4* shared, bool bf16, ExpertView& v) {
    if (!W) return QL_ERR_INVALID_ARG;
    int rc = check_w4(W->qweight, W->scales, W->biases, W->K, W->N, W->group_size);
    if (rc != QL_OK) return rc;
    if (shared) {
        rc = check_w4(shared->qweight, shared->scales, shared->biases, shared->K, shared->N,
                      shared->group_size);
        if (rc != QL_OK) return rc;
        if (shared->K != W->K || shared->N != W->N) return QL_ERR_INVALID_ARG;
    }
    v = ExpertView{W->qweight, W->scales, W->biases,
                   shared ? shared->qweight : nullptr,
                   shared ? shared->scales : nullptr,
                   shared ? shared->biases : nullptr,
                   W->K, W->N, W->num_experts, bf16, 0};
    return QL_OK;
}

static int check_fp8(const uint8_t* codes, const uint16_t* scales, int32_t K, int32_t N) {
    if (N < 0 || K < 0) return QL_ERR_INVALID_ARG;
    if (K == 0 || K % QL_GROUP_SIZE != 0 || K > QL_MAX_K) return QL_ERR_UNSUPPORTED_SHAPE;
    if (N == 0) return QL_OK;
    if (!codes || !scales) return QL_ERR_INVALID_ARG;
    if (!aligned(codes, 16) || !aligned(scales, 2)) return QL_ERR_MISALIGNED;
    return QL_OK;
}

static int grouped_impl(const ExpertView& w, const uint16_t* X, int32_t T, int32_t topk, int32_t op,
                        const int32_t* offsets, const int32_t* sorted_assign,
                        const float* topk_gates, const int32_t* assign_pos, const void* workspace,
                        size_t ws_bytes, uint16_t* Y, void* stream) {
    const bool shared_only = (op & QL_OP_SHARED_ONLY) != 0;
    op &= ~QL_OP_SHARED_ONLY;
    if (op != QL_OP_GATE_UP_SILU && op != QL_OP_DOWN && op != QL_OP_DOWN_COMBINE)
        return QL_ERR_INVALID_ARG;
    if (shared_only && (op == QL_OP_DOWN_COMBINE || !w.sqw)) return QL_ERR_INVALID_ARG;
    const int32_t E = w.E;
    if (T < 0 || E <= 0 || topk <= 0 || topk > E) return QL_ERR_INVALID_ARG;
    if (E > QL_MAX_EXPERTS || topk > QL_MAX_TOPK) return QL_ERR_UNSUPPORTED_SHAPE;
    if (op == QL_OP_GATE_UP_SILU && w.N % 2 != 0) return QL_ERR_UNSUPPORTED_SHAPE;
    if (T == 0 || w.N == 0) return QL_OK;
    if ((int64_t)T * topk > 0x7fffffff / 2) return QL_ERR_UNSUPPORTED_SHAPE;
    if (!X || !Y) return QL_ERR_INVALID_ARG;
    if (!aligned(X, 16) || !aligned(Y, 2)) return QL_ERR_MISALIGNED;
    if (shared_only) {
        ql::GroupedArgs a{w.qw, w.sc, w.bi, w.sqw, w.ssc, w.sbi,
                          X, nullptr, nullptr, nullptr, nullptr, nullptr, Y,
                          w.K, w.N, E, T, topk, op, w.bf16, w.wf, w.gscales, w.sgscale};
        a.shared_only = true;
        return ql::launch_moe_grouped(a, as_stream(stream));
    }
    if (!offsets || !sorted_assign) return QL_ERR_INVALID_ARG;
    if (!aligned(offsets, 4) || !aligned(sorted_assign, 4)) return QL_ERR_MISALIGNED;
    if (!workspace || ws_bytes < moe_workspace_bytes(T, E, topk)) return QL_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return QL_ERR_MISALIGNED;

    // The row-parallel decode kernels take fp16 activations (w4, FP8 or
    // NVFP4 weights); the bf16 layer runs every T on the tiled path.
    const bool rows_path = !w.bf16 && T <= QL_DECODE_MAX_T && ql::moe_rows_supported(w.K);
    if (op == QL_OP_DOWN_COMBINE) {
        if (!rows_path) return QL_ERR_UNSUPPORTED_SHAPE;
        if (!topk_gates || !assign_pos) return QL_ERR_INVALID_ARG;
        if (!aligned(topk_gates, 4) || !aligned(assign_pos, 4)) return QL_ERR_MISALIGNED;
        const int J = topk + (w.sqw ? 1 : 0);
        if ((int64_t)J * w.K * 2 > 49152) return QL_ERR_UNSUPPORTED_SHAPE;
    }
    ql::GroupedArgs a{w.qw, w.sc, w.bi, w.sqw, w.ssc, w.sbi,
                      X, offsets, sorted_assign, topk_gates, assign_pos,
                      static_cast<const unsigned char*>(workspace), Y,
                      w.K, w.N, E, T, topk, op, w.bf16, w.wf, w.gscales, w.sgscale};
    if (rows_path) return ql::launch_moe_rows(a, as_stream(stream));
    return ql::launch_moe_grouped(a, as_stream(stream));
}

int moe_grouped_gemm(const ql_w4_experts* W, const ql_w4* shared, const uint16_t* X, int32_t T,
                     int32_t topk, int32_t op, const int32_t* offsets,
                     const int32_t* sorted_assign, const float* topk_gates,
                     const int32_t* assign_pos, const void* workspace, size_t ws_bytes,
                     uint16_t* Y, void* stream) {
    ExpertView v;
    if (const int rc = w4_view(W, shared, false, v)) return rc;
    return grouped_impl(v, X, T, topk, op, offsets, sorted_assign, topk_gates, assign_pos,
                        workspace, ws_bytes, Y, stream);
}

int moe_grouped_gemm_bf16(const ql_w4_experts* W, const ql_w4* shared, const uint16_t* X,
                          int32_t T, int32_t topk, int32_t op, const int32_t* offsets,
                          const int32_t* sorted_assign, const void* workspace, size_t ws_bytes,
                          uint16_t* Y, void* stream) {
    ExpertView v;
    if (const int rc = w4_view(W, shared, true, v)) return rc;
    if (op == QL_OP_DOWN_COMBINE) return QL_ERR_UNSUPPORTED_SHAPE;
    return grouped_impl(v, X, T, topk, op, offsets, sorted_assign, nullptr, nullptr,
                        workspace, ws_bytes, Y, stream);
}

static int fp8_view(const ql_fp8_experts* W, const ql_fp8* shared, ExpertView& v) {
    if (!W) return QL_ERR_INVALID_ARG;
    int rc = check_fp8(W->codes, W->scales, W->K, W->N);
    if (rc != QL_OK) return rc;
    if (shared) {
        rc = check_fp8(shared->codes, shared->scales, shared->K, shared->N);
        if (rc != QL_OK) return rc;
        if (shared->K != W->K || shared->N != W->N) return QL_ERR_INVALID_ARG;
    }
    v = ExpertView{reinterpret_cast<const uint32_t*>(W->codes), W->scales, nullptr,
                   shared ? reinterpret_cast<const uint32_t*>(shared->codes) : nullptr,
                   shared ? shared->scales : nullptr, nullptr,
                   W->K, W->N, W->num_experts, false, 1};
    return QL_OK;
}

static int nvfp4_view(const ql_nvfp4_experts* W, const ql_nvfp4* shared, ExpertView& v) {
    if (!W || W->N < 0 || W->K < 0) return QL_ERR_INVALID_ARG;
    if (W->K == 0 || W->K % QL_GROUP_SIZE != 0 || W->K > QL_MAX_K) return QL_ERR_UNSUPPORTED_SHAPE;
    if (W->N > 0) {
        if (!W->qweight || !W->block_scales || !W->global_scales) return QL_ERR_INVALID_ARG;
        if (!aligned(W->qweight, 16) || !aligned(W->block_scales, 4) || !aligned(W->global_scales, 4))
            return QL_ERR_MISALIGNED;
    }
    if (shared) {
        if (shared->K != W->K || shared->N != W->N) return QL_ERR_INVALID_ARG;
        if (!std::isfinite(shared->global_scale)) return QL_ERR_INVALID_ARG;
        if (W->N > 0) {
            if (!shared->qweight || !shared->block_scales) return QL_ERR_INVALID_ARG;
            if (!aligned(shared->qweight, 16) || !aligned(shared->block_scales, 4)) return QL_ERR_MISALIGNED;
        }
    }
    v = ExpertView{W->qweight, reinterpret_cast<const uint16_t*>(W->block_scales), nullptr,
                   shared ? shared->qweight : nullptr,
                   shared ? reinterpret_cast<const uint16_t*>(shared->block_scales) : nullptr, nullptr,
                   W->K, W->N, W->num_experts, false, 2};
    v.gscales = W->global_scales;
    v.sgscale = shared ? shared->global_scale : 0.f;
    return QL_OK;
}

int moe_grouped_gemm_fp8(const ql_fp8_experts* W, const ql_fp8* shared, const uint16_t* X,
                         int32_t T, int32_t topk, int32_t op, const int32_t* offsets,
                         const int32_t* sorted_assign, const float* topk_gates,
                         const int32_t* assign_pos, const void* workspace, size_t ws_bytes,
                         uint16_t* Y, void* stream) {
    ExpertView v;
    if (const int rc = fp8_view(W, shared, v)) return rc;
    return grouped_impl(v, X, T, topk, op, offsets, sorted_assign, topk_gates, assign_pos, workspace,
                        ws_bytes, Y, stream);
}

int moe_grouped_gemm_nvfp4(const ql_nvfp4_experts* W, const ql_nvfp4* shared, const uint16_t* X,
                           int32_t T, int32_t topk, int32_t op, const int32_t* offsets,
                           const int32_t* sorted_assign, const float* topk_gates,
                           const int32_t* assign_pos, const void* workspace, size_t ws_bytes,
                           uint16_t* Y, void* stream) {
    ExpertView v;
    if (const int rc = nvfp4_view(W, shared, v)) return rc;
    return grouped_impl(v, X, T, topk, op, offsets, sorted_assign, topk_gates, assign_pos, workspace,
                        ws_bytes, Y, stream);
}

size_t moe_decode_workspace_bytes(int32_t T, int32_t E, int32_t topk, int32_t I) {
    if (T < 0 || T > QL_DECODE_MAX_T || E <= 0 || E > QL_MAX_EXPERTS || topk <= 0 || topk > E ||
        topk > QL_MAX_TOPK || I <= 0 || I > QL_MAX_K)
        return 0;
    return ql::moe_decode_layout(T, E, topk, I).total;
}

size_t moe_decode_logits_offset(int32_t T, int32_t E, int32_t topk) {
    if (moe_decode_workspace_bytes(T, E, topk, 64) == 0) return 0;
    return ql::moe_decode_layout(T, E, topk, 64).logits;
}

// The whole decode layer for two expert views (gate/up and down, each with
// its shared matrix or none).  ws_mode 0: the caller's workspace; 1: the
// library's scratch array (moe_decode_noalloc), checked against
// QL_DECODE_SCRATCH_BYTES.
static int decode_run(const ExpertView& gu, const ExpertView& dn, bool has_shared, const uint16_t* H,
                      const uint16_t* Wr, const float* logit_bias, int32_t T, int32_t D, int32_t E,
                      int32_t topk, int32_t* topk_ids, float* topk_gates, void* workspace,
                      size_t ws_bytes, uint16_t* out, void* stream, int ws_mode) {
    if (T < 0 || E <= 0 || topk <= 0 || topk > E || D <= 0) return QL_ERR_INVALID_ARG;
    if (T > QL_DECODE_MAX_T || E > QL_MAX_EXPERTS || topk > QL_MAX_TOPK) return QL_ERR_UNSUPPORTED_SHAPE;
    if (gu.E != E || dn.E != E) return QL_ERR_INVALID_ARG;
    const int32_t I = dn.K;
    if (gu.K != D || dn.N != D || gu.N != 2 * I) return QL_ERR_INVALID_ARG;
    if (!ql::moe_rows_supported(D) || !ql::moe_rows_supported(I)) return QL_ERR_UNSUPPORTED_SHAPE;
    const int J = topk + (has_shared ? 1 : 0);
    if ((int64_t)J * I * 2 > 49152) return QL_ERR_UNSUPPORTED_SHAPE;
    if (T == 0) return QL_OK;
    if (!H || !Wr || !topk_ids || !topk_gates || !out) return QL_ERR_INVALID_ARG;
    if (!aligned(H, 16) || !aligned(Wr, 16) || !aligned(logit_bias, 4) || !aligned(topk_ids, 4) ||
        !aligned(topk_gates, 4) || !aligned(out, 2))
        return QL_ERR_MISALIGNED;
    if (ws_mode == 1) {
        if (moe_decode_workspace_bytes(T, E, topk, I) > QL_DECODE_SCRATCH_BYTES) return QL_ERR_WORKSPACE;
        unsigned char* p = nullptr;
        if (const int rc2 = ql::decode_scratch(&p)) return rc2;
        workspace = p;
    } else {
        if (!workspace || ws_bytes < moe_decode_workspace_bytes(T, E, topk, I)) return QL_ERR_WORKSPACE;
        if (!aligned(workspace, 256)) return QL_ERR_MISALIGNED;
    }
    ql::DecodeArgs a{H, Wr, logit_bias, T, D, E, topk, I,
                     gu.qw, gu.sc, gu.bi, dn.qw, dn.sc, dn.bi,
                     has_shared ? gu.sqw : nullptr, has_shared ? gu.ssc : nullptr,
                     has_shared ? gu.sbi : nullptr, has_shared ? dn.sqw : nullptr,
                     has_shared ? dn.ssc : nullptr, has_shared ? dn.sbi : nullptr,
                     topk_ids, topk_gates, static_cast<unsigned char*>(workspace), out, gu.bf16};
    a.wf = gu.wf;
    a.gu_gscales = gu.gscales;
    a.dn_gscales = dn.gscales;
    a.sgu_gscale = gu.sgscale;
    a.sdn_gscale = dn.sgscale;
    return ql::launch_moe_decode(a, as_stream(stream));
}

static int decode_impl(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T,
                       int32_t D, int32_t E, int32_t topk, const ql_w4_experts* gate_up,
                       const ql_w4_experts* down, const ql_w4* shared_gate_up,
                       const ql_w4* shared_down, int32_t* topk_ids, float* topk_gates,
                       void* workspace, size_t ws_bytes, uint16_t* out, void* stream, bool bf16,
                       int ws_mode = 0) {
    if (!gate_up || !down) return QL_ERR_INVALID_ARG;
    if ((shared_gate_up == nullptr) != (shared_down == nullptr)) return QL_ERR_INVALID_ARG;
    ExpertView gu, dn;
    if (const int rc = w4_view(gate_up, shared_gate_up, bf16, gu)) return rc;
    if (const int rc = w4_view(down, shared_down, bf16, dn)) return rc;
    return decode_run(gu, dn, shared_gate_up != nullptr, H, Wr, logit_bias, T, D, E, topk, topk_ids,
                      topk_gates, workspace, ws_bytes, out, stream, ws_mode);
}

int moe_decode(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T, int32_t D,
               int32_t E, int32_t topk, const ql_w4_experts* gate_up, const ql_w4_experts* down,
               const ql_w4* shared_gate_up, const ql_w4* shared_down, int32_t* topk_ids,
               float* topk_gates, void* workspace, size_t ws_bytes, uint16_t* out, void* stream) {
    return decode_impl(H, Wr, logit_bias, T, D, E, topk, gate_up, down, shared_gate_up, shared_down,
                       topk_ids, topk_gates, workspace, ws_bytes, out, stream, false);
}

int moe_decode_bf16(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T,
                    int32_t D, int32_t E, int32_t topk, const ql_w4_experts* gate_up,
                    const ql_w4_experts* down, const ql_w4* shared_gate_up,
                    const ql_w4* shared_down, int32_t* topk_ids, float* topk_gates,
                    void* workspace, size_t ws_bytes, uint16_t* out, void* stream) {
    return decode_impl(H, Wr, logit_bias, T, D, E, topk, gate_up, down, shared_gate_up, shared_down,
                       topk_ids, topk_gates, workspace, ws_bytes, out, stream, true);
}

int moe_decode_fp8(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T, int32_t D,
                   int32_t E, int32_t topk, const ql_fp8_experts* gate_up, const ql_fp8_experts* down,
                   const ql_fp8* shared_gate_up, const ql_fp8* shared_down, int32_t* topk_ids,
                   float* topk_gates, void* workspace, size_t ws_bytes, uint16_t* out, void* stream) {
    if (!gate_up || !down) return QL_ERR_INVALID_ARG;
    if ((shared_gate_up == nullptr) != (shared_down == nullptr)) return QL_ERR_INVALID_ARG;
    ExpertView gu, dn;
    if (const int rc = fp8_view(gate_up, shared_gate_up, gu)) return rc;
    if (const int rc = fp8_view(down, shared_down, dn)) return rc;
    return decode_run(gu, dn, shared_gate_up != nullptr, H, Wr, logit_bias, T, D, E, topk, topk_ids,
                      topk_gates, workspace, ws_bytes, out, stream, 0);
}

int moe_decode_nvfp4(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T,
                     int32_t D, int32_t E, int32_t topk, const ql_nvfp4_experts* gate_up,
                     const ql_nvfp4_experts* down, const ql_nvfp4* shared_gate_up,
                     const ql_nvfp4* shared_down, int32_t* topk_ids, float* topk_gates, void* workspace,
                     size_t ws_bytes, uint16_t* out, void* stream) {
    if (!gate_up || !down) return QL_ERR_INVALID_ARG;
    if ((shared_gate_up == nullptr) != (shared_down == nullptr)) return QL_ERR_INVALID_ARG;
    ExpertView gu, dn;
    if (const int rc = nvfp4_view(gate_up, shared_gate_up, gu)) return rc;
    if (const int rc = nvfp4_view(down, shared_down, dn)) return rc;
    return decode_run(gu, dn, shared_gate_up != nullptr, H, Wr, logit_bias, T, D, E, topk, topk_ids,
                      topk_gates, workspace, ws_bytes, out, stream, 0);
}

int moe_decode_noalloc(const uint16_t* H, const uint16_t* Wr, const float* logit_bias, int32_t T,
                       int32_t D, int32_t E, int32_t topk, const ql_w4_experts* gate_up,
                       const ql_w4_experts* down, const ql_w4* shared_gate_up,
                       const ql_w4* shared_down, int32_t* topk_ids, float* topk_gates,
                       uint16_t* out, void* stream) {
    return decode_impl(H, Wr, logit_bias, T, D, E, topk, gate_up, down, shared_gate_up, shared_down,
                       topk_ids, topk_gates, nullptr, 0, out, stream, false, 1);
}

static int combine_impl(const uint16_t* Ydown, const float* topk_gates, const int32_t* assign_pos,
                        int32_t T, int32_t topk, int32_t N, int32_t has_shared, uint16_t* out,
                        void* stream, bool bf16) {
    if (T < 0 || N < 0 || topk <= 0) return QL_ERR_INVALID_ARG;
    if (topk > QL_MAX_TOPK) return QL_ERR_UNSUPPORTED_SHAPE;
    if (T == 0 || N == 0) return QL_OK;
    if (!Ydown || !topk_gates || !assign_pos || !out) return QL_ERR_INVALID_ARG;
    const uintptr_t va = (N % 8 == 0) ? 16 : 2;
    if (!aligned(Ydown, va) || !aligned(out, va) || !aligned(topk_gates, 4) ||
        !aligned(assign_pos, 4))
        return QL_ERR_MISALIGNED;
    return ql::launch_combine(Ydown, topk_gates, assign_pos, T, topk, N, has_shared ? 1 : 0, out,
                              as_stream(stream), bf16);
}

int moe_combine(const uint16_t* Ydown, const float* topk_gates, const int32_t* assign_pos,
                int32_t T, int32_t topk, int32_t N, int32_t has_shared, uint16_t* out,
                void* stream) {
    return combine_impl(Ydown, topk_gates, assign_pos, T, topk, N, has_shared, out, stream, false);
}

int moe_combine_bf16(const uint16_t* Ydown, const float* topk_gates, const int32_t* assign_pos,
                     int32_t T, int32_t topk, int32_t N, int32_t has_shared, uint16_t* out,
                     void* stream) {
    return combine_impl(Ydown, topk_gates, assign_pos, T, topk, N, has_shared, out, stream, true);
}

}  // extern "C"
