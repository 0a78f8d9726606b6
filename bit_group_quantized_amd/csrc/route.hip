// On-GPU router and dispatch for the routed-expert layer.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon":
//  * Qwen 创建了三种不同的工作负载形状 - the router scores E experts per token
//    and keeps 8.  Reading taken for the gates: softmax over all logits, keep
//    the top-k, renormalize; this equals a softmax over the k chosen logits,
//    and the choice is the k largest logits (ties toward the lower index).
//  * 将专家路由保留在 GPU 上 - histogram of assignments per expert, prefix scan
//    to start offsets, scatter of rows into expert groups, and a block map of
//    fixed-size tiles for the grouped GEMM; the whole sequence stays on the
//    GPU with no host pause.
//  * 使瓦片大小与专家负载相匹配 - tiles are cut per expert.
//
// Determinism: the scatter is stable (ascending a = t*topk + j inside an
// expert) and never depends on the order of atomic operations: per chunk of
// 256 tokens a bit mask per expert marks which tokens chose it (an atomic OR,
// whose result does not depend on order), and the rank of a token inside
// its expert is a population count of the mask below it.
#include "ql_device.h"
#include "ql_internal.h"

#include <float.h>

namespace ql {

namespace {

constexpr int kChunk = kRouteChunkTokens;
constexpr int kMaskWords = kChunk / 32;
constexpr int kRouterParts = 32;

__device__ __forceinline__ bool better(float v, int e, float bv, int be) {
    return v > bv || (v == bv && e < be);
}

// Inclusive scan of one int per thread across a block of up to 1024 threads.
__device__ int block_inclusive_scan(int v, int* s_tmp /* >= 16 ints */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int nw = (blockDim.x + 63) >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int o = __shfl_up(v, off, 64);
        if (lane >= off) v += o;
    }
    if (lane == 63) s_tmp[wave] = v;
    __syncthreads();
    int base = 0;
    for (int w = 0; w < wave; ++w) base += s_tmp[w];
    (void)nw;
    __syncthreads();
    return v + base;
}

// ---------------------------------------------------------------------------
// Small-T router: partial logits over D/32-row slices, summed by the top-k
// step in a fixed order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256)
router_partial_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wr,
                      float* __restrict__ partials, int D, int E) {
    __shared__ float hs[QL_MAX_K / kRouterParts];
    const int t = blockIdx.y, p = blockIdx.x;
    const int rows = D / kRouterParts;
    const int d0 = p * rows;
    for (int i = threadIdx.x; i < rows; i += blockDim.x) hs[i] = h2f(H[(size_t)t * D + d0 + i]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float acc = 0.f;
        for (int d = 0; d < rows; ++d) acc += hs[d] * h2f(Wr[(size_t)(d0 + d) * E + e]);
        partials[((size_t)t * kRouterParts + p) * E + e] = acc;
    }
}

// ---------------------------------------------------------------------------
// Top-k of one token by one wave.  Logits are the sum of `nparts` partial
// rows (fixed order) plus the optional bias; they are written back to
// `logits_out`.  Lane j < topk ends up holding choice j.
// ---------------------------------------------------------------------------
template <int EPL>
__device__ void topk_one_token(const float* __restrict__ src, int nparts,
                               const float* __restrict__ bias, float* __restrict__ logits_out,
                               int t, int E, int topk, int* sel_e, float* sel_g) {
    const int lane = threadIdx.x & 63;
    float v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        float s = -INFINITY;
        if (e < E) {
            s = 0.f;
            for (int p = 0; p < nparts; ++p) s += src[((size_t)t * nparts + p) * E + e];
            if (bias) s += bias[e];
            logits_out[(size_t)t * E + e] = s;
            if (s != s) s = -INFINITY;  // NaN never wins
        }
        v[i] = s;
    }
    uint32_t taken = 0;
    float my_v = 0.f;
    int my_e = 0;
    float vmax = 0.f;
    for (int j = 0; j < topk; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane + 64 * i;
            if (e < E && !((taken >> i) & 1u) && better(v[i], e, bv, be)) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off, 64);
            const int oe = __shfl_xor(be, off, 64);
            if (better(ov, oe, bv, be)) {
                bv = ov;
                be = oe;
            }
        }
        // be < E always: topk <= E and every lane saw every untaken expert.
        if ((be & 63) == lane) taken |= 1u << (be >> 6);
        if (j == 0) vmax = bv;
        if (lane == j) {
            my_v = bv;
            my_e = be;
        }
    }
    float ex = (lane < topk) ? __expf(my_v - vmax) : 0.f;
    float sum = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) sum += __shfl_xor(sum, off, 64);
    if (lane < topk) {
        sel_e[lane] = my_e;
        sel_g[lane] = ex / sum;
    }
}

template <int EPL>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ src, int nparts, const float* __restrict__ bias,
            float* __restrict__ logits_out, int T, int E, int topk,
            int* __restrict__ ids, float* __restrict__ gates) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave leaves together
    topk_one_token<EPL>(src, nparts, bias, logits_out, t, E, topk, ids + (size_t)t * topk,
                        gates + (size_t)t * topk);
}

// ---------------------------------------------------------------------------
// Dispatch for many tokens: per-chunk masks and counts, one scan block, and
// the stable scatter.
// ---------------------------------------------------------------------------
__device__ int build_chunk_masks(const int* __restrict__ ids, int T, int E, int topk, int c,
                                 uint32_t* mask) {
    for (int i = threadIdx.x; i < E * kMaskWords; i += blockDim.x) mask[i] = 0u;
    __syncthreads();
    const int tl = threadIdx.x;
    const int t = c * kChunk + tl;
    int err = 0;
    if (t < T) {
        const uint32_t bit = 1u << (tl & 31);
        for (int j = 0; j < topk; ++j) {
            const int e = ids[(size_t)t * topk + j];
            if ((unsigned)e >= (unsigned)E) {
                err = 1;
                continue;
            }
            const uint32_t old = atomicOr(&mask[e * kMaskWords + (tl >> 5)], bit);
            if (old & bit) err = 1;
        }
    }
    __syncthreads();
    return err;
}

__global__ void __launch_bounds__(kChunk)
dispatch_count_kernel(const int* __restrict__ ids, int T, int E, int topk,
                      int* __restrict__ chunk_counts, int* __restrict__ chunk_err) {
    extern __shared__ uint32_t mask[];
    const int c = blockIdx.x;
    const int err = build_chunk_masks(ids, T, E, topk, c, mask);
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) cnt += __popc(mask[e * kMaskWords + w]);
        chunk_counts[(size_t)c * E + e] = cnt;
    }
    const int any = __syncthreads_or(err);
    if (threadIdx.x == 0) chunk_err[c] = any;
}

__global__ void __launch_bounds__(1024)
dispatch_scan_kernel(int* __restrict__ chunk_counts, const int* __restrict__ chunk_err,
                     int nchunks, int E, int* __restrict__ counts, int* __restrict__ offsets,
                     int* __restrict__ ws_header, int* __restrict__ tiles) {
    __shared__ int s_tmp[16];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        for (int c = 0; c < nchunks; ++c) {
            const int v = chunk_counts[(size_t)c * E + e];
            chunk_counts[(size_t)c * E + e] = run;  // becomes the chunk's base inside e
            run += v;
        }
        counts[e] = run;
    }
    const int cnt = (e < E) ? run : 0;
    const int incl = block_inclusive_scan(cnt, s_tmp);
    const int excl = incl - cnt;
    if (e < E) offsets[e] = excl;
    if (e == E - 1) offsets[E] = incl;
    const int nt = (cnt + QL_MOE_TILE_ROWS - 1) / QL_MOE_TILE_ROWS;
    const int tincl = block_inclusive_scan(nt, s_tmp);
    const int ts = tincl - nt;
    for (int j = 0; j < nt; ++j) {
        int* tp = tiles + (size_t)(ts + j) * 4;
        tp[0] = e;
        tp[1] = excl + j * QL_MOE_TILE_ROWS;
        tp[2] = min(QL_MOE_TILE_ROWS, cnt - j * QL_MOE_TILE_ROWS);
        tp[3] = 0;
    }
    int err = 0;
    for (int c = e; c < nchunks; c += blockDim.x) err |= chunk_err[c];
    const int any = __syncthreads_or(err);
    if (e == E - 1) ws_header[0] = tincl;
    if (e == 0) {
        ws_header[1] = QL_MOE_TILE_ROWS;
        ws_header[2] = any;
        ws_header[3] = 0;
    }
}

__global__ void __launch_bounds__(kChunk)
dispatch_scatter_kernel(const int* __restrict__ ids, int T, int E, int topk,
                        const int* __restrict__ offsets, const int* __restrict__ chunk_base,
                        int* __restrict__ sorted_assign, int* __restrict__ pos) {
    extern __shared__ uint32_t mask[];
    const int c = blockIdx.x;
    build_chunk_masks(ids, T, E, topk, c, mask);
    const int tl = threadIdx.x;
    const int t = c * kChunk + tl;
    if (t >= T) return;
    const int w = tl >> 5;
    const uint32_t below = (1u << (tl & 31)) - 1u;
    for (int j = 0; j < topk; ++j) {
        const int a = t * topk + j;
        const int e = ids[a];
        if ((unsigned)e >= (unsigned)E) {
            pos[a] = -1;
            continue;
        }
        int rank = __popc(mask[e * kMaskWords + w] & below);
        for (int ww = 0; ww < w; ++ww) rank += __popc(mask[e * kMaskWords + ww]);
        const int r = offsets[e] + chunk_base[(size_t)c * E + e] + rank;
        sorted_assign[r] = a;
        pos[a] = r;
    }
}

// ---------------------------------------------------------------------------
// Small T (decode): top-k and the whole dispatch in one block.
// ---------------------------------------------------------------------------
template <int EPL, bool DO_TOPK>
__global__ void __launch_bounds__(256)
route_small_kernel(const float* __restrict__ partials, int nparts, const float* __restrict__ bias,
                   float* __restrict__ logits_out, int T, int E, int topk,
                   int* __restrict__ ids, float* __restrict__ gates, int* __restrict__ counts,
                   int* __restrict__ offsets, int* __restrict__ sorted_assign,
                   int* __restrict__ pos, int* __restrict__ ws_header, int* __restrict__ tiles) {
    __shared__ int s_ids[kRouterSmallT * QL_MAX_TOPK_DEV];
    __shared__ float s_gates[kRouterSmallT * QL_MAX_TOPK_DEV];
    __shared__ int s_cnt[QL_MAX_EXPERTS_DEV];
    __shared__ int s_off[QL_MAX_EXPERTS_DEV + 1];
    __shared__ int s_tmp[16];
    const int wave = threadIdx.x >> 6;
    const int nass = T * topk;
    if constexpr (DO_TOPK) {
        for (int t = wave; t < T; t += 4)
            topk_one_token<EPL>(partials, nparts, bias, logits_out, t, E, topk, s_ids + t * topk,
                                s_gates + t * topk);
        __syncthreads();
        for (int a = threadIdx.x; a < nass; a += blockDim.x) {
            ids[a] = s_ids[a];
            gates[a] = s_gates[a];
        }
    } else {
        for (int a = threadIdx.x; a < nass; a += blockDim.x) s_ids[a] = ids[a];
    }
    int err = 0;
    for (int a = threadIdx.x; a < nass; a += blockDim.x)
        if ((unsigned)s_ids[a] >= (unsigned)E) err = 1;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_cnt[e] = 0;
    __syncthreads();
    for (int a = threadIdx.x; a < nass; a += blockDim.x) {
        const int e = s_ids[a];
        if ((unsigned)e < (unsigned)E) {
            atomicAdd(&s_cnt[e], 1);
            // repeated expert inside one token
            const int t = a / topk;
            for (int j = t * topk; j < a; ++j)
                if (s_ids[j] == e) err = 1;
        }
    }
    __syncthreads();
    // Exclusive scan over experts, 256 threads x ceil(E/256) experts each.
    const int per = (E + blockDim.x - 1) / blockDim.x;
    int local = 0;
    for (int i = 0; i < per; ++i) {
        const int e = threadIdx.x * per + i;
        if (e < E) local += s_cnt[e];
    }
    const int incl = block_inclusive_scan(local, s_tmp);
    int run = incl - local;
    int tiles_local = 0;
    for (int i = 0; i < per; ++i) {
        const int e = threadIdx.x * per + i;
        if (e < E) {
            s_off[e] = run;
            run += s_cnt[e];
            tiles_local += (s_cnt[e] + QL_MOE_TILE_ROWS - 1) / QL_MOE_TILE_ROWS;
        }
    }
    if (threadIdx.x == blockDim.x - 1) s_off[E] = incl;
    const int tincl = block_inclusive_scan(tiles_local, s_tmp);
    int ts = tincl - tiles_local;
    for (int i = 0; i < per; ++i) {
        const int e = threadIdx.x * per + i;
        if (e < E) {
            const int cnt = s_cnt[e];
            counts[e] = cnt;
            offsets[e] = s_off[e];
            for (int j = 0; j * QL_MOE_TILE_ROWS < cnt; ++j, ++ts) {
                int* tp = tiles + (size_t)ts * 4;
                tp[0] = e;
                tp[1] = s_off[e] + j * QL_MOE_TILE_ROWS;
                tp[2] = min(QL_MOE_TILE_ROWS, cnt - j * QL_MOE_TILE_ROWS);
                tp[3] = 0;
            }
        }
    }
    if (threadIdx.x == blockDim.x - 1) offsets[E] = incl;
    __syncthreads();
    // Stable rank: assignments of the same expert with a smaller index.
    for (int a = threadIdx.x; a < nass; a += blockDim.x) {
        const int e = s_ids[a];
        if ((unsigned)e >= (unsigned)E) {
            pos[a] = -1;
            continue;
        }
        int rank = 0;
        for (int b = 0; b < a; ++b) rank += (s_ids[b] == e);
        const int r = min(s_off[e] + rank, s_off[e + 1] - 1);
        sorted_assign[r] = a;
        pos[a] = r;
    }
    const int any = __syncthreads_or(err);
    if (threadIdx.x == blockDim.x - 1) {
        ws_header[0] = tincl;  // inclusive scan of the last thread = all tiles
        ws_header[1] = QL_MOE_TILE_ROWS;
        ws_header[2] = any;
        ws_header[3] = 0;
    }
}

template <int EPL>
int launch_small(const RouteArgs& a, const MoeWorkspace& L, bool do_topk, hipStream_t st) {
    float* partials = reinterpret_cast<float*>(a.ws + L.partials);
    float* logits = reinterpret_cast<float*>(a.ws + L.logits);
    int* hdr = reinterpret_cast<int*>(a.ws + L.header);
    int* tiles = reinterpret_cast<int*>(a.ws + L.tiles);
    if (do_topk)
        hipLaunchKernelGGL((route_small_kernel<EPL, true>), dim3(1), dim3(256), 0, st, partials,
                           L.nparts, a.bias, logits, a.T, a.E, a.topk, a.ids, a.gates, a.counts,
                           a.offsets, a.sorted_assign, a.pos, hdr, tiles);
    else
        hipLaunchKernelGGL((route_small_kernel<EPL, false>), dim3(1), dim3(256), 0, st, partials,
                           L.nparts, a.bias, logits, a.T, a.E, a.topk, a.ids, a.gates, a.counts,
                           a.offsets, a.sorted_assign, a.pos, hdr, tiles);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

int launch_small_any(const RouteArgs& a, const MoeWorkspace& L, bool do_topk, hipStream_t st) {
    const int epl = (a.E + 63) / 64;
    if (epl <= 1) return launch_small<1>(a, L, do_topk, st);
    if (epl <= 2) return launch_small<2>(a, L, do_topk, st);
    if (epl <= 4) return launch_small<4>(a, L, do_topk, st);
    if (epl <= 8) return launch_small<8>(a, L, do_topk, st);
    return launch_small<16>(a, L, do_topk, st);
}

template <int EPL>
void launch_topk_t(const float* src, int nparts, const RouteArgs& a, float* logits, hipStream_t st) {
    hipLaunchKernelGGL((topk_kernel<EPL>), dim3((a.T + 3) / 4), dim3(256), 0, st, src, nparts,
                       a.bias, logits, a.T, a.E, a.topk, a.ids, a.gates);
}

void launch_topk(const float* src, int nparts, const RouteArgs& a, float* logits, hipStream_t st) {
    const int epl = (a.E + 63) / 64;
    if (epl <= 1) launch_topk_t<1>(src, nparts, a, logits, st);
    else if (epl <= 2) launch_topk_t<2>(src, nparts, a, logits, st);
    else if (epl <= 4) launch_topk_t<4>(src, nparts, a, logits, st);
    else if (epl <= 8) launch_topk_t<8>(src, nparts, a, logits, st);
    else launch_topk_t<16>(src, nparts, a, logits, st);
}

int launch_dispatch_large(const RouteArgs& a, const MoeWorkspace& L, hipStream_t st) {
    int* cc = reinterpret_cast<int*>(a.ws + L.chunk_counts);
    int* cerr = reinterpret_cast<int*>(a.ws + L.chunk_err);
    int* hdr = reinterpret_cast<int*>(a.ws + L.header);
    int* tiles = reinterpret_cast<int*>(a.ws + L.tiles);
    const size_t smem = (size_t)a.E * kMaskWords * sizeof(uint32_t);
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(L.nchunks), dim3(kChunk), smem, st, a.ids, a.T,
                       a.E, a.topk, cc, cerr);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, cc, cerr, L.nchunks, a.E,
                       a.counts, a.offsets, hdr, tiles);
    hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(L.nchunks), dim3(kChunk), smem, st, a.ids, a.T,
                       a.E, a.topk, a.offsets, cc, a.sorted_assign, a.pos);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool router_uses_mfma(int T, int E) { return T > kRouterSmallT && E % 8 == 0; }

MoeWorkspace moe_workspace_layout(int T, int E, int topk, int /*unused*/) {
    MoeWorkspace L;
    L.max_tiles = (int)(((int64_t)T * topk) / QL_MOE_TILE_ROWS) + E;
    L.nchunks = (T + kChunk - 1) / kChunk;
    L.nparts = router_uses_mfma(T, E) ? router_mfma_parts() : kRouterParts;
    size_t off = 0;
    L.header = off;
    off += 16;
    L.tiles = off;
    off += (size_t)L.max_tiles * 16;
    off = align256(off);
    L.logits = off;
    off += (size_t)T * E * sizeof(float);
    off = align256(off);
    L.partials = off;
    off += (size_t)T * L.nparts * E * sizeof(float);
    off = align256(off);
    L.chunk_counts = off;
    off += (size_t)L.nchunks * E * sizeof(int);
    off = align256(off);
    L.chunk_err = off;
    off += (size_t)L.nchunks * sizeof(int);
    L.total = align256(off);
    return L;
}


int launch_route(const RouteArgs& a, hipStream_t st) {
    const MoeWorkspace L = moe_workspace_layout(a.T, a.E, a.topk, a.D);
    float* logits = reinterpret_cast<float*>(a.ws + L.logits);
    float* partials = reinterpret_cast<float*>(a.ws + L.partials);
    if (router_uses_mfma(a.T, a.E)) {
        const int rc = launch_router_logits_mfma(a.H, a.Wr, partials, a.T, a.D, a.E, st);
        if (rc != QL_OK) return rc;
    } else {
        hipLaunchKernelGGL(router_partial_kernel, dim3(kRouterParts, a.T), dim3(256), 0, st, a.H,
                           a.Wr, partials, a.D, a.E);
        if (hipGetLastError() != hipSuccess) return QL_ERR_HIP;
        if (a.T <= kRouterSmallT) return launch_small_any(a, L, true, st);
    }
    launch_topk(partials, L.nparts, a, logits, st);
    if (hipGetLastError() != hipSuccess) return QL_ERR_HIP;
    return launch_dispatch_large(a, L, st);
}

int launch_dispatch(const RouteArgs& a, hipStream_t st) {
    const MoeWorkspace L = moe_workspace_layout(a.T, a.E, a.topk, 0);
    if (a.T <= kRouterSmallT) return launch_small_any(a, L, false, st);
    return launch_dispatch_large(a, L, st);
}

}  // namespace ql
