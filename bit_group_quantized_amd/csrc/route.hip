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
#include "ql_topk.h"

#include <float.h>

namespace ql {

namespace {

constexpr int kChunk = kRouteChunkTokens;
constexpr int kMaskWords = kChunk / 32;
constexpr int kRouterParts = kRouterSmallParts;  // row-parallel router: D split in 8 slices
constexpr int kRouterMfmaParts = kRouterMfmaSplit;  // MFMA router: K split

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
// 16-bit value of H or Wr as fp32: fp16, or bf16 for the bf16 variant.
template <bool BF16>
__device__ __forceinline__ float in16(uint16_t v) {
    if constexpr (BF16) return bf2f(v);
    else return h2f(v);
}

template <bool BF16>
__device__ __forceinline__ void router_partial_body(const uint16_t* __restrict__ H,
                                                    const uint16_t* __restrict__ Wr,
                                                    float* __restrict__ partials, int D, int E) {
    __shared__ float hs[QL_MAX_K / kRouterParts];
    const int t = blockIdx.y, p = blockIdx.x;
    const int rows = D / kRouterParts;
    const int d0 = p * rows;
    for (int i = threadIdx.x; i < rows; i += blockDim.x) hs[i] = in16<BF16>(H[(size_t)t * D + d0 + i]);
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        float acc = 0.f;
        for (int d = 0; d < rows; ++d) acc += hs[d] * in16<BF16>(Wr[(size_t)(d0 + d) * E + e]);
        partials[((size_t)t * kRouterParts + p) * E + e] = acc;
    }
}

// The same partial sums, one block per (D slice, group of 32 experts), for
// more parallelism at few tokens (8 x as many blocks, each reading 16 KB of
// the router weight at D = 2048): thread (rl, sg) covers the slice's rows
// rl, rl + 64, ... for experts 32g + 8sg .. 32g + 8sg + 7 (one 16-byte load
// per row); the 64 row lanes of each expert are summed in a fixed order
// (eight groups of eight, then the eight group sums).  Requires E % 8 == 0.
template <bool BF16>
__device__ __forceinline__ void router_partial_grp_body(const uint16_t* __restrict__ H,
                                                        const uint16_t* __restrict__ Wr,
                                                        float* __restrict__ partials, int D, int E) {
    __shared__ float red[64][33];
    __shared__ float red2[8][32];
    const int p = blockIdx.x, g = blockIdx.y, t = blockIdx.z;
    const int rows = D / kRouterParts;
    const int d0 = p * rows;
    const int rl = threadIdx.x >> 2;  // 0..63
    const int sg = threadIdx.x & 3;   // 0..3
    const int e8 = g * 32 + sg * 8;
    float acc[8];
#pragma unroll
    for (int v = 0; v < 8; ++v) acc[v] = 0.f;
    if (e8 < E) {
#pragma unroll 4  // a slice of 256 rows: the four row loads of a thread go out together
        for (int d = rl; d < rows; d += 64) {
            const float h = in16<BF16>(H[(size_t)t * D + d0 + d]);
            const u32x4 wv = ld_u32x4(Wr + (size_t)(d0 + d) * E + e8);
            const uint32_t ww[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                acc[2 * v] += h * in16<BF16>((uint16_t)(ww[v] & 0xFFFFu));
                acc[2 * v + 1] += h * in16<BF16>((uint16_t)(ww[v] >> 16));
            }
        }
    }
#pragma unroll
    for (int v = 0; v < 8; ++v) red[rl][sg * 8 + v] = acc[v];
    __syncthreads();
    const int c = threadIdx.x & 31, q = threadIdx.x >> 5;
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += red[q * 8 + i][c];
    red2[q][c] = s;
    __syncthreads();
    if (threadIdx.x < 32 && g * 32 + c < E) {
        float tot = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) tot += red2[i][c];
        partials[((size_t)t * kRouterParts + p) * E + g * 32 + c] = tot;
    }
}

template <bool BF16>
__global__ void __launch_bounds__(256)
router_partial_grp_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wr,
                          float* __restrict__ partials, int D, int E) {
    router_partial_grp_body<BF16>(H, Wr, partials, D, E);
}

template <bool BF16>
__global__ void __launch_bounds__(256)
router_partial_kernel(const uint16_t* __restrict__ H, const uint16_t* __restrict__ Wr,
                      float* __restrict__ partials, int D, int E) {
    router_partial_body<BF16>(H, Wr, partials, D, E);
}

template <int EPL, int NP>
__global__ void __launch_bounds__(256)
topk_kernel(const float* __restrict__ src, const float* __restrict__ bias,
            float* __restrict__ logits_out, int T, int E, int topk,
            int* __restrict__ ids, float* __restrict__ gates) {
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;  // whole wave leaves together
    topk_one_token<EPL, NP>(src, bias, logits_out, t, E, topk, ids + (size_t)t * topk,
                            gates + (size_t)t * topk);
}

// ---------------------------------------------------------------------------
// Dispatch for many tokens: per-chunk masks and counts, one scan block, and
// the stable scatter.
// ---------------------------------------------------------------------------
// Per-chunk masks in LDS: bit (t % 32) of mask[e][t / 32] is set when token
// t of the chunk chose expert e.  With s_ids given, the chunk's ids are also
// kept in LDS ([token][topk]).  Returns 1 if an id was out of range or
// repeated within a token.
__device__ int build_chunk_masks(const int* __restrict__ ids, int T, int E, int topk, int c,
                                 uint32_t* mask, int* s_ids) {
    for (int i = threadIdx.x; i < E * kMaskWords; i += blockDim.x) mask[i] = 0u;
    __syncthreads();
    const int tl = threadIdx.x;
    const int t = c * kChunk + tl;
    int err = 0;
    if (t < T) {
        const uint32_t bit = 1u << (tl & 31);
        // Eight ids are loaded before any is used (clamped, unconditional
        // loads: a conditional one would be waited for on its own).
        for (int j0 = 0; j0 < topk; j0 += 8) {
            int v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = ids[(size_t)t * topk + min(j0 + u, topk - 1)];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int j = j0 + u;
                if (j >= topk) break;
                const int e = v[u];
                if (s_ids) s_ids[tl * topk + j] = e;
                if ((unsigned)e >= (unsigned)E) {
                    err = 1;
                    continue;
                }
                const uint32_t old = atomicOr(&mask[e * kMaskWords + (tl >> 5)], bit);
                if (old & bit) err = 1;
            }
        }
    }
    __syncthreads();
    return err;
}

__global__ void __launch_bounds__(kChunk)
dispatch_count_kernel(const int* __restrict__ ids, int T, int E, int topk,
                      int* __restrict__ chunk_counts, int* __restrict__ chunk_err,
                      uint32_t* __restrict__ chunk_masks) {
    extern __shared__ __align__(16) uint32_t mask[];
    const int c = blockIdx.x;
    const int err = build_chunk_masks(ids, T, E, topk, c, mask, nullptr);
    static_assert(kMaskWords == 8, "two 16-byte stores per expert");
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        int cnt = 0;
#pragma unroll
        for (int w = 0; w < kMaskWords; ++w) cnt += __popc(mask[e * kMaskWords + w]);
        chunk_counts[(size_t)c * E + e] = cnt;
        // the expert's masks of this chunk, for the scatter
        u32x4* dst = reinterpret_cast<u32x4*>(chunk_masks + ((size_t)c * E + e) * kMaskWords);
        dst[0] = *reinterpret_cast<const u32x4*>(mask + e * kMaskWords);
        dst[1] = *reinterpret_cast<const u32x4*>(mask + e * kMaskWords + 4);
    }
    const int any = __syncthreads_or(err);
    if (threadIdx.x == 0) chunk_err[c] = any;
}

// One block, one thread per expert: chunk bases (in place), counts, offsets
// and the load-matched tile map (section 使瓦片大小与专家负载相匹配): an
// expert's rows go into tiles of 2 * QL_MOE_TILE_ROWS rows while a full one
// remains, the rest into tiles of at most QL_MOE_TILE_ROWS rows; the tall
// tiles are listed first.  short_order lists the short tiles (as indices
// after the tall ones) by cost for the grouped GEMM's scheduling: those of
// more than kTinyTileRows rows first, then the rest, each group in map order.
__global__ void __launch_bounds__(1024)
dispatch_scan_kernel(int* __restrict__ chunk_counts, const int* __restrict__ chunk_err,
                     int nchunks, int E, int* __restrict__ counts, int* __restrict__ offsets,
                     int* __restrict__ ws_header, int* __restrict__ tiles, int* __restrict__ short_order) {
    constexpr int SR = QL_MOE_TILE_ROWS, BR = 2 * QL_MOE_TILE_ROWS;
    __shared__ int s_tmp[16];
    __shared__ int s_tot[3];
    const int e = threadIdx.x;
    int run = 0;
    if (e < E) {
        // Sixteen chunk counts are loaded before any is used, so the loop costs
        // one memory round trip per sixteen chunks.
        for (int c0 = 0; c0 < nchunks; c0 += 16) {
            // clamped, unconditional loads (a conditional load would be
            // waited for on its own)
            int v[16];
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = chunk_counts[(size_t)min(c0 + u, nchunks - 1) * E + e];
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (c0 + u < nchunks) {
                    chunk_counts[(size_t)(c0 + u) * E + e] = run;  // the chunk's base inside e
                    run += v[u];
                }
            }
        }
        counts[e] = run;
    }
    const int cnt = (e < E) ? run : 0;
    const int incl = block_inclusive_scan(cnt, s_tmp);
    const int excl = incl - cnt;
    if (e < E) offsets[e] = excl;
    if (e == E - 1) offsets[E] = incl;
    const int nb = cnt / BR;
    const int rem = cnt - nb * BR;
    const int ns = (rem + SR - 1) / SR;
    // Only an expert's last short tile can have kTinyTileRows rows or fewer.
    const int ntiny = (ns > 0 && rem - (ns - 1) * SR <= kTinyTileRows) ? 1 : 0;
    const int binc = block_inclusive_scan(nb, s_tmp);
    const int sinc = block_inclusive_scan(ns, s_tmp);
    const int winc = block_inclusive_scan(ns - ntiny, s_tmp);
    if (threadIdx.x == blockDim.x - 1) {
        s_tot[0] = binc;
        s_tot[1] = sinc;
        s_tot[2] = winc;
    }
    __syncthreads();
    const int nbig = s_tot[0];
    const int nwide = s_tot[2];
    const int tinc = (sinc - winc);  // tiny tiles of experts 0 .. e (inclusive)
    for (int j = 0; j < nb; ++j) {
        int* tp = tiles + (size_t)(binc - nb + j) * 4;
        tp[0] = e;
        tp[1] = excl + j * BR;
        tp[2] = BR;
        tp[3] = BR;
    }
    for (int j = 0; j < ns; ++j) {
        int* tp = tiles + (size_t)(nbig + sinc - ns + j) * 4;
        tp[0] = e;
        tp[1] = excl + nb * BR + j * SR;
        tp[2] = min(SR, rem - j * SR);
        tp[3] = SR;
        const bool tiny = ntiny && j == ns - 1;
        short_order[tiny ? nwide + tinc - 1 : winc - (ns - ntiny) + j] = sinc - ns + j;
    }
    int err = 0;
    for (int c = e; c < nchunks; c += blockDim.x) err |= chunk_err[c];
    const int any = __syncthreads_or(err);
    if (threadIdx.x == blockDim.x - 1) {
        ws_header[0] = nbig + s_tot[1];
        ws_header[3] = nbig;
    }
    if (e == 0) {
        ws_header[1] = SR;
        ws_header[2] = any;
    }
}

// The scatter with one block per 32 tokens (one mask word of a chunk) and
// one thread per assignment: the rank of token t inside expert e is the
// population count of the chunk's mask words of e before t's word, plus
// that of t's word below bit t; the chunk's base inside e comes from the
// scan (chunk_counts, rewritten in place).
__global__ void __launch_bounds__(1024)
dispatch_scatter_words_kernel(const int* __restrict__ ids, int T, int E, int topk,
                              const int* __restrict__ offsets, const int* __restrict__ chunk_base,
                              const uint32_t* __restrict__ chunk_masks, int* __restrict__ sorted_assign,
                              int* __restrict__ pos, int2* __restrict__ row_info,
                              int2* __restrict__ assign_info) {
    const int c = blockIdx.x / kMaskWords, w = blockIdx.x % kMaskWords;
    const int al = threadIdx.x;
    if (al >= 32 * topk) return;
    const int tl = al / topk;  // token within the word
    const int t = c * kChunk + w * 32 + tl;
    if (t >= T) return;
    const int a = t * topk + al % topk;
    const int e = ids[a];
    if ((unsigned)e >= (unsigned)E) {
        pos[a] = -1;
        assign_info[a] = make_int2(-1, -1);
        return;
    }
    const u32x4* mk = reinterpret_cast<const u32x4*>(chunk_masks + ((size_t)c * E + e) * kMaskWords);
    const u32x4 m0 = mk[0], m1 = mk[1];
    const uint32_t words[kMaskWords] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    int rank = 0;
#pragma unroll
    for (int ww = 0; ww < kMaskWords; ++ww) {
        if (ww < w) rank += __popc(words[ww]);
        else if (ww == w) rank += __popc(words[ww] & ((1u << tl) - 1u));
    }
    const int r = offsets[e] + chunk_base[(size_t)c * E + e] + rank;
    sorted_assign[r] = a;
    pos[a] = r;
    row_info[r] = make_int2(e, t);
    assign_info[a] = make_int2(e, r);
}

// ---------------------------------------------------------------------------
// Small T (decode): top-k and the whole dispatch in one block.  With at most
// kRouterSmallT tokens one 32-bit mask per expert records which tokens chose
// it; counts are population counts, the rank of token t inside its expert
// is the population count of the mask below bit t (stable by construction),
// and one block scan over the experts gives both the row offsets and the
// tile indices (every expert has at most one tile here).
// ---------------------------------------------------------------------------
// Logits of at most this many (token, expert) pairs stay in LDS.
constexpr int kSmallLogitsLds = 4096;

template <int EPL, bool DO_TOPK>
__device__ __forceinline__ void route_small_body(const float* __restrict__ partials, const float* __restrict__ bias,
                 float* __restrict__ logits_out, int T, int E, int topk,
                 int* __restrict__ ids, float* __restrict__ gates, int* __restrict__ counts,
                 int* __restrict__ offsets, int* __restrict__ sorted_assign,
                 int* __restrict__ pos, int* __restrict__ ws_header, int* __restrict__ tiles,
                 int2* __restrict__ row_info, int2* __restrict__ assign_info, int* __restrict__ short_order) {
    static_assert(kRouterSmallT <= 32 && kRouterSmallT * QL_MAX_TOPK_DEV <= 4 * QL_MAX_EXPERTS_DEV,
                  "token masks are 32 bits wide");
    static_assert(QL_MOE_TILE_ROWS >= kRouterSmallT, "one tile per expert");
    static_assert(kTinyTileRows >= kRouterSmallT, "every tile is one of the cheapest kind");
    // Every intermediate stays in LDS and every global store is issued after
    // the last barrier: a barrier waits for the block's outstanding stores.
    __shared__ int s_ids[kRouterSmallT * QL_MAX_TOPK_DEV];
    __shared__ float s_gates[kRouterSmallT * QL_MAX_TOPK_DEV];
    __shared__ uint32_t s_mask[QL_MAX_EXPERTS_DEV];
    __shared__ int s_off[QL_MAX_EXPERTS_DEV];
    __shared__ int s_tile[QL_MAX_EXPERTS_DEV];
    __shared__ float s_logits[kSmallLogitsLds];
    __shared__ int s_tmp[16];
    __shared__ int s_total;
    const int wave = threadIdx.x >> 6;
    const int nass = T * topk;
    const bool lds_logits = T * E <= kSmallLogitsLds;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s_mask[e] = 0u;
    if constexpr (DO_TOPK) {
        // Logits of all tokens, one (token, expert) per thread: the partial
        // rows are summed in a fixed order, all of their loads issued at once.
        float* lg = lds_logits ? s_logits : logits_out;
        for (int idx = threadIdx.x; idx < T * E; idx += blockDim.x) {
            const int tt = idx / E, e = idx - tt * E;
            float part[kRouterParts];
#pragma unroll
            for (int p = 0; p < kRouterParts; ++p) part[p] = partials[((size_t)tt * kRouterParts + p) * E + e];
            float sum = 0.f;
#pragma unroll
            for (int p = 0; p < kRouterParts; ++p) sum += part[p];
            if (bias) sum += bias[e];
            lg[idx] = sum;
        }
        __syncthreads();
        for (int t = wave; t < T; t += 4)
            topk_one_token<EPL, 1>(lg, nullptr, lg, t, E, topk, s_ids + t * topk, s_gates + t * topk);
        __syncthreads();
    } else {
        for (int a = threadIdx.x; a < nass; a += blockDim.x) s_ids[a] = ids[a];
        __syncthreads();
    }
    int err = 0;
    for (int a = threadIdx.x; a < nass; a += blockDim.x) {
        const int e = s_ids[a];
        if ((unsigned)e >= (unsigned)E) {
            err = 1;
            continue;
        }
        const uint32_t bit = 1u << (a / topk);
        if (atomicOr(&s_mask[e], bit) & bit) err = 1;  // expert repeated within a token
    }
    const int any = __syncthreads_or(err);
    // Per thread a contiguous run of experts; scan of (rows, tiles) packed
    // in one int (rows < 2^16 here).
    const int per = (E + blockDim.x - 1) / blockDim.x;
    int local = 0;
    for (int i = 0; i < per; ++i) {
        const int e = threadIdx.x * per + i;
        if (e < E) {
            const int c = __popc(s_mask[e]);
            local += c + ((c > 0) << 16);
        }
    }
    const int incl = block_inclusive_scan(local, s_tmp);
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
        const int e = threadIdx.x * per + i;
        if (e < E) {
            const int c = __popc(s_mask[e]);
            s_off[e] = run & 0xFFFF;
            s_tile[e] = run >> 16;
            run += c + ((c > 0) << 16);
        }
    }
    if (threadIdx.x == blockDim.x - 1) s_total = incl;
    __syncthreads();
    // ---- outputs (no barrier from here on) ----
    if constexpr (DO_TOPK) {
        if (lds_logits)
            for (int idx = threadIdx.x; idx < T * E; idx += blockDim.x) logits_out[idx] = s_logits[idx];
        for (int a = threadIdx.x; a < nass; a += blockDim.x) {
            ids[a] = s_ids[a];
            gates[a] = s_gates[a];
        }
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const int c = __popc(s_mask[e]);
        counts[e] = c;
        offsets[e] = s_off[e];
        if (c > 0) {
            int* tp = tiles + (size_t)s_tile[e] * 4;
            tp[0] = e;
            tp[1] = s_off[e];
            tp[2] = c;
            tp[3] = QL_MOE_TILE_ROWS;  // tile height: short tiles only here
            short_order[s_tile[e]] = s_tile[e];  // all of them have at most kRouterSmallT rows
        }
    }
    for (int a = threadIdx.x; a < nass; a += blockDim.x) {
        const int e = s_ids[a];
        if ((unsigned)e >= (unsigned)E) {
            pos[a] = -1;
            assign_info[a] = make_int2(-1, -1);
            continue;
        }
        const int t = a / topk;
        const int r = s_off[e] + __popc(s_mask[e] & ((1u << t) - 1u));
        sorted_assign[r] = a;
        pos[a] = r;
        row_info[r] = make_int2(e, t);
        assign_info[a] = make_int2(e, r);
    }
    if (threadIdx.x == blockDim.x - 1) {
        offsets[E] = s_total & 0xFFFF;
        ws_header[0] = s_total >> 16;  // all tiles
        ws_header[1] = QL_MOE_TILE_ROWS;
        ws_header[2] = any;
        ws_header[3] = 0;
    }
}

template <int EPL, bool DO_TOPK>
__global__ void __launch_bounds__(256)
route_small_kernel(const float* __restrict__ partials, const float* __restrict__ bias,
                   float* __restrict__ logits_out, int T, int E, int topk,
                   int* __restrict__ ids, float* __restrict__ gates, int* __restrict__ counts,
                   int* __restrict__ offsets, int* __restrict__ sorted_assign,
                   int* __restrict__ pos, int* __restrict__ ws_header, int* __restrict__ tiles,
                   int2* __restrict__ row_info, int2* __restrict__ assign_info, int* __restrict__ short_order) {
    route_small_body<EPL, DO_TOPK>(partials, bias, logits_out, T, E, topk, ids, gates, counts, offsets,
                                   sorted_assign, pos, ws_header, tiles, row_info, assign_info, short_order);
}


template <int EPL>
int launch_small(const RouteArgs& a, const MoeWorkspace& L, bool do_topk, hipStream_t st) {
    float* partials = reinterpret_cast<float*>(a.ws + L.partials);
    float* logits = reinterpret_cast<float*>(a.ws + L.logits);
    int* hdr = reinterpret_cast<int*>(a.ws + L.header);
    int* tiles = reinterpret_cast<int*>(a.ws + L.tiles);
    int2* rinfo = reinterpret_cast<int2*>(a.ws + L.row_info);
    int2* ainfo = reinterpret_cast<int2*>(a.ws + L.assign_info);
    int* sorder = reinterpret_cast<int*>(a.ws + L.short_order);
    if (do_topk)
        hipLaunchKernelGGL((route_small_kernel<EPL, true>), dim3(1), dim3(256), 0, st, partials,
                           a.bias, logits, a.T, a.E, a.topk, a.ids, a.gates, a.counts,
                           a.offsets, a.sorted_assign, a.pos, hdr, tiles, rinfo, ainfo, sorder);
    else
        hipLaunchKernelGGL((route_small_kernel<EPL, false>), dim3(1), dim3(256), 0, st, partials,
                           a.bias, logits, a.T, a.E, a.topk, a.ids, a.gates, a.counts,
                           a.offsets, a.sorted_assign, a.pos, hdr, tiles, rinfo, ainfo, sorder);
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

template <int EPL, int NP>
void launch_topk_t(const float* src, const RouteArgs& a, float* logits, hipStream_t st) {
    hipLaunchKernelGGL((topk_kernel<EPL, NP>), dim3((a.T + 3) / 4), dim3(256), 0, st, src, a.bias,
                       logits, a.T, a.E, a.topk, a.ids, a.gates);
}

template <int NP>
void launch_topk_np(const float* src, const RouteArgs& a, float* logits, hipStream_t st) {
    const int epl = (a.E + 63) / 64;
    if (epl <= 1) launch_topk_t<1, NP>(src, a, logits, st);
    else if (epl <= 2) launch_topk_t<2, NP>(src, a, logits, st);
    else if (epl <= 4) launch_topk_t<4, NP>(src, a, logits, st);
    else if (epl <= 8) launch_topk_t<8, NP>(src, a, logits, st);
    else launch_topk_t<16, NP>(src, a, logits, st);
}

void launch_topk(const float* src, int nparts, const RouteArgs& a, float* logits, hipStream_t st) {
    if (nparts == kRouterParts) launch_topk_np<kRouterParts>(src, a, logits, st);
    else launch_topk_np<kRouterMfmaParts>(src, a, logits, st);
}

int launch_dispatch_large(const RouteArgs& a, const MoeWorkspace& L, hipStream_t st) {
    int* cc = reinterpret_cast<int*>(a.ws + L.chunk_counts);
    int* cerr = reinterpret_cast<int*>(a.ws + L.chunk_err);
    int* hdr = reinterpret_cast<int*>(a.ws + L.header);
    int* tiles = reinterpret_cast<int*>(a.ws + L.tiles);
    const size_t smem = (size_t)a.E * kMaskWords * sizeof(uint32_t);  // at most 32 KB
    uint32_t* masks = reinterpret_cast<uint32_t*>(a.ws + L.chunk_masks);
    hipLaunchKernelGGL(dispatch_count_kernel, dim3(L.nchunks), dim3(kChunk), smem, st, a.ids, a.T,
                       a.E, a.topk, cc, cerr, masks);
    hipLaunchKernelGGL(dispatch_scan_kernel, dim3(1), dim3(1024), 0, st, cc, cerr, L.nchunks, a.E,
                       a.counts, a.offsets, hdr, tiles, reinterpret_cast<int*>(a.ws + L.short_order));
    const int threads = (32 * a.topk + 63) / 64 * 64;
    hipLaunchKernelGGL(dispatch_scatter_words_kernel, dim3(L.nchunks * kMaskWords), dim3(threads), 0, st,
                       a.ids, a.T, a.E, a.topk, a.offsets, cc, masks, a.sorted_assign, a.pos,
                       reinterpret_cast<int2*>(a.ws + L.row_info),
                       reinterpret_cast<int2*>(a.ws + L.assign_info));
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

}  // namespace

bool router_uses_mfma(int T, int E) { return T > kRouterSmallT && E % 8 == 0; }

MoeWorkspace moe_workspace_layout(int T, int E, int topk) {
    MoeWorkspace L;
    L.max_tiles = (int)(((int64_t)T * topk) / QL_MOE_TILE_ROWS) + E;
    L.nchunks = (T + kChunk - 1) / kChunk;
    L.nparts = router_uses_mfma(T, E) ? kRouterMfmaParts : kRouterParts;
    size_t off = 0;
    L.header = off;
    off += 32;
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
    off = align256(off);
    L.chunk_masks = off;
    off += (size_t)L.nchunks * E * kMaskWords * sizeof(uint32_t);
    off = align256(off);
    L.row_info = off;
    off += (size_t)T * topk * 2 * sizeof(int);
    off = align256(off);
    L.assign_info = off;
    off += (size_t)T * topk * 2 * sizeof(int);
    off = align256(off);
    L.short_order = off;
    off += (size_t)L.max_tiles * sizeof(int);
    L.total = align256(off);
    return L;
}


namespace {

template <bool BF16>
void launch_router_partials_t(const uint16_t* H, const uint16_t* Wr, float* partials, int T, int D,
                              int E, hipStream_t st) {
    if (E % 8 == 0)
        hipLaunchKernelGGL((router_partial_grp_kernel<BF16>), dim3(kRouterParts, (E + 31) / 32, T), dim3(256),
                           0, st, H, Wr, partials, D, E);
    else
        hipLaunchKernelGGL((router_partial_kernel<BF16>), dim3(kRouterParts, T), dim3(256), 0, st, H,
                           Wr, partials, D, E);
}

}  // namespace

int launch_router_partials_small(const uint16_t* H, const uint16_t* Wr, float* partials, int T,
                                 int D, int E, hipStream_t st, bool bf16) {
    if (bf16) launch_router_partials_t<true>(H, Wr, partials, T, D, E, st);
    else launch_router_partials_t<false>(H, Wr, partials, T, D, E, st);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

int launch_route(const RouteArgs& a, hipStream_t st) {
    const MoeWorkspace L = moe_workspace_layout(a.T, a.E, a.topk);
    float* logits = reinterpret_cast<float*>(a.ws + L.logits);
    float* partials = reinterpret_cast<float*>(a.ws + L.partials);
    if (router_uses_mfma(a.T, a.E)) {
        const int rc = launch_router_logits_mfma(a.H, a.Wr, partials, a.T, a.D, a.E, st, a.bf16);
        if (rc != QL_OK) return rc;
    } else {
        const int rc = launch_router_partials_small(a.H, a.Wr, partials, a.T, a.D, a.E, st, a.bf16);
        if (rc != QL_OK) return rc;
        if (a.T <= kRouterSmallT) return launch_small_any(a, L, true, st);
    }
    launch_topk(partials, L.nparts, a, logits, st);
    if (hipGetLastError() != hipSuccess) return QL_ERR_HIP;
    return launch_dispatch_large(a, L, st);
}

int launch_dispatch(const RouteArgs& a, hipStream_t st) {
    const MoeWorkspace L = moe_workspace_layout(a.T, a.E, a.topk);
    if (a.T <= kRouterSmallT) return launch_small_any(a, L, false, st);
    return launch_dispatch_large(a, L, st);
}

}  // namespace ql
