// Top-k selection of one token's expert logits by one wave, shared by the
// router kernels and the fused decode expert kernel.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// Qwen 创建了三种不同的工作负载形状: the router keeps the k best of E experts.
// Reading taken: the k largest logits, ties toward the lower expert index;
// the gates are a softmax over the k chosen logits (the same as a softmax
// over all E renormalized over the chosen k).
#pragma once

#include <math.h>

#include "ql_device.h"
#include "ql_internal.h"

namespace ql {

// ---------------------------------------------------------------------------
// Top-k of one token by one wave.  The order is "larger logit first, then
// lower expert index" on 32-bit monotone keys (mono32: -0 folded into +0, so
// equal logits have equal keys; NaN enters as -inf).  Instead of k rounds of
// wave maxima (a long chain of dependent cross-lane steps), the wave
//  1. takes each lane's largest key and the k-th largest of those 64 lane
//     maxima, tau: at least k keys (those maxima) reach tau, so every key
//     of the top k does;
//  2. compacts the keys >= tau into LDS in ascending expert order (usually
//     little more than k of them);
//  3. ranks each candidate against all candidates (a key beats another if
//     it is larger, or equal with a lower index, i.e. an earlier slot); the
//     rank of a top-k key among the candidates is its rank among all keys,
//     since every key that beats it is itself a candidate.
// The result is exact for any input, ties included; with many equal keys
// step 3 simply has more candidates.
// ---------------------------------------------------------------------------
template <int EPL>
struct __align__(16) TopkScratch {
    uint32_t lane_max[4][64];
    uint32_t ck[4][64 * EPL + 4];     // candidate keys (+ zero padding to a multiple of 4)
    uint16_t ce[4][64 * EPL];         // candidate expert indices
    uint32_t sk[4][QL_MAX_TOPK_DEV];  // selected keys by rank
    int se[4][QL_MAX_TOPK_DEV];       // selected experts by rank
};

// LDS written by some lanes of a wave and then read by others: the wave's
// LDS operations complete in program order, so only the compiler must be
// kept from moving them across this point.
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// Logits of token t are the sum of `nparts` partial rows (fixed order) plus
// the optional bias; they are written to logits_out.  Writes the topk
// chosen experts (descending) and their renormalized gates to sel_e/sel_g.
// Called by whole waves of a 256-thread block.
template <int EPL, int NP>
__device__ void topk_one_token(const float* __restrict__ src, const float* __restrict__ bias,
                               float* __restrict__ logits_out, int t, int E, int topk, int* sel_e,
                               float* sel_g) {
    __shared__ TopkScratch<EPL> scr;
    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    // Every partial of every logit this lane owns is loaded before the first
    // sum (NP and EPL are compile-time), so the whole token costs one round
    // trip to memory.
    float part[EPL][NP];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = min(lane + 64 * i, E - 1);
#pragma unroll
        for (int p = 0; p < NP; ++p) part[i][p] = src[((size_t)t * NP + p) * E + e];
    }
    // Lane l holds the keys of experts l, l + 64, ...; 0 past E (below the
    // key of any float).
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + 64 * i;
        key[i] = 0u;
        if (e < E) {
            float s = 0.f;
#pragma unroll
            for (int p = 0; p < NP; ++p) s += part[i][p];
            if (bias) s += bias[e];
            logits_out[(size_t)t * E + e] = s;
            key[i] = mono32((s != s) ? -INFINITY : s + 0.0f);  // NaN never wins
        }
    }
    // 1. tau = the topk-th largest lane maximum, counted with multiplicity:
    //    the smallest maximum that fewer than topk maxima exceed.
    uint32_t m = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) m = max(m, key[i]);
    uint32_t* const lmax = scr.lane_max[wv];
    lmax[lane] = m;
    wave_lds_sync();
    int above = 0;
#pragma unroll
    for (int c = 0; c < 64; c += 4) {
        const uint4 q = *reinterpret_cast<const uint4*>(lmax + c);
        above += (q.x > m) + (q.y > m) + (q.z > m) + (q.w > m);
    }
    const uint32_t tau = wave_min_u32(above < topk ? m : 0xFFFFFFFFu);
    // 2. candidates in ascending expert order (slot order = index order).
    uint32_t* const ck = scr.ck[wv];
    uint16_t* const ce = scr.ce[wv];
    int C = 0;  // uniform
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const bool is = key[i] >= tau;
        const uint64_t b = __ballot(is);
        if (is) {
            const int at = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
            ck[at] = key[i];
            ce[at] = (uint16_t)(lane + 64 * i);
        }
        C += __popcll(b);
    }
    if (lane < 4) ck[C + lane] = 0u;  // never beats a candidate (tau > 0)
    wave_lds_sync();
    // 3. ranks; the candidates of rank < topk are the result.
    uint32_t* const sk = scr.sk[wv];
    int* const se = scr.se[wv];
    const int C4 = (C + 3) & ~3;
    for (int slot = lane; slot < C; slot += 64) {
        const uint32_t k = ck[slot];
        int r = 0;
        for (int c = 0; c < C4; c += 4) {
            const uint4 q = *reinterpret_cast<const uint4*>(ck + c);
            r += (q.x > k) + (q.y > k) + (q.z > k) + (q.w > k);
            r += (q.x == k && c < slot) + (q.y == k && c + 1 < slot) + (q.z == k && c + 2 < slot) +
                 (q.w == k && c + 3 < slot);
        }
        if (r < topk) {
            sk[r] = k;
            se[r] = ce[slot];
        }
    }
    wave_lds_sync();
    const float vmax = unmono32(sk[0]);
    float my_v = 0.f;
    int my_e = 0;
    if (lane < topk) {
        my_v = unmono32(sk[lane]);
        my_e = se[lane];
    }
    float ex = (lane < topk) ? __expf(my_v - vmax) : 0.f;
    const float exs[1] = {ex};
    int unused;
    const float sum = reduce_rows64<1>(exs, lane, unused);  // every lane: the total
    if (lane < topk) {
        sel_e[lane] = my_e;
        sel_g[lane] = ex / sum;
    }
}

// ---------------------------------------------------------------------------
// The same selection by a whole 256-thread block for one token with E <= 256
// experts (thread t holds expert t), for the fused decode expert launch where
// all four waves would otherwise wait for one: the threshold tau of
// topk_one_token is the topk-th largest of the 64 quad maxima (keys of
// experts 4q .. 4q+3), each thread counting the maxima above its quad's
// against a quarter of them; candidates (keys >= tau) are compacted into LDS
// in expert order across the waves, ranked as in topk_one_token, and wave 0
// writes the topk experts and their renormalized gates.  Same results as
// topk_one_token, bit for bit.  logits: LDS, the token's E logits (with any
// bias already added).  Called by all 256 threads; ends with a barrier.
// ---------------------------------------------------------------------------
struct __align__(16) TopkBlockScratch {
    uint32_t qm[64];          // quad maxima
    uint32_t tau[4];          // per-wave minima
    int cnt[4];               // candidates per wave
    uint32_t ck[256 + 4];     // candidate keys in expert order (+ zero padding)
    uint16_t ce[256];         // candidate experts
    uint32_t sk[QL_MAX_TOPK_DEV];
    int se[QL_MAX_TOPK_DEV];
};

__device__ void topk_block_small(const float* __restrict__ logits, int E, int topk, int* sel_e,
                                 float* sel_g) {
    __shared__ TopkBlockScratch scr;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wv = tid >> 6;
    uint32_t key = 0u;
    if (tid < E) {
        const float s = logits[tid];
        key = mono32((s != s) ? -INFINITY : s + 0.0f);  // NaN never wins
    }
    // 1. quad maxima
    uint32_t m = max(key, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)key, 0xB1, 0xF, 0xF, true));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, true));
    if ((tid & 3) == 0) scr.qm[tid >> 2] = m;
    __syncthreads();
    // 2. maxima above this quad's, a quarter per thread, summed over the quad
    const int c = tid & 3;
    int above = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint4 q = *reinterpret_cast<const uint4*>(scr.qm + 16 * c + 4 * i);
        above += (q.x > m) + (q.y > m) + (q.z > m) + (q.w > m);
    }
    above += __builtin_amdgcn_update_dpp(0, above, 0xB1, 0xF, 0xF, true);
    above += __builtin_amdgcn_update_dpp(0, above, 0x4E, 0xF, 0xF, true);
    const uint32_t tw = wave_min_u32(above < topk ? m : 0xFFFFFFFFu);
    if (lane == 0) scr.tau[wv] = tw;
    __syncthreads();
    const uint32_t tau = min(min(scr.tau[0], scr.tau[1]), min(scr.tau[2], scr.tau[3]));
    // 3. candidates in expert order across the four waves
    const bool is = key >= tau;
    const uint64_t b = __ballot(is);
    if (lane == 0) scr.cnt[wv] = __popcll(b);
    __syncthreads();
    int base = 0, C = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        base += (w < wv) ? scr.cnt[w] : 0;
        C += scr.cnt[w];
    }
    if (is) {
        const int at = base + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
        scr.ck[at] = key;
        scr.ce[at] = (uint16_t)tid;
    }
    if (tid < 4) scr.ck[C + tid] = 0u;  // padding: never beats a candidate
    __syncthreads();
    // 4. ranks; the candidates of rank < topk are the result
    const int C4 = (C + 3) & ~3;
    for (int slot = tid; slot < C; slot += 256) {
        const uint32_t k = scr.ck[slot];
        int r = 0;
        for (int cc = 0; cc < C4; cc += 4) {
            const uint4 q = *reinterpret_cast<const uint4*>(scr.ck + cc);
            r += (q.x > k) + (q.y > k) + (q.z > k) + (q.w > k);
            r += (q.x == k && cc < slot) + (q.y == k && cc + 1 < slot) + (q.z == k && cc + 2 < slot) +
                 (q.w == k && cc + 3 < slot);
        }
        if (r < topk) {
            scr.sk[r] = k;
            scr.se[r] = scr.ce[slot];
        }
    }
    __syncthreads();
    // 5. gates: softmax over the chosen logits
    if (wv == 0) {
        const float vmax = unmono32(scr.sk[0]);
        float my_v = 0.f;
        int my_e = 0;
        if (lane < topk) {
            my_v = unmono32(scr.sk[lane]);
            my_e = scr.se[lane];
        }
        const float ex = (lane < topk) ? __expf(my_v - vmax) : 0.f;
        const float exs[1] = {ex};
        int unused;
        const float sum = reduce_rows64<1>(exs, lane, unused);
        if (lane < topk) {
            sel_e[lane] = my_e;
            sel_g[lane] = ex / sum;
        }
    }
    __syncthreads();
}

}  // namespace ql
