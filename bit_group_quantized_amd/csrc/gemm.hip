// MFMA GEMM kernels with the w4 dequantization fused into the tile loop:
// the dense prefill GEMM, the grouped expert GEMMs over routed tiles, and the
// fp16 router GEMM.
//
// Perplexity, "Optimizing on-device inference for Apple Silicon", section
// 在矩阵乘法期间进行权重反量化: the grouped GEMM dequantizes one small weight
// tile at a time into on-chip memory, keeps it only long enough to multiply
// it with the routed activation rows, accumulates in fp32 and writes 16-bit
// outputs; the full dequantized matrix never exists in memory.  Section
// 使瓦片大小与专家负载相匹配: each expert's rows are cut into fixed-height tiles
// and every tile is one workgroup.
//
// gfx950 mapping.  A workgroup of WGM x WGN waves owns a BM x BN output
// tile; each wave owns (32*WM) x (32*WN) and issues v_mfma_f32_32x32x16_f16
// on it.  Dense prefill with M >= 2048 uses 8 waves (two per SIMD) of
// 128 x 64 on 256 x 256 tiles; the grouped expert GEMMs use 8 waves of
// 64 x 64 on 128-row tiles.  One K step is 64 = one quantization group.
// Per step the workgroup stages the activation tile (BM x 64 fp16) and the
// dequantized weight tile (BN x 64 fp16, produced from BN x 32 bytes of
// codes plus one scale and bias per column) into LDS; both are double
// buffered, and the global loads run two steps ahead, so one barrier per
// step suffices.  LDS rows are padded to 72 halves (144 bytes), which keeps
// the 128-bit staging writes and fragment reads free of bank conflicts.
//
// MFMA operand order: for one 16-wide K slice, lane l supplies row l % 32 of
// A and column l % 32 of B, each as 8 fp16 values; element v of half h = l/32
// is paired across A and B.  Any bijection between (h, v) and the 16 k of
// the slice therefore gives the same dot product.  Slice s of a K step uses
// k = 32h + 8s + v, so a lane's 8 values are one contiguous 16-byte chunk of
// an LDS row and one packed word of codes.  The weight fragment is the first
// MFMA operand, so the accumulators hold the tile transposed and a lane owns
// runs of 4 consecutive output columns; the epilogue bounces each wave's
// tile through LDS and writes whole 128-byte row segments.
//
// Tiles are dealt to the chip's 8 XCDs (each with its own L2) in contiguous
// runs, so tiles that share activation rows or an expert's weights run on
// the same XCD at about the same time.
#include <type_traits>

#include "ql_device.h"
#include "ql_codecs.h"
#include "ql_internal.h"

namespace ql {

namespace {

constexpr int kLdk = 72;  // padded LDS row length in fp16

enum : int { MODE_DENSE = 0, MODE_ROUTER = 1, MODE_GATEUP = 2, MODE_DOWN = 3 };

struct KParams {
    // A operand
    const uint16_t* A;  // rows of K fp16
    int64_t M;          // dense / router row count
    // B operand (w4)
    const uint32_t* qw;
    const uint16_t* sc;
    const uint16_t* bi;
    const uint32_t* sqw;  // shared expert (grouped modes)
    const uint16_t* ssc;
    const uint16_t* sbi;
    // B operand (fp16 [K][N], router)
    const uint16_t* Bh;
    // grouped routing
    const int* ws_header;
    const int* tiles;
    const int* short_order;  // short tiles by cost (indices after the tall ones)
    const int* sorted_assign;
    int max_tiles;  // routed tile slots in the grid
    int T, topk, E;
    // output
    uint16_t* Y;
    float* Yf;
    int K, N;
    int ksplit;  // router: number of K splits
    float gscale;           // NVFP4 weights: global scale (dense GEMM, shared expert)
    const float* gscales;   // NVFP4 experts: one global scale per expert (device)
    int grid_n, grid_m;  // dense: tile grid; grouped: N blocks (grid_n), shared tiles (grid_m)
};

// Work item of a workgroup when the grid is launched one-dimensional: the
// hardware deals workgroups to the 8 XCDs in turn (workgroup w to XCD w % 8),
// so item = (w % 8) * per + w / 8 gives every XCD one contiguous run of
// items.  Returns -1 for workgroups past the end.
__device__ __forceinline__ int xcd_item(int total) {
    const int per = (total + 7) >> 3;
    const int lin = blockIdx.x;
    const int idx = lin >> 3;
    const int item = (lin & 7) * per + idx;
    return (idx < per && item < total) ? item : -1;
}

// Workgroup of WGM x WGN waves; every wave owns (32*WM) x (32*WN) outputs.
template <int WM, int WN, int WGM, int WGN>
struct Tile {
    static constexpr int NT = 64 * WGM * WGN;           // threads per workgroup
    static constexpr int BM = 32 * WM * WGM;
    static constexpr int BN = 32 * WN * WGN;
    static constexpr int A_ROWS = NT / 8;                // A rows staged per 16-byte load round
    static constexpr int A_LOADS = BM / A_ROWS;          // 16-byte A loads per thread per step
    static constexpr int TPC = NT / BN;                  // threads per B column (1 or 2)
    static constexpr int WPT = 8 / TPC;                  // code words per thread per step
    static constexpr int LDS_A = BM * kLdk;              // fp16 per A buffer
    static constexpr int LDS_B = BN * kLdk;              // fp16 per B buffer
    static constexpr size_t LDS_BYTES = (size_t)2 * (LDS_A + LDS_B) * 2;
    static_assert(BM % A_ROWS == 0 && A_LOADS % 1 == 0, "A staging must tile the rows");
    static_assert(NT % BN == 0 && (TPC == 1 || TPC == 2), "one or two threads per B column");
};

// Waves holding at most this many 32 x 32 subtiles read a whole step's MFMA
// fragments at once (measured: 10% faster 64 x 128 tiles and router GEMM,
// no change for larger tiles, which cover the latency with their MFMAs).
constexpr int kEagerFragsMaxSubtiles = 4;

// One output tile for one workgroup: where its rows, columns, K range and
// weights come from.
struct Job {
    int rows_valid;   // rows of this tile that exist
    int out_row0;     // first output row
    int n0;           // first output column (act column for GATEUP)
    int kbeg, kend;   // K steps of this workgroup
    int tile_kind;    // grouped: 0 routed, 1 shared
    int tile_first;   // grouped: first row (routed r or shared token)
    int kz;           // router: index of the K split
    const uint32_t* wq;
    const uint16_t* ws;
    const uint16_t* wb;
    float gscale;     // NVFP4: global scale of this tile's matrix
};

// DT: 0 = fp16 activations, scales, biases, outputs and MFMA operands;
// 1 = bf16 throughout (the router's weight is then bf16 too; its logits
// stay fp32 partials in both cases).
// WF: weight format of the dense GEMM: 0 = w4 (codes, scale, bias);
// 1 = FP8-E4M3 codes [N][K] (bytes, through p.qw) with an fp16 scale per 64
// along K and no bias, staged as fp16(e4m3 * scale), one rounding;
// 2 = NVFP4: E2M1 codes in the w4 packing, E4M3 block scales [N][K/16]
// (bytes, through p.sc) and the matrix's global scale job.gscale, staged as
// fp16(e2m1 * (e4m3 * global)) with the block scale and the product in fp32
// and one rounding to fp16.
// KG: K groups.  With KG = 2 the workgroup holds two copies of the tile's
// waves; group g stages and multiplies K steps [kbeg + g*h, kbeg + (g+1)*h)
// (h = half the steps, their count must be even) in LDS of its own, so the
// two halves' latency chains run side by side on every SIMD, and group 1
// hands its fp32 sums to group 0 through LDS: each output is (sum over the
// first half) + (sum over the second half), rounded once.
template <int WM, int WN, int WGM, int WGN, int MODE, int DT = 0, int WF = 0, int KG = 1>
__device__ __forceinline__ void gemm_tile(const KParams& p, const Job& job, f16* lds_all) {
    using TL = Tile<WM, WN, WGM, WGN>;
    constexpr int BM = TL::BM, BN = TL::BN;
    static_assert(KG == 1 || (KG == 2 && MODE == MODE_DENSE), "K groups: dense GEMM only");
    // Group of this wave (uniform) and the thread's index inside its group.
    const int grp = (KG == 2) ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / TL::NT) : 0;
    f16* const lds = lds_all + (size_t)grp * (TL::LDS_BYTES / 2);
    f16* As = lds;                     // [2][BM][kLdk]
    f16* Bs = lds + 2 * TL::LDS_A;     // [2][BN][kLdk]

    const int tid = (int)threadIdx.x - grp * TL::NT;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wave_n = wave % WGN;
    const int wm0 = (wave / WGN) * (32 * WM);  // wave row offset in the tile
    const int wn0 = wave_n * (32 * WN);        // wave column offset in the tile
    const int K = p.K;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int rows_valid = job.rows_valid;
    const int out_row0 = job.out_row0;
    const int n0 = job.n0;
    const int khalf = (job.kend - job.kbeg) / KG;
    const int kbeg = job.kbeg + grp * khalf, kend = (KG == 2) ? kbeg + khalf : job.kend;
    const int tile_kind = job.tile_kind;
    const int tile_first = job.tile_first;
    const uint32_t* const wq = job.wq;
    const uint16_t* const ws = job.ws;
    const uint16_t* const wb = job.wb;
    (void)BM;

    // ---- A row sources (one per 32-row slab this thread stages) -------------
    const uint16_t* arow[TL::A_LOADS];
    const int a_chunk = tid & 7;
#pragma unroll
    for (int i = 0; i < TL::A_LOADS; ++i) {
        const int lr = min(i * TL::A_ROWS + (tid >> 3), rows_valid - 1);
        int64_t src;
        if constexpr (MODE == MODE_DENSE || MODE == MODE_ROUTER) {
            src = out_row0 + lr;
        } else if constexpr (MODE == MODE_GATEUP) {
            src = (tile_kind == 0) ? min(max(p.sorted_assign[tile_first + lr] / p.topk, 0), p.T - 1)
                                   : tile_first + lr;
        } else {
            src = out_row0 + lr;  // act rows are already in output order
        }
        arow[i] = p.A + src * K + a_chunk * 8;
    }

    // ---- B column source for this thread -------------------------------------
    const int bc = tid / TL::TPC;           // local column 0..BN-1
    const int bpart = tid % TL::TPC;        // which words of the column
    int bcol;
    if constexpr (MODE == MODE_GATEUP) {
        // Wave column block w holds WN/2 subtiles of gate then the matching
        // WN/2 subtiles of up, so a lane finds gate and up of the same output
        // column in subtiles ni and ni + WN/2.
        const int w = bc / (32 * WN);
        const int s = (bc % (32 * WN)) / 32;
        const int l = bc % 32;
        const int half = p.N / 2;
        bcol = n0 + w * (16 * WN) + (s % (WN / 2)) * 32 + l;
        bcol = min(bcol, half - 1) + ((s >= WN / 2) ? half : 0);
    } else {
        bcol = min(n0 + bc, p.N - 1);
    }

    f32x16 acc[WM][WN];
#pragma unroll
    for (int i = 0; i < WM; ++i)
#pragma unroll
        for (int j = 0; j < WN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    // Two register sets of staged global data: the loads of step i + 2 are
    // issued while step i + 1 (loaded one step earlier) is dequantized into
    // LDS and step i runs on the matrix cores.
    static_assert(WF == 0 || (DT == 0 && MODE != MODE_ROUTER), "codec weights: fp16 GEMMs");
    constexpr int BREG = (MODE == MODE_ROUTER) ? 1 : (WF == 1) ? TL::WPT / 2 : TL::WPT / 4;
    constexpr int HREG = (MODE == MODE_ROUTER) ? 8 : 1;
    u32x4 areg[2][TL::A_LOADS];
    u32x4 breg[2][BREG];
    uint16_t sreg[2] = {0, 0}, bireg[2] = {0, 0};
    uint32_t nreg[2] = {0, 0};  // NVFP4: the four block scales of a column's step
    // router B staging: an 8 x 8 block of fp16 per thread (8 rows of 16 bytes)
    u32x4 hreg[2][HREG];

    auto load_stage = [&](auto set, int ks) {
        constexpr int S = decltype(set)::value;
        const int k0 = ks * kGroup;
#pragma unroll
        for (int i = 0; i < TL::A_LOADS; ++i) areg[S][i] = ld_u32x4(arow[i] + k0);
        if constexpr (MODE == MODE_ROUTER) {
            // One 8 x 8 block per thread: k rows 8*kb .. 8*kb+7 of the step,
            // columns 8*nb .. 8*nb+7 of the tile.
            static_assert(BN == 256 && TL::NT == 256, "router staging: one 8 x 8 block per thread");
            const int kb = tid & 7, nb = tid >> 3;
            const int col = min(n0 + 8 * nb, p.N - 8);
#pragma unroll
            for (int r = 0; r < 8; ++r) hreg[S][r] = ld_u32x4(p.Bh + (size_t)(k0 + 8 * kb + r) * p.N + col);
        } else if constexpr (WF == 1) {
            // this thread's WPT * 8 codes of the column's 64 in this step
            const uint8_t* src = reinterpret_cast<const uint8_t*>(wq) + (size_t)bcol * K + k0 +
                                 bpart * TL::WPT * 8;
#pragma unroll
            for (int i = 0; i < BREG; ++i) breg[S][i] = ld_u32x4(src + 16 * i);
            sreg[S] = ws[(size_t)bcol * G + ks];
        } else {
            const uint32_t* src = wq + (size_t)bcol * wpr + ks * 8 + bpart * TL::WPT;
#pragma unroll
            for (int i = 0; i < BREG; ++i) breg[S][i] = ld_u32x4(src + 4 * i);
            if constexpr (WF == 2) {
                nreg[S] = *reinterpret_cast<const uint32_t*>(reinterpret_cast<const uint8_t*>(ws) +
                                                             (size_t)bcol * (K / 16) + ks * 4);
            } else {
                sreg[S] = ws[(size_t)bcol * G + ks];
                bireg[S] = wb[(size_t)bcol * G + ks];
            }
        }
    };

    // Stage one quarter (piece p of 4) of a step: A chunks and dequantized B
    // words from register set S into LDS buffer `buf`.
    auto store_piece = [&](auto set, int buf, auto piece) {
        constexpr int S = decltype(set)::value;
        constexpr int P = decltype(piece)::value;
        f16* a_dst = As + buf * TL::LDS_A;
#pragma unroll
        for (int i = P * TL::A_LOADS / 4; i < (P + 1) * TL::A_LOADS / 4; ++i)
            *reinterpret_cast<u32x4*>(a_dst + (i * TL::A_ROWS + (tid >> 3)) * kLdk + a_chunk * 8) = areg[S][i];
        f16* b_dst = Bs + buf * TL::LDS_B;
        if constexpr (MODE == MODE_ROUTER) {
            // Transpose the 8 x 8 block in registers: output row j (column
            // 8*nb + j) pairs element j of k rows (2i, 2i+1).
            const int kb = tid & 7, nb = tid >> 3;
#pragma unroll
            for (int j = 2 * P; j < 2 * P + 2; ++j) {
                const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
                u32x4 o;
                o.x = __builtin_amdgcn_perm(hreg[S][1][j >> 1], hreg[S][0][j >> 1], sel);
                o.y = __builtin_amdgcn_perm(hreg[S][3][j >> 1], hreg[S][2][j >> 1], sel);
                o.z = __builtin_amdgcn_perm(hreg[S][5][j >> 1], hreg[S][4][j >> 1], sel);
                o.w = __builtin_amdgcn_perm(hreg[S][7][j >> 1], hreg[S][6][j >> 1], sel);
                *reinterpret_cast<u32x4*>(b_dst + (8 * nb + j) * kLdk + 8 * kb) = o;
            }
        } else if constexpr (WF == 1) {
            // The E4M3 codes decode exactly to fp16 (NaN codes to NaN); one
            // packed fp16 multiply by the group's scale rounds each product
            // once: the weight is fp16(e4m3 * scale).
            const f16 sv = __builtin_bit_cast(f16, sreg[S]);
            const f16x2 s2 = {sv, sv};
            constexpr int W = TL::WPT;  // groups of 8 codes of this thread per step
#pragma unroll
            for (int w = P * W / 4; w < (P + 1) * W / 4; ++w) {
                const uint32_t c0 = breg[S][(2 * w) >> 2][(2 * w) & 3];
                const uint32_t c1 = breg[S][(2 * w + 1) >> 2][(2 * w + 1) & 3];
                u32x4 o;
                o.x = as_u32(e4m3x2_to_f16x2<false>(c0) * s2);
                o.y = as_u32(e4m3x2_to_f16x2<true>(c0) * s2);
                o.z = as_u32(e4m3x2_to_f16x2<false>(c1) * s2);
                o.w = as_u32(e4m3x2_to_f16x2<true>(c1) * s2);
                const int word = bpart * W + w;  // 0..7 within the group
                *reinterpret_cast<u32x4*>(b_dst + bc * kLdk + word * 8) = o;
            }
        } else if constexpr (WF == 2) {
            // The block scale e4m3 * global is formed in fp32, each E2M1 code
            // (exact) is multiplied by it in fp32 and the product is rounded
            // once to fp16.  This thread's words cover blocks starting at
            // (bpart * W) / 2 of the step's four.
            constexpr int W = TL::WPT;  // words of 8 codes of this thread per step
            const uint32_t nsh = nreg[S] >> (8 * ((bpart * W) >> 1));
            float bsc[(W + 1) / 2];
#pragma unroll
            for (int i = 0; i < (W + 1) / 2; ++i) bsc[i] = e4m3_to_f32<0>(nsh >> (8 * i)) * job.gscale;
#pragma unroll
            for (int w = P * W / 4; w < (P + 1) * W / 4; ++w) {
                const int word = bpart * W + w;  // 0..7 within the step: block word / 2
                const float sc = bsc[w >> 1];
                const uint32_t u = breg[S][w >> 2][w & 3];
                const f32x2 q0 = e2m1x2_to_f32x2<0>(u), q1 = e2m1x2_to_f32x2<1>(u);
                const f32x2 q2 = e2m1x2_to_f32x2<2>(u), q3 = e2m1x2_to_f32x2<3>(u);
                u32x4 o;
                o.x = f32x2_to_f16x2(q0[0] * sc, q0[1] * sc);
                o.y = f32x2_to_f16x2(q1[0] * sc, q1[1] * sc);
                o.z = f32x2_to_f16x2(q2[0] * sc, q2[1] * sc);
                o.w = f32x2_to_f16x2(q3[0] * sc, q3[1] * sc);
                *reinterpret_cast<u32x4*>(b_dst + bc * kLdk + word * 8) = o;
            }
        } else if constexpr (DT == 1) {
            const float sf = bf2f(sreg[S]), bf = bf2f(bireg[S]);
            constexpr int W = TL::WPT;  // words of this thread's column per step
#pragma unroll
            for (int w = P * W / 4; w < (P + 1) * W / 4; ++w) {
                const uint32_t u = breg[S][w >> 2][w & 3];
                const int word = bpart * W + w;  // 0..7 within the group
                *reinterpret_cast<u32x4*>(b_dst + bc * kLdk + word * 8) = dequant_word_bf16(u, sf, bf);
            }
        } else {
            const f16 sv = __builtin_bit_cast(f16, sreg[S]);
            const f16 bv = __builtin_bit_cast(f16, bireg[S]);
            const f16x2 s2 = {sv, sv};
            const f16x2 b2 = {bv, bv};
            constexpr int W = TL::WPT;  // words of this thread's column per step
#pragma unroll
            for (int w = P * W / 4; w < (P + 1) * W / 4; ++w) {
                const uint32_t u = breg[S][w >> 2][w & 3];
                const int word = bpart * W + w;  // 0..7 within the group
                *reinterpret_cast<f16x8*>(b_dst + bc * kLdk + word * 8) = dequant_word(u, s2, b2);
            }
        }
    };

    const int fl = lane & 31;   // row (A) / column (B) inside a 32-wide subtile
    const int fh = lane >> 5;   // which half of the 16-wide K slice
    // NA (compile time) = how many of the wave's WM row subtiles hold real
    // rows; the others are padding and get neither fragment reads nor MFMAs.
    auto read_frags = [&](auto na, int buf, int s, f16x8 (&af)[WM], f16x8 (&bf)[WN]) {
        constexpr int NA = decltype(na)::value;
        const f16* a_src = As + buf * TL::LDS_A + (wm0 + fl) * kLdk + (4 * fh + s) * 8;
        const f16* b_src = Bs + buf * TL::LDS_B + (wn0 + fl) * kLdk + (4 * fh + s) * 8;
#pragma unroll
        for (int i = 0; i < NA; ++i) af[i] = *reinterpret_cast<const f16x8*>(a_src + i * 32 * kLdk);
        if constexpr (NA > 0) {
#pragma unroll
            for (int j = 0; j < WN; ++j) bf[j] = *reinterpret_cast<const f16x8*>(b_src + j * 32 * kLdk);
        }
    };
    auto mfmas = [&](auto na, const f16x8 (&af)[WM], const f16x8 (&bf)[WN]) {
        constexpr int NA = decltype(na)::value;
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
            for (int j = 0; j < WN; ++j)
                if constexpr (DT == 1)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                        __builtin_bit_cast(bf16x8, bf[j]), __builtin_bit_cast(bf16x8, af[i]), acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
    };

    // One 16-wide K slice of step data in LDS buffer S: its MFMAs, a quarter
    // of the next step's staging (program order keeps the LDS stores after
    // this slice's fragment reads), then the next slice's fragment reads.
    // The compiler interleaves them; fixed interleaving hints measured slower.
    auto slice = [&](auto set, auto sl, auto na, f16x8 (&af)[WM], f16x8 (&bf)[WN], f16x8 (&an)[WM],
                     f16x8 (&bn)[WN]) {
        constexpr int S = decltype(set)::value;
        constexpr int SL = decltype(sl)::value;
        mfmas(na, af, bf);
        store_piece(std::integral_constant<int, S ^ 1>{}, S ^ 1, sl);
        if constexpr (SL < 3) read_frags(na, S, SL + 1, an, bn);
        __builtin_amdgcn_sched_barrier(0);
    };

    // The loop body for the step `i` (relative to kbeg) whose data sits in
    // LDS buffer S = i & 1.  Loads and stores past the last step are clamped
    // to the last step (harmless repeats) so that the body has no branches.
    auto body = [&](auto set, auto na, int i) {
        constexpr int S = decltype(set)::value;
        load_stage(set, min(kbeg + i + 2, kend - 1));
        if constexpr (WM * WN <= kEagerFragsMaxSubtiles) {
            // Few subtiles per wave: a slice's MFMAs are too short to cover
            // the LDS latency of the next slice's fragment reads, so all four
            // slices' fragments are read up front and the latency is paid
            // once per step.
            f16x8 af[4][WM], bf[4][WN];
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) read_frags(na, S, sl, af[sl], bf[sl]);
            auto run = [&](auto sl) {
                constexpr int SL = decltype(sl)::value;
                mfmas(na, af[SL], bf[SL]);
                store_piece(std::integral_constant<int, S ^ 1>{}, S ^ 1, sl);
                __builtin_amdgcn_sched_barrier(0);
            };
            run(std::integral_constant<int, 0>{});
            run(std::integral_constant<int, 1>{});
            run(std::integral_constant<int, 2>{});
            run(std::integral_constant<int, 3>{});
        } else {
            f16x8 a0[WM], b0[WN], a1[WM], b1[WN];
            read_frags(na, S, 0, a0, b0);
            slice(set, std::integral_constant<int, 0>{}, na, a0, b0, a1, b1);
            slice(set, std::integral_constant<int, 1>{}, na, a1, b1, a0, b0);
            slice(set, std::integral_constant<int, 2>{}, na, a0, b0, a1, b1);
            slice(set, std::integral_constant<int, 3>{}, na, a1, b1, a0, b0);
        }
        __syncthreads();
    };

    auto store_stage = [&](auto set, int buf) {
        store_piece(set, buf, std::integral_constant<int, 0>{});
        store_piece(set, buf, std::integral_constant<int, 1>{});
        store_piece(set, buf, std::integral_constant<int, 2>{});
        store_piece(set, buf, std::integral_constant<int, 3>{});
    };

    const std::integral_constant<int, 0> set0{};
    const std::integral_constant<int, 1> set1{};
    const int nk = kend - kbeg;
    if (nk > 0) {
        load_stage(set0, kbeg);
        store_stage(set0, 0);
        load_stage(set1, min(kbeg + 1, kend - 1));
    }
    __syncthreads();
    auto main_loop = [&](auto na) {
        int i = 0;
        for (; i + 1 < nk; i += 2) {
            body(set0, na, i);
            body(set1, na, i + 1);
        }
        if (i < nk) body(set0, na, i);
    };
    if constexpr ((MODE == MODE_GATEUP || MODE == MODE_DOWN) && WM == 2) {
        // Short routed tiles end in padding rows; every wave still stages its
        // share (the barriers are reached by all), but skips subtiles past
        // the end.  (Tall routed tiles are always full.)
        const int na = __builtin_amdgcn_readfirstlane(min(max((rows_valid - wm0 + 31) / 32, 0), WM));
        if (na >= 2) main_loop(std::integral_constant<int, 2>{});
        else if (na == 1) main_loop(std::integral_constant<int, 1>{});
        else main_loop(std::integral_constant<int, 0>{});
    } else {
        main_loop(std::integral_constant<int, WM>{});
    }
    // Only group 0 writes outputs; group 1 still passes every barrier below.
    const bool writer = (grp == 0);
    if constexpr (KG == 2) {
        // Group 1's sums to group 0 through LDS (the staging buffers are
        // free once both groups pass the barrier): [i][j][r][thread].
        __syncthreads();
        float* const xch = reinterpret_cast<float*>(lds_all);
        static_assert((size_t)TL::NT * WM * WN * 16 * 4 <= (size_t)TL::LDS_BYTES, "exchange fits");
        if (!writer) {
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) xch[((i * WN + j) * 16 + r) * TL::NT + tid] = acc[i][j][r];
        }
        __syncthreads();
        if (writer) {
#pragma unroll
            for (int i = 0; i < WM; ++i)
#pragma unroll
                for (int j = 0; j < WN; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        acc[i][j][r] = acc[i][j][r] + xch[((i * WN + j) * 16 + r) * TL::NT + tid];
        }
    }

    // ---- epilogue -------------------------------------------------------------
    auto to16 = [](float v) -> uint16_t {
        if constexpr (DT == 1) return f2bf(v);
        else return f2h(v);
    };
    // The MFMAs take the weight fragment as their first operand, so each
    // accumulator holds the transposed product: acc[i][j][r] is output row
    // 32i + l%32 of the wave tile and column 32j + 8(r/4) + 4h + r%4.  A lane
    // thus owns runs of 4 consecutive columns of one row.
    const int out_cols = (MODE == MODE_GATEUP) ? p.N / 2 : p.N;
    // Output columns of one wave per row subtile.
    constexpr int WC = (MODE == MODE_GATEUP) ? 16 * WN : 32 * WN;
    auto out_vals = [&](int i, int j, int g, float (&v)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
    };
    // 16-bit outputs; gate/up: silu(gate) * up, rounded once to fp16.
    auto out16 = [&](int i, int j, int g, uint16_t (&h)[4]) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (MODE == MODE_GATEUP) {
                const float gt = silu(acc[i][j][4 * g + e]), up = acc[i][j + WN / 2][4 * g + e];
                if constexpr (DT == 1) h[e] = f2bf(gt * up);
                else h[e] = mul_to_f16(gt, up);
            } else {
                h[e] = to16(acc[i][j][4 * g + e]);
            }
        }
    };
    const int wcol0 = (MODE == MODE_GATEUP) ? n0 + wave_n * (16 * WN) : n0 + wn0;
    if constexpr (MODE == MODE_ROUTER) {
        // fp32 partials: four consecutive experts are one 16-byte store
        // (E % 8 == 0 on this path).
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            const int lrow = wm0 + 32 * i + fl;
            if (lrow >= rows_valid) continue;
            const int64_t orow = (int64_t)out_row0 + lrow;
#pragma unroll
            for (int j = 0; j < WN; ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    float v[4];
                    out_vals(i, j, g, v);
                    const int col = wcol0 + 32 * j + 8 * g + 4 * fh;
                    if (col < out_cols)
                        *reinterpret_cast<f32x4*>(p.Yf + (orow * p.ksplit + job.kz) * out_cols + col) =
                            f32x4{v[0], v[1], v[2], v[3]};
                }
        }
    } else if ((out_cols & 7) == 0 && ((uintptr_t)p.Y & 15) == 0) {
        // Each wave bounces one 32-row subtile at a time through its own LDS
        // region (two regions, alternating), then writes whole row segments:
        // 16-byte stores, 8 lanes per 128 bytes of a row.
        constexpr int LDR = WC + 8;                   // padded row, fp16
        constexpr int CPR = WC / 8;                   // 16-byte chunks per row
        static_assert(2 * 32 * LDR * (TL::NT / 64) <= TL::LDS_A * 2 + TL::LDS_B * 2,
                      "epilogue regions fit in the staging buffers");
        static_assert((32 * CPR) % 64 == 0, "whole chunks per lane");
        __syncthreads();  // every wave is done with the staging buffers
        f16* const region0 = lds + (size_t)wave * 2 * 32 * LDR;
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            f16* const reg = region0 + (i & 1) * 32 * LDR;
            if (writer) {
#pragma unroll
                for (int j = 0; j < ((MODE == MODE_GATEUP) ? WN / 2 : WN); ++j)
#pragma unroll
                    for (int g = 0; g < 4; ++g) {
                        uint16_t h[4];
                        out16(i, j, g, h);
                        const uint32_t lo = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
                        const uint32_t hi = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
                        *reinterpret_cast<uint2*>(reg + fl * LDR + 32 * j + 8 * g + 4 * fh) = make_uint2(lo, hi);
                    }
            }
            __syncthreads();
            if (writer) {
#pragma unroll
                for (int q = 0; q < 32 * CPR / 64; ++q) {
                    const int c = q * 64 + lane;
                    const int row = c / CPR, ch = c % CPR;
                    const int lrow = wm0 + 32 * i + row;
                    const int col = wcol0 + ch * 8;
                    const u32x4 d = *reinterpret_cast<const u32x4*>(reg + row * LDR + ch * 8);
                    if (lrow < rows_valid && col < out_cols)
                        *reinterpret_cast<u32x4*>(p.Y + ((int64_t)out_row0 + lrow) * out_cols + col) = d;
                }
            }
        }
    } else if (writer) {
        // Unaligned output: element stores.
#pragma unroll
        for (int i = 0; i < WM; ++i) {
            const int lrow = wm0 + 32 * i + fl;
            if (lrow >= rows_valid) continue;
            uint16_t* const yrow = p.Y + ((int64_t)out_row0 + lrow) * out_cols;
#pragma unroll
            for (int j = 0; j < ((MODE == MODE_GATEUP) ? WN / 2 : WN); ++j)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint16_t h[4];
                    out16(i, j, g, h);
                    const int col = wcol0 + 32 * j + 8 * g + 4 * fh;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        if (col + e < out_cols) yrow[col + e] = h[e];
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Few-row GEMM, weight-stationary.  A workgroup of 8 waves owns 32 output
// columns; wave w owns K range [w*K/8, (w+1)*K/8) of them (GW groups).  The
// wave dequantizes its 32 x (K/8) weight block once into MFMA operand
// registers (fp16 s*q + b, one rounding, as everywhere else) and then
// streams the activation rows past it, 32 rows per chunk (the next chunk's
// fragments load while the current one runs): they come straight from
// global memory (small and shared by every workgroup, so they stay in L2),
// MFMA 32x32x16 with the activations as the first operand, and the 8 K
// partials of each output are summed in LDS in wave order (a fixed order,
// so results are deterministic).  Every weight byte is read and dequantized
// exactly once; the activations are read once per 32 output columns, which
// is what bounds this kernel as M grows (the tiled GEMM reads them once per
// 256 columns), so it is the choice for few rows only.
// ---------------------------------------------------------------------------
constexpr int kWsCols = 32;  // output columns per workgroup
constexpr int kWsWaves = 8;  // K slices per workgroup

template <int GW>
__global__ void __launch_bounds__(64 * kWsWaves)
gemm_ws_kernel(const uint16_t* __restrict__ X, const uint32_t* __restrict__ qw,
               const uint16_t* __restrict__ sc, const uint16_t* __restrict__ bi,
               uint16_t* __restrict__ Y, int64_t M, int K, int N) {
    __shared__ __align__(16) float red[kWsWaves][kWsCols][32 + 4];  // [wave][col][row]
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int fl = lane & 31, fh = lane >> 5;
    const int G = K / kGroup;
    const int wpr = K / 8;
    const int n0 = blockIdx.x * kWsCols;
    const int col = min(n0 + fl, N - 1);
    const int g0 = wave * GW;  // first group of this wave

    // Weight block: group g, slice s -> 8 fp16 weights of k = 64(g0+g) + 32h + 8s + v.
    f16x8 wf[GW][4];
    {
        u32x4 cw[GW];
        uint16_t sv[GW], bv[GW];
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            cw[g] = ld_stream_u32x4(qw + (size_t)col * wpr + (g0 + g) * 8 + 4 * fh);
            sv[g] = sc[(size_t)col * G + g0 + g];
            bv[g] = bi[(size_t)col * G + g0 + g];
        }
#pragma unroll
        for (int g = 0; g < GW; ++g) {
            const f16 s1 = __builtin_bit_cast(f16, sv[g]), b1 = __builtin_bit_cast(f16, bv[g]);
            const f16x2 s2 = {s1, s1}, b2 = {b1, b1};
#pragma unroll
            for (int sl = 0; sl < 4; ++sl) wf[g][sl] = dequant_word(cw[g][sl], s2, b2);
        }
    }

    const int64_t nchunks = (M + 31) / 32;
    auto load_x = [&](int64_t c, f16x8 (&xf)[GW][4]) {
        const int64_t row = min(c * 32 + fl, M - 1);
        const uint16_t* xr = X + row * K + (size_t)g0 * kGroup + 32 * fh;
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int sl = 0; sl < 4; ++sl)
                xf[g][sl] = __builtin_bit_cast(f16x8, ld_u32x4(xr + g * kGroup + 8 * sl));
    };
    f16x8 xa[GW][4], xb[GW][4];
    auto chunk = [&](int64_t c, f16x8 (&xf)[GW][4], f16x8 (&xn)[GW][4]) {
        if (c + 1 < nchunks) load_x(c + 1, xn);  // next chunk's activations in flight
        f32x16 acc;
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
        for (int g = 0; g < GW; ++g)
#pragma unroll
            for (int sl = 0; sl < 4; ++sl)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xf[g][sl], wf[g][sl], acc, 0, 0, 0);
        // acc[r]: row 8(r/4) + 4h + r%4 of the chunk, column l%32.
#pragma unroll
        for (int q = 0; q < 4; ++q)
            *reinterpret_cast<f32x4*>(&red[wave][fl][8 * q + 4 * fh]) =
                f32x4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
        __syncthreads();
        // 1024 outputs of the chunk, two adjacent columns of one row per thread.
        const int orow = tid >> 4, ocol = (tid & 15) * 2;
        float s0 = 0.f, s1 = 0.f;
#pragma unroll
        for (int w = 0; w < kWsWaves; ++w) {
            s0 += red[w][ocol][orow];
            s1 += red[w][ocol + 1][orow];
        }
        const int64_t m = c * 32 + orow;
        const int n = n0 + ocol;
        if (m < M) {
            uint16_t* yp = Y + m * N + n;
            if (n + 1 < N && ((N & 1) == 0) && ((uintptr_t)Y & 3) == 0) {
                *reinterpret_cast<uint32_t*>(yp) = (uint32_t)f2h(s0) | ((uint32_t)f2h(s1) << 16);
            } else {
                if (n < N) yp[0] = f2h(s0);
                if (n + 1 < N) yp[1] = f2h(s1);
            }
        }
        __syncthreads();  // red is rewritten by the next chunk
    };
    load_x(0, xa);
    int64_t c = 0;
    for (; c + 1 < nchunks; c += 2) {
        chunk(c, xa, xb);
        chunk(c + 1, xb, xa);
    }
    if (c < nchunks) chunk(c, xa, xb);
}

// Dense prefill GEMM and the router GEMM (KG: K groups, see gemm_tile).
template <int WM, int WN, int WGM, int WGN, int MODE, int DT, int WF = 0, int KG = 1>
__global__ void __launch_bounds__(64 * WGM * WGN * KG)
gemm_w4_kernel(const KParams p) {
    using TL = Tile<WM, WN, WGM, WGN>;
    constexpr int BM = TL::BM, BN = TL::BN;
    extern __shared__ __align__(16) f16 lds[];
    const int G = p.K / kGroup;
    Job job{};
    job.kbeg = 0;
    job.kend = G;
    job.gscale = p.gscale;
    job.wq = p.qw;
    job.ws = p.sc;
    job.wb = p.bi;
    if constexpr (MODE == MODE_DENSE) {
        const int item = xcd_item(p.grid_n * p.grid_m);
        if (item < 0) return;
        // Inside an XCD's run, groups of 4 row blocks sweep the column blocks
        // together, so concurrent tiles share both activation rows and weights.
        constexpr int GM = 4;
        const int in_group = GM * p.grid_n;
        const int first_m = (item / in_group) * GM;
        const int gm = min(p.grid_m - first_m, GM);
        const int r = item % in_group;
        job.n0 = (r / gm) * BN;
        job.out_row0 = (first_m + r % gm) * BM;
    } else {
        static_assert(MODE == MODE_ROUTER, "dense or router");
        job.n0 = blockIdx.y * BN;
        job.out_row0 = blockIdx.x * BM;
        const int per = (G + p.ksplit - 1) / p.ksplit;
        job.kbeg = blockIdx.z * per;
        job.kend = min(G, job.kbeg + per);
        job.kz = blockIdx.z;
    }
    job.rows_valid = (int)min<int64_t>(BM, p.M - job.out_row0);
    gemm_tile<WM, WN, WGM, WGN, MODE, DT, WF, KG>(p, job, lds);
}

// ---------------------------------------------------------------------------
// Routed tile of at most 32 rows (a lightly loaded expert).  In the staged
// tile such an expert costs as much per K step as a full one, and its time
// goes to streaming the weights with only two K steps of loads in flight.
// Here the tile's activation rows (32 x K fp16, at most 128 KB) are staged
// into LDS once, behind a single barrier, and each of the 8 waves owns 32
// weight columns (gate/up: 16 gate columns and the 16 matching up columns)
// over the whole K: every lane streams its own fragment's codes (16 bytes per
// K step, 32 for FP8) straight into registers, 16 K steps ahead (8 for FP8),
// decodes them in registers exactly as the staged tile does and issues the
// same MFMAs on the same operand layout in the same order (weights first,
// k = 32h + 8s + v in slice s, slices and steps ascending), so every output
// bit is the same.  G = K / 64 is a template argument (8, 16 or 32) so that
// the K loop unrolls and every register ring index is static; the scales
// (and biases) of the whole K sit in registers.
// ---------------------------------------------------------------------------
constexpr int kTinyRows = kTinyTileRows;

__host__ __device__ constexpr size_t tiny_lds_bytes(int K) { return (size_t)kTinyRows * (K + 8) * 2; }

// Byte b (0..3) of w as E4M3 / its two E2M1 codes as fp32; b is a constant
// after unrolling.
__device__ __forceinline__ float e4m3_byte(uint32_t w, int b) {
    switch (b) {
        case 0: return e4m3_to_f32<0>(w);
        case 1: return e4m3_to_f32<1>(w);
        case 2: return e4m3_to_f32<2>(w);
        default: return e4m3_to_f32<3>(w);
    }
}

// WF: weight format as in gemm_tile (0 w4, 1 FP8-E4M3, 2 NVFP4).
template <int MODE, int DT, int G, int WF>
__device__ __forceinline__ void tiny_tile(const KParams& p, const Job& job, f16* lds) {
    constexpr int K = G * kGroup, wpr = K / 8;
    constexpr int LDR = K + 8;  // padded LDS row (fp16): 16-byte fragment reads of 32 rows hit distinct banks
    static_assert(G == 8 || G == 16 || G == 32, "tiny tile: K of 512, 1024 or 2048");
    static_assert(WF == 0 || DT == 0, "codec weights: fp16 activations");
    // K steps of code loads in flight per lane (FP8 codes take twice the registers).
    constexpr int AHEAD = (WF == 1) ? 8 : 16;
    constexpr int AH = AHEAD < G ? AHEAD : G;
    constexpr int CW = (WF == 1) ? 2 : 1;  // 16-byte code loads per lane and step
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int fl = lane & 31, fh = lane >> 5;
    // This lane's weight column (first MFMA operand row fl).
    int bcol;
    if constexpr (MODE == MODE_GATEUP) {
        const int half = p.N / 2;
        bcol = min(job.n0 + wave * 16 + (fl & 15), half - 1) + ((fl >= 16) ? half : 0);
    } else {
        bcol = min(job.n0 + wave * 32 + fl, p.N - 1);
    }
    // w4 / NVFP4: words 4h .. 4h+3 of a step (word 4h + s = slice s); FP8:
    // bytes 32h .. 32h+31 of a step (bytes 32h + 8s .. +7 = slice s).
    const uint32_t* const wrow = (WF == 1) ? job.wq + ((size_t)bcol * K + 32 * fh) / 4
                                           : job.wq + (size_t)bcol * wpr + 4 * fh;
    constexpr int WSTEP = (WF == 1) ? kGroup / 4 : 8;  // u32 words per K step of one column

    // Code loads of the first AH steps go out first.
    u32x4 cw[AH][CW];
#pragma unroll
    for (int d = 0; d < AH; ++d)
#pragma unroll
        for (int c = 0; c < CW; ++c) cw[d][c] = ld_u32x4(wrow + d * WSTEP + 4 * c);
    // Scales (and biases) of the whole K: fp16 per step, eight steps per
    // 16-byte load (w4, FP8); NVFP4: E4M3 block-scale bytes, four steps per
    // 16-byte load.
    constexpr int NS = (WF == 2) ? G / 4 : G / 8;
    u32x4 s8[NS], b8[(WF == 0) ? G / 8 : 1];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
        if constexpr (WF == 2)
            s8[i] = ld_u32x4(reinterpret_cast<const uint8_t*>(job.ws) + (size_t)bcol * (K / 16) + 16 * i);
        else
            s8[i] = ld_u32x4(job.ws + (size_t)bcol * G + 8 * i);
        if constexpr (WF == 0) b8[i] = ld_u32x4(job.wb + (size_t)bcol * G + 8 * i);
    }
    // Activation rows -> LDS: 16 threads per row (32 rows), each loading
    // every 16th 16-byte chunk of it; padding rows repeat the last real row
    // (their outputs are not stored).
    {
        constexpr int CPT = K / 8 / 16;  // chunks per thread
        const int r = tid >> 4, c0 = tid & 15;
        const int lr = min(r, job.rows_valid - 1);
        int64_t src_row;
        if constexpr (MODE == MODE_GATEUP)
            src_row = min(max(p.sorted_assign[job.tile_first + lr] / p.topk, 0), p.T - 1);
        else
            src_row = job.out_row0 + lr;
        const uint16_t* const xr = p.A + src_row * K;
        u32x4 st[CPT];
#pragma unroll
        for (int i = 0; i < CPT; ++i) st[i] = ld_u32x4(xr + (c0 + 16 * i) * 8);
#pragma unroll
        for (int i = 0; i < CPT; ++i) *reinterpret_cast<u32x4*>(lds + r * LDR + (c0 + 16 * i) * 8) = st[i];
    }
    __syncthreads();

    const f16* const arow = lds + fl * LDR + 32 * fh;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < G; ++ks) {
        const int set = ks % AH;
        f16x8 xf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) xf[s] = *reinterpret_cast<const f16x8*>(arow + ks * kGroup + 8 * s);
        f16x8 wf[4];
        if constexpr (WF == 1) {
            // fp16(e4m3 * scale): exact decode, one packed fp16 multiply.
            const uint32_t sw = s8[ks / 8][(ks % 8) / 2] >> (16 * (ks & 1));
            const f16 sv = __builtin_bit_cast(f16, (uint16_t)sw);
            const f16x2 s2 = {sv, sv};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const uint32_t c0 = cw[set][s >> 1][2 * (s & 1)], c1 = cw[set][s >> 1][2 * (s & 1) + 1];
                u32x4 o;
                o.x = as_u32(e4m3x2_to_f16x2<false>(c0) * s2);
                o.y = as_u32(e4m3x2_to_f16x2<true>(c0) * s2);
                o.z = as_u32(e4m3x2_to_f16x2<false>(c1) * s2);
                o.w = as_u32(e4m3x2_to_f16x2<true>(c1) * s2);
                wf[s] = __builtin_bit_cast(f16x8, o);
            }
        } else if constexpr (WF == 2) {
            // fp16(e2m1 * (e4m3 * global)) with the products in fp32; the
            // block of slice s (k = 32h + 8s ..) is byte 2h + s/2 of the step.
            const uint32_t nw = s8[ks / 4][ks % 4] >> (16 * fh);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float sc = e4m3_byte(nw, s >> 1) * job.gscale;
                const uint32_t u = cw[set][0][s];
                const f32x2 q0 = e2m1x2_to_f32x2<0>(u), q1 = e2m1x2_to_f32x2<1>(u);
                const f32x2 q2 = e2m1x2_to_f32x2<2>(u), q3 = e2m1x2_to_f32x2<3>(u);
                u32x4 o;
                o.x = f32x2_to_f16x2(q0[0] * sc, q0[1] * sc);
                o.y = f32x2_to_f16x2(q1[0] * sc, q1[1] * sc);
                o.z = f32x2_to_f16x2(q2[0] * sc, q2[1] * sc);
                o.w = f32x2_to_f16x2(q3[0] * sc, q3[1] * sc);
                wf[s] = __builtin_bit_cast(f16x8, o);
            }
        } else {
            const uint32_t sw = s8[ks / 8][(ks % 8) / 2] >> (16 * (ks & 1));
            const uint32_t bw = b8[ks / 8][(ks % 8) / 2] >> (16 * (ks & 1));
            if constexpr (DT == 1) {
                const float sf = bf2f((uint16_t)sw), bf = bf2f((uint16_t)bw);
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    wf[s] = __builtin_bit_cast(f16x8, dequant_word_bf16(cw[set][0][s], sf, bf));
            } else {
                const f16 s1 = __builtin_bit_cast(f16, (uint16_t)sw), b1 = __builtin_bit_cast(f16, (uint16_t)bw);
                const f16x2 s2 = {s1, s1}, b2 = {b1, b1};
#pragma unroll
                for (int s = 0; s < 4; ++s) wf[s] = dequant_word(cw[set][0][s], s2, b2);
            }
        }
        if (ks + AH < G) {
#pragma unroll
            for (int c = 0; c < CW; ++c) cw[set][c] = ld_u32x4(wrow + (ks + AH) * WSTEP + 4 * c);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if constexpr (DT == 1)
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, wf[s]),
                                                               __builtin_bit_cast(bf16x8, xf[s]), acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(wf[s], xf[s], acc, 0, 0, 0);
        }
    }

    // acc[r] = output (weight column 8(r/4) + 4h + r%4 of the wave's 32,
    // activation row fl).  Gate/up: columns c and c + 16 are gate and up of
    // one output column, i.e. acc[r] and acc[r + 8] for r < 8.
    if (fl >= job.rows_valid) return;
    auto to16 = [](float v) -> uint16_t {
        if constexpr (DT == 1) return f2bf(v);
        else return f2h(v);
    };
    const int out_cols = (MODE == MODE_GATEUP) ? p.N / 2 : p.N;
    const int wcol0 = job.n0 + wave * ((MODE == MODE_GATEUP) ? 16 : 32);
    uint16_t* const yrow = p.Y + ((int64_t)job.out_row0 + fl) * out_cols;
    const bool vec = (out_cols & 3) == 0 && ((uintptr_t)p.Y & 7) == 0;
    constexpr int NG = (MODE == MODE_GATEUP) ? 2 : 4;  // runs of 4 columns per lane
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        uint16_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            if constexpr (MODE == MODE_GATEUP) {
                const float gt = silu(acc[4 * g + e]), up = acc[4 * g + e + 8];
                if constexpr (DT == 1) h[e] = f2bf(gt * up);
                else h[e] = mul_to_f16(gt, up);
            } else {
                h[e] = to16(acc[4 * g + e]);
            }
        }
        const int col = wcol0 + 8 * g + 4 * fh;
        if (vec) {
            if (col < out_cols)
                *reinterpret_cast<uint2*>(yrow + col) =
                    make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
                if (col + e < out_cols) yrow[col + e] = h[e];
        }
    }
}

// Grouped expert GEMM over the load-matched tile map: tall tiles (256 rows,
// 8 waves of 128 x 64) and short tiles (128 rows, 8 waves of 64 x 64), both
// 256 columns wide, in one launch; short routed tiles of at most 32 rows
// (K of 512, 1024 or 2048) take tiny_tile instead.  The tall class (tall
// routed tiles, then the shared expert's tiles) comes first in the grid,
// dealt to the XCDs in contiguous runs of (tile, column block) items; then
// the short class, whole tiles dealt to the XCDs in turn in the order the
// dispatch wrote (wider tiles before tiny ones), so that every XCD gets an
// equal share of each kind and starts its cheapest items last.
using TallTile = Tile<4, 2, 2, 4>;
using ShortTile = Tile<2, 2, 2, 4>;
static_assert(TallTile::NT == ShortTile::NT && TallTile::BN == ShortTile::BN, "one workgroup shape");
static_assert(ShortTile::BM == QL_MOE_TILE_ROWS && TallTile::BM == 2 * QL_MOE_TILE_ROWS,
              "tile heights of the tile map");
constexpr size_t kGroupedLds =
    TallTile::LDS_BYTES > ShortTile::LDS_BYTES ? TallTile::LDS_BYTES : ShortTile::LDS_BYTES;
static_assert(tiny_lds_bytes(2048) <= kGroupedLds, "tiny tiles stage their rows in the grouped launch's LDS");

// WF = 1: FP8 experts (codes [E][N][K] bytes through p.qw, fp16 scales
// [E][N][K/64] through p.sc, no biases); WF = 2: NVFP4 experts (codes as the
// w4 words, E4M3 block scales [E][N][K/16] bytes through p.sc, global
// scales p.gscales[E]; the shared expert's is p.gscale).
template <int MODE, int DT, int WF = 0>
__global__ void __launch_bounds__(TallTile::NT)
gemm_w4_grouped_kernel(const KParams p) {
    extern __shared__ __align__(16) f16 lds[];
    const int G = p.K / kGroup;
    const int wpr = p.K / 8;
    const int NB = p.grid_n;  // column blocks
    // No header: the shared expert's tiles only.
    const int nt = p.ws_header ? min(max(p.ws_header[0], 0), p.max_tiles) : 0;
    const int nbig = p.ws_header ? min(max(p.ws_header[3], 0), nt) : 0;
    const int big_items = (nbig + p.grid_m) * NB;  // grid_m: shared-expert tiles
    const int nshort = nt - nbig;
    const int per_b = (big_items + 7) >> 3;
    const int lin = blockIdx.x;
    bool tall;
    int tslot, nblk;
    if (lin < 8 * per_b) {
        const int item = (lin & 7) * per_b + (lin >> 3);
        if (item >= big_items) return;
        tall = true;
        tslot = item / NB;
        nblk = item % NB;
    } else {
        // Short tiles are dealt to the XCDs in turn in the order of
        // short_order (the costlier ones first), all column blocks of a tile
        // on one XCD: the workgroups an XCD starts last are its cheapest.
        const int l2 = lin - 8 * per_b;
        const int idx = l2 >> 3;
        const int pos = (l2 & 7) + 8 * (idx / NB);
        if (pos >= nshort) return;
        tall = false;
        tslot = nbig + min(max(p.short_order[pos], 0), nshort - 1);
        nblk = idx % NB;
    }
    const int height = tall ? TallTile::BM : ShortTile::BM;
    Job job{};
    job.kbeg = 0;
    job.kend = G;
    if (tall && tslot >= nbig) {
        job.tile_kind = 1;
        job.tile_first = (tslot - nbig) * height;
        job.rows_valid = min(height, p.T - job.tile_first);
        job.out_row0 = p.T * p.topk + job.tile_first;
        job.wq = p.sqw;
        job.ws = p.ssc;
        job.wb = p.sbi;
        job.gscale = p.gscale;
    } else {
        const int* tp = p.tiles + (size_t)tslot * 4;
        // Clamped so that a corrupted tile map can never index out of bounds.
        const int e = min(max(tp[0], 0), p.E - 1);
        job.rows_valid = min(min(max(tp[2], 1), height), p.T * p.topk);
        job.tile_first = min(max(tp[1], 0), p.T * p.topk - job.rows_valid);
        job.out_row0 = job.tile_first;
        // u32 words per expert: N * K / 8 (w4 and NVFP4 codes) or N * K / 4
        // (FP8 bytes); 16-bit words of scales: N * K / 64, or N * K / 32 for
        // the NVFP4 block-scale bytes
        job.wq = p.qw + (size_t)e * p.N * (WF == 1 ? 2 * wpr : wpr);
        job.ws = p.sc + (size_t)e * p.N * (WF == 2 ? 2 * G : G);
        job.wb = (WF == 0) ? p.bi + (size_t)e * p.N * G : nullptr;
        if constexpr (WF == 2) job.gscale = p.gscales[e];
    }
    job.n0 = nblk * ((MODE == MODE_GATEUP) ? TallTile::BN / 2 : TallTile::BN);
    if (!tall && job.rows_valid <= kTinyRows) {
        if (G == 32) { tiny_tile<MODE, DT, 32, WF>(p, job, lds); return; }
        if (G == 16) { tiny_tile<MODE, DT, 16, WF>(p, job, lds); return; }
        if (G == 8) { tiny_tile<MODE, DT, 8, WF>(p, job, lds); return; }
    }
    if (tall)
        gemm_tile<4, 2, 2, 4, MODE, DT, WF>(p, job, lds);
    else
        gemm_tile<2, 2, 2, 4, MODE, DT, WF>(p, job, lds);
}

template <int WM, int WN, int WGM, int WGN, int MODE, int DT = 0, int WF = 0, int KG = 1>
int launch_t(const KParams& p, dim3 grid, hipStream_t st) {
    using TL = Tile<WM, WN, WGM, WGN>;
    static std::atomic<uint32_t> lds_set{0};
    if (const int rc = set_max_dynamic_lds((const void*)gemm_w4_kernel<WM, WN, WGM, WGN, MODE, DT, WF, KG>,
                                           TL::LDS_BYTES * KG, lds_set))
        return rc;
    hipLaunchKernelGGL((gemm_w4_kernel<WM, WN, WGM, WGN, MODE, DT, WF, KG>), grid, dim3(TL::NT * KG),
                       TL::LDS_BYTES * KG, st, p);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

}  // namespace

template <int DT, int WF = 0>
int launch_gemm_dt(const GemmArgs& a, hipStream_t st) {
    KParams p{};
    p.A = a.X;
    p.M = a.M;
    p.qw = a.qweight;
    p.sc = a.scales;
    p.bi = a.biases;
    p.Y = a.Y;
    p.K = a.K;
    p.N = a.N;
    p.gscale = a.gscale;
    // One-dimensional grid of tiles, rounded up to whole XCD rounds.
    auto grid_for = [&](int bm, int bn, dim3& grid) {
        const int64_t gn = (a.N + bn - 1) / bn, gm = (a.M + bm - 1) / bm;
        if (gn * gm > 0x7fffff00LL) return false;
        p.grid_n = (int)gn;
        p.grid_m = (int)gm;
        grid = dim3((unsigned)((gn * gm + 7) / 8 * 8));
        return true;
    };
    // Tile shape from a static table keyed by the number of 128 x 128 output
    // tiles (measured on MI355X for K = 512 and 2048, N = 1024 to 8192, M =
    // 128 to 4096): the largest tile that still gives the 256 CUs enough
    // workgroups.  Every shape accumulates each output element over the same
    // K steps in the same order, so the choice never changes a result bit.
    const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    dim3 grid;
#define QL_DENSE(A, B, C, D)                                                       \
    do {                                                                           \
        using TL = Tile<A, B, C, D>;                                               \
        if (!grid_for(TL::BM, TL::BN, grid)) return QL_ERR_UNSUPPORTED_SHAPE;      \
        return launch_t<A, B, C, D, MODE_DENSE, DT, WF>(p, grid, st);              \
    } while (0)
    if (t128 > 512) QL_DENSE(4, 2, 2, 4);  // 256 x 256, 8 waves of 128 x 64
    if (t128 > 256) QL_DENSE(2, 2, 2, 4);  // 128 x 256, 8 waves of 64 x 64
    if (t128 > 128) QL_DENSE(2, 2, 2, 2);  // 128 x 128, 4 waves of 64 x 64
    // At most 128 tiles of 64 x 128 leave CUs idle: 64 x 64 tiles of two
    // waves double the workgroups (each activation row is then staged once
    // per 64 columns instead of 128, which costs more than it gains once
    // the 64 x 128 grid fills the chip).
    if (((a.M + 63) / 64) * ((a.N + 127) / 128) <= 128) QL_DENSE(1, 2, 2, 1);  // 64 x 64, 2 waves of 32 x 64
    QL_DENSE(1, 2, 2, 2);                  // 64 x 128, 4 waves of 32 x 64
#undef QL_DENSE
}

int launch_gemm(const GemmArgs& a, hipStream_t st) { return launch_gemm_dt<0>(a, st); }

bool gemm_ksplit_supported(int K) { return K % (2 * kGroup) == 0 && K >= 2 * kGroup; }

// Two-group tiles (gemm_tile with KG = 2): 64 x 128 while that gives at
// most 128 of them (the smallest class of qlinear_gemm's table), 128 x 128
// for every larger shape.  Both split K into the same two halves, so a
// row's bits do not depend on M within this entry point either.
int launch_gemm_ksplit(const GemmArgs& a, hipStream_t st) {
    KParams p{};
    p.A = a.X;
    p.M = a.M;
    p.qw = a.qweight;
    p.sc = a.scales;
    p.bi = a.biases;
    p.Y = a.Y;
    p.K = a.K;
    p.N = a.N;
    p.gscale = 1.f;
    const int64_t t128 = ((a.M + 127) / 128) * ((a.N + 127) / 128);
    auto go = [&](auto tl) -> int {
        using TL = decltype(tl);
        const int64_t gn = (a.N + TL::BN - 1) / TL::BN, gm = (a.M + TL::BM - 1) / TL::BM;
        if (gn * gm > 0x7fffff00LL) return QL_ERR_UNSUPPORTED_SHAPE;
        p.grid_n = (int)gn;
        p.grid_m = (int)gm;
        const dim3 grid((unsigned)((gn * gm + 7) / 8 * 8));
        if constexpr (TL::BM == 64) return launch_t<1, 2, 2, 2, MODE_DENSE, 0, 0, 2>(p, grid, st);
        else return launch_t<2, 2, 2, 2, MODE_DENSE, 0, 0, 2>(p, grid, st);
    };
    if (t128 <= 128) return go(Tile<1, 2, 2, 2>{});
    return go(Tile<2, 2, 2, 2>{});
}

int launch_gemm_bf16(const GemmArgs& a, hipStream_t st) { return launch_gemm_dt<1>(a, st); }

int launch_gemm_fp8(const GemmArgs& a, hipStream_t st) { return launch_gemm_dt<0, 1>(a, st); }

int launch_gemm_nvfp4(const GemmArgs& a, hipStream_t st) { return launch_gemm_dt<0, 2>(a, st); }

bool gemm_ws_supported(int K) { return K == 512 || K == 1024 || K == 2048; }

int launch_gemm_ws(const GemmArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.N + kWsCols - 1) / kWsCols));
    const dim3 block(64 * kWsWaves);
    switch (a.K / (kGroup * kWsWaves)) {
        case 1:
            hipLaunchKernelGGL((gemm_ws_kernel<1>), grid, block, 0, st, a.X, a.qweight, a.scales,
                               a.biases, a.Y, a.M, a.K, a.N);
            break;
        case 2:
            hipLaunchKernelGGL((gemm_ws_kernel<2>), grid, block, 0, st, a.X, a.qweight, a.scales,
                               a.biases, a.Y, a.M, a.K, a.N);
            break;
        case 4:
            hipLaunchKernelGGL((gemm_ws_kernel<4>), grid, block, 0, st, a.X, a.qweight, a.scales,
                               a.biases, a.Y, a.M, a.K, a.N);
            break;
        default:
            return QL_ERR_UNSUPPORTED_SHAPE;
    }
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

constexpr int kRouterSplit = kRouterMfmaSplit;

int launch_router_logits_mfma(const uint16_t* H, const uint16_t* Wr, float* partials, int T, int D,
                              int E, hipStream_t st, bool bf16) {
    KParams p{};
    p.A = H;
    p.M = T;
    p.Bh = Wr;
    p.Yf = partials;
    p.K = D;
    p.N = E;
    p.ksplit = kRouterSplit;
    using TL = Tile<1, 4, 2, 2>;
    dim3 grid((T + TL::BM - 1) / TL::BM, (E + TL::BN - 1) / TL::BN, kRouterSplit);
    if (bf16) return launch_t<1, 4, 2, 2, MODE_ROUTER, 1>(p, grid, st);
    return launch_t<1, 4, 2, 2, MODE_ROUTER>(p, grid, st);
}


template <int MODE, int DT, int WF = 0>
int launch_grouped_t(const KParams& p, dim3 grid, hipStream_t st) {
    static std::atomic<uint32_t> lds_set{0};
    if (const int rc = set_max_dynamic_lds((const void*)gemm_w4_grouped_kernel<MODE, DT, WF>, kGroupedLds,
                                           lds_set))
        return rc;
    hipLaunchKernelGGL((gemm_w4_grouped_kernel<MODE, DT, WF>), grid, dim3(TallTile::NT), kGroupedLds, st, p);
    return hipGetLastError() == hipSuccess ? QL_OK : QL_ERR_HIP;
}

int launch_moe_grouped(const GroupedArgs& a, hipStream_t st) {
    const MoeWorkspace L = moe_workspace_layout(a.T, a.E, a.topk);
    KParams p{};
    p.A = a.X;
    p.qw = a.qw;
    p.sc = a.sc;
    p.bi = a.bi;
    p.sqw = a.sqw;
    p.ssc = a.ssc;
    p.sbi = a.sbi;
    if (a.shared_only) {
        p.ws_header = nullptr;  // no routed tiles
        p.tiles = nullptr;
        p.max_tiles = 0;
    } else {
        p.ws_header = reinterpret_cast<const int*>(a.ws + L.header);
        p.tiles = reinterpret_cast<const int*>(a.ws + L.tiles);
        p.short_order = reinterpret_cast<const int*>(a.ws + L.short_order);
        p.max_tiles = L.max_tiles;
    }
    p.sorted_assign = a.sorted_assign;
    p.T = a.T;
    p.topk = a.topk;
    p.E = a.E;
    p.Y = a.Y;
    p.K = a.K;
    p.N = a.N;
    p.grid_n = (a.op == QL_OP_GATE_UP_SILU) ? (a.N / 2 + TallTile::BN / 2 - 1) / (TallTile::BN / 2)
                                            : (a.N + TallTile::BN - 1) / TallTile::BN;
    p.grid_m = a.sqw ? (a.T + TallTile::BM - 1) / TallTile::BM : 0;  // shared-expert tiles
    // Upper bounds of both classes; workgroups past the actual items exit.
    const int64_t max_tall = (a.shared_only ? 0 : ((int64_t)a.T * a.topk) / TallTile::BM) + p.grid_m;
    // Short class: up to ceil(max_tiles / 8) tiles of grid_n items per XCD.
    const int64_t items_b = max_tall * p.grid_n, items_s = ((int64_t)p.max_tiles + 7) / 8 * 8 * p.grid_n;
    const int64_t blocks = (items_b + 7) / 8 * 8 + items_s;
    if (blocks > 0x7fffff00LL) return QL_ERR_UNSUPPORTED_SHAPE;
    if (blocks == 0) return QL_OK;
    const dim3 grid((unsigned)blocks);
    if (a.wf == 1) {
        if (a.op == QL_OP_GATE_UP_SILU) return launch_grouped_t<MODE_GATEUP, 0, 1>(p, grid, st);
        return launch_grouped_t<MODE_DOWN, 0, 1>(p, grid, st);
    }
    if (a.wf == 2) {
        p.gscales = a.gscales;
        p.gscale = a.sgscale;
        if (a.op == QL_OP_GATE_UP_SILU) return launch_grouped_t<MODE_GATEUP, 0, 2>(p, grid, st);
        return launch_grouped_t<MODE_DOWN, 0, 2>(p, grid, st);
    }
    if (a.bf16) {
        if (a.op == QL_OP_GATE_UP_SILU) return launch_grouped_t<MODE_GATEUP, 1>(p, grid, st);
        return launch_grouped_t<MODE_DOWN, 1>(p, grid, st);
    }
    if (a.op == QL_OP_GATE_UP_SILU) return launch_grouped_t<MODE_GATEUP, 0>(p, grid, st);
    return launch_grouped_t<MODE_DOWN, 0>(p, grid, st);
}

}  // namespace ql
