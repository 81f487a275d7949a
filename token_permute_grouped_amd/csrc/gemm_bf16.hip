// Grouped expert GEMMs in bf16 on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// GEMM1 + SwiGLU (Megatron-LM "Support GEMM + Swiglu fused MLP"; the fused
// kernel of FlashInfer "[SM90] Add W4A8 MegaMoE support"):
//     h[r, c] = silu(g) * u,  g = x_perm[r] . W1_e[gate row of c],  u = x_perm[r] . W1_e[up row of c]
// GEMM2:  y_perm[r, :] = h[r] W2_e^T.
// Rows r of expert e are [offsets[e], offsets[e+1]): one ragged group per expert,
// with no padding of the groups (Megatron-LM's "skip routed expert padding").
//
// Tiling.  One workgroup of 8 waves (two per SIMD) owns a 256 x 256 output tile:
// kBM token rows of one expert x kBN weight rows; each wave computes 128 token rows
// x 64 weight rows as 4 x 2 blocks of 32 x 32 (8 independent MFMAs per 16-wide K
// step).  Two waves per SIMD let one issue MFMAs while the other waits on LDS or
// global memory; with one wave per SIMD (128 x 128 each) the same loop ran ~10%
// slower.  Both operands are K-contiguous in HBM; K advances kBK = 64 per stage.
//
// Pipeline.  LDS (160 KB) holds two activation stages of 32 KB and a ring of three
// 32 KB weight stages.  Activations go global -> registers -> LDS: while the MFMAs of
// stage k run, the wave writes stage k+1 from one of its two register sets into the
// free LDS buffer and refills that set with the loads of stage k+3.  Weights go
// straight to LDS by buffer-load DMA, requested two stages ahead.  The LDS writes of a
// stage (activation stores and weight DMAs) are split over two K steps: a burst of
// them stalls the MFMA issue.  Per stage there is one barrier, taken before the last
// 16-wide K step so that the next stage's first fragments load under that step's
// MFMAs and the MFMA issue does not drain.  Fragment reads of step s+1 are
// interleaved with the MFMAs of step s.  Sparse tiles (at most 64 live rows) use a
// second layout of the same LDS: 8 KB activation stages and a four-slot weight ring,
// the weights requested three stages ahead (their arithmetic is small, the weight
// stream is what they wait for).
//
// LDS layout.  A stage row is 64 bf16 = eight 16-byte chunks; chunk kc of row r sits
// at slot kc ^ ((r & 7) ^ ((r >> 3) & 1)).  A fragment read (32 rows, one chunk)
// then hits distinct banks within every 8 rows (32-bank view) and every 16 rows
// (64-bank view), and a thread's writes (rows r, r+32, ...) share one slot.
//
// Operand order.  The weight fragment is the MFMA's first operand, so a lane's 16
// accumulators of a block are 4 runs of 4 consecutive output columns of one token
// row (8-byte bf16 writes into the epilogue's LDS staging of the output tile).
//
// SwiGLU fusion.  For GEMM1 an n-tile holds the weight rows of 128 output columns
// c0..c0+127 ordered [gate 32 | up 32] x 4 (one pair per wave column), so gate and
// up of a column are in the same lane of two blocks and silu(g) * u is formed in
// registers.  With the
// interleave-32 layout these 256 rows are one contiguous slice of W1; with
// [gate | up] they are two 128-row slices I rows apart.
//
// Ragged tails.  Raw buffer resources bound every load: activation rows past the
// tile's live rows, and weight rows past N (GEMM2 with H % 256 == 128), read as
// zero.  A wave skips the MFMAs of 32-row blocks that hold no live row (the K loop
// is instantiated per live-block count, so it stays branch-free) and only live
// rows are stored.
//
// Fused gather.  GEMM1 can read its activation rows straight from the token rows x
// [T][K] through the row_src table (row r of the expert-major order is token
// row_src[r] / k), so the forward needs no separate permuted copy of x: the permute
// of Megatron-LM "add permute fusion into hybrid ep" then happens in the tile loads,
// the way the FlashInfer split kernels fold dispatch into their first GEMM.  Each
// 128-byte piece of a row is still one whole cache line, so the loads stay coalesced.
//
// Scheduling.  The device-side tile list gives the m-tiles (expert, first row);
// tile_map assigns them to workgroups by band and XCD rectangle (below).
// Workgroups past the tile count exit before any barrier.
#include <type_traits>

#include "moe_internal.h"

namespace tpg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = kGemmBM;  // token rows per tile (256)
constexpr int kBN = 256;      // weight rows per tile
constexpr int kBK = 64;       // K per stage
constexpr int kWaves = 8;     // two per SIMD
constexpr int kThreads = 64 * kWaves;
constexpr int kWaveN = 4;     // waves along the weight rows; each wave owns 128 token x 64 weight rows
constexpr int kRowBytes = kBK * 2;                    // 128: one row of one stage
constexpr int kAStage = kBM * kRowBytes;               // 32 KB: activation rows of one stage
constexpr int kBStage = kBN * kRowBytes;               // 32 KB: weight rows of one stage
constexpr int kBStages = 3;                            // weight ring depth (DMA two stages ahead)
constexpr int kBBase = 2 * kAStage;                    // weights follow the two activation stages
constexpr int kLoads = kBM * kRowBytes / 16 / kThreads;  // 16-byte activation loads per thread (4)
constexpr int kOpsB = kBStage / 1024 / kWaves;         // 1 KB weight DMAs per wave per stage (4)
constexpr int kLRows = kThreads / 8;                   // tile rows one activation load covers (64)
// Sparse tiles (at most 64 live rows): activation stages of 64 rows (8 KB, one load per thread)
// leave room for a fourth weight slot, so the weights are requested three stages ahead.
constexpr int kSpRows = 64;
constexpr int kAStageSp = kSpRows * kRowBytes;        // 8 KB
constexpr int kBBaseSp = 2 * kAStageSp;               // 16 KB
constexpr int kBStagesSp = 4;
static_assert(kBBaseSp + kBStagesSp * kBStage <= kBBase + kBStages * kBStage, "sparse layout fits the LDS");
static_assert(kSpRows == kLRows, "a sparse stage is the first activation load of every thread");

// Workgroup -> tile map.  Workgroup b runs on XCD b % 8.  Bands of tm.gm m-tiles take
// tm.per_band workgroups each; a band is cut into 8 rectangles (xm rows of m-tiles x xn
// columns of n-tiles, about 32 tiles each: one per CU of an XCD), and XCD x takes
// rectangle x.  The 32 tiles an XCD runs at once then share ~8 activation slabs and ~4
// weight slabs in its L2, and all XCDs stay on one band (a few experts) in the MALL.
struct TileMap {
    int xn, nc, gm, per_band;  // rectangle columns, n-tiles per column, band m-tiles, workgroups per band
};
__host__ __device__ inline TileMap tile_map(int nb_n) {
    const int xn = nb_n >= 4 ? 4 : nb_n >= 2 ? 2 : 1;
    const int nc = (nb_n + xn - 1) / xn;
    const int rm = 32 / nc > 1 ? 32 / nc : 1;  // m-tiles per rectangle
    return {xn, nc, (8 / xn) * rm, 8 * rm * nc};
}

__device__ __forceinline__ int slot(int r, int kc) { return kc ^ ((r & 7) ^ ((r >> 3) & 1)); }

__device__ __forceinline__ float silu_mul(float g, float u, float clamp) {
    if (clamp > 0.f) {
        g = fminf(fmaxf(g, -clamp), clamp);
        u = fminf(fmaxf(u, -clamp), clamp);
    }
    // hardware exp2 / reciprocal (about 1 ulp each): far below the bf16 rounding of h
    return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)) * u;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return pack_bf16x2(a, b);
}

// one 16-byte-per-lane DMA from a raw buffer straight into LDS (1 KB per wave, lane-linear)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, void *dst) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)dst, 16, voff, soff, 0, 0);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// LDS barrier without a global-memory fence: register loads stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// scheduling pattern: NR fragment reads (DS) spread evenly over M MFMAs
template <int NR, int M, int I = 0>
__device__ __forceinline__ void interleave_ds_mfma() {
    if constexpr (I < NR) {
        constexpr int m = (M * (I + 1)) / NR - (M * I) / NR;
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);                       // DS read
        if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);  // MFMA
        interleave_ds_mfma<NR, M, I + 1>();
    }
}

// pattern with extra work: per group, X instructions of class `cls`, one DS read, MFMAs
template <int cls, int X, int NR, int M, int I = 0>
__device__ __forceinline__ void interleave_x_ds_mfma() {
    if constexpr (I < NR) {
        constexpr int m = (M * (I + 1)) / NR - (M * I) / NR;
        constexpr int x = (X * (I + 1)) / NR - (X * I) / NR;
        if constexpr (x > 0) __builtin_amdgcn_sched_group_barrier(cls, x, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if constexpr (m > 0) __builtin_amdgcn_sched_group_barrier(0x008, m, 0);
        interleave_x_ds_mfma<cls, X, NR, M, I + 1>();
    }
}

}  // namespace

template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads, 1) void grouped_gemm_bf16_kernel(
    const uint16_t *__restrict__ A,        // [S][K] activations in expert-contiguous row order, or
                                           // with row_src: the token rows [a_rows][K]
    const int32_t *__restrict__ row_src,   // NULL, or [S]: row r reads token row row_src[r] / gather_k
    int gather_k, int a_rows,
    const uint16_t *__restrict__ W,        // [E][N][K] expert weights
    const int32_t *__restrict__ offsets,   // [E+1]
    const int32_t *__restrict__ tiles,     // [2 * n_tiles]: expert, first row within the expert
    const int32_t *__restrict__ n_tiles,   // [1]
    int K, int N, int I, int il, float clamp,
    uint16_t *__restrict__ C, int ldc,     // [S][ldc]
    const int32_t *__restrict__ row_dst) { // NULL, or [S]: row r of the tile order is stored to row row_dst[r] of C
    __shared__ __attribute__((aligned(1024))) unsigned char lds[kBBase + kBStages * kBStage];  // 160 KB

    // ---- tile of this workgroup: band of m-tiles, XCD rectangle within the band, tile within it
    const int nb_n = (N + kBN - 1) / kBN;
    const TileMap tm = tile_map(nb_n);
    const int n_mt = n_tiles[0];
    const int band = blockIdx.x / tm.per_band, p = blockIdx.x % tm.per_band;
    const int first_m = band * tm.gm;
    const int gm = min(tm.gm, n_mt - first_m);  // m-tiles in this band
    const int xm = 8 / tm.xn;
    const int ma = (gm + xm - 1) / xm;          // m-tiles per rectangle row
    const int x = p & 7, q = p >> 3;            // XCD (blockIdx % 8) and position on it
    const int mi = q / tm.nc, ni = q % tm.nc;
    const int v = first_m + (x / tm.xn) * ma + mi;  // position in the interleaved m-tile order
    const int nt = (x % tm.xn) * tm.nc + ni;
    if (gm <= 0 || mi >= ma || v >= first_m + gm || nt >= nb_n) return;
    // The list holds the full m-tiles, then one partial m-tile per expert.  A partial tile
    // does little MFMA work for the weights it streams, so partial tiles are spread evenly
    // through the order (position v is partial when floor(v P / n) steps) and their weight
    // streaming overlaps the full tiles' MFMAs instead of forming a memory-bound tail.
    const int n_part = n_mt - n_tiles[1];
    const int cp = (int)((int64_t)v * n_part / n_mt), cp1 = (int)((int64_t)(v + 1) * n_part / n_mt);
    const int mt = cp1 > cp ? n_tiles[1] + cp : v - cp;

    const int e = tiles[2 * mt];
    const int row_begin = offsets[e] + tiles[2 * mt + 1];
    const int rows = min(kBM, offsets[e + 1] - row_begin);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / kWaveN, wn = wave % kWaveN;

    // ---- activations: global -> registers -> LDS.  Thread loads chunk (tid & 7) of tile rows
    //      (tid >> 3) + 32 i.  Weights: DMA straight into LDS, wave w filling rows w*64 .. w*64+63,
    //      8 rows per 1 KB op (row lane/8, slot lane%8).  Raw buffer resources bound every read:
    //      rows past the tile's live rows, and weight rows past N, read as zero.
    const int lrow = tid >> 3, lkc = tid & 7;
    const bool gather = row_src != nullptr;
    // source rows of this thread's activation loads (fused gather): issued first, used after
    // the first weight DMA so that their latency overlaps it
    // (no lane-dependent branch or select touches these before their use, which keeps the
    // compiler from waiting for them early and the buffer descriptors in scalar registers)
    int src[kLoads] = {};
    if (gather) {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) src[i] = row_src[row_begin + min(lrow + kLRows * i, rows - 1)];
    }
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(A + (gather ? 0 : (int64_t)row_begin * K)), (short)0, gather ? a_rows * K * 2 : rows * K * 2,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsB = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(W + (int64_t)e * N * K), (short)0, N * K * 2, 0x00020000);
    uint32_t offA[kLoads], offB[kOpsB];
    // Byte offsets of the activation loads.  Rows past the tile's live rows get an offset
    // beyond the buffer (a_rows * K * 2 < 2^31, checked by the host), so they read zero.
    // Token of slot s = t*k + j: s / k in double precision, exact for integers below 2^31 (the
    // fractional part of a non-integer quotient is at least 1/k, far above the rounding error).
    auto init_offA = [&]() {
#pragma unroll
        for (int i = 0; i < kLoads; ++i) {
            const int r = lrow + kLRows * i;
            asm volatile("" : "+v"(src[i])::"memory");  // consumed here, after the first weight DMA
            const int t = (int)((double)src[i] / (double)gather_k);
            offA[i] = !gather ? (uint32_t)(r * K + lkc * 8) * 2u
                      : r >= rows ? 0x80000000u  // a row past the tile: read as zero
                                  : (uint32_t)(t * K + lkc * 8) * 2u;
        }
    };
#pragma unroll
    for (int i = 0; i < kOpsB; ++i) {
        const int r = wave * (kBN / kWaves) + i * 8 + (lane >> 3);  // tile weight row
        int wr;
        if (kSwiGLU) {
            // tile row r: wave column r >> 6, gate/up block (r >> 5) & 1 -> [g | u]
            const int c = nt * (kBN / 2) + (r >> 6) * 32 + (r & 31);
            const bool up = (r >> 5) & 1;
            wr = il == 0 ? (up ? I + c : c) : (c / il) * 2 * il + (up ? il : 0) + c % il;
        } else {
            wr = nt * kBN + r;  // rows >= N read as zero
        }
        const int kc = slot(r, lane & 7);  // the logical chunk LDS slot (lane & 7) holds
        offB[i] = (uint32_t)(wr * K + kc * 8) * 2u;
    }
    // LDS byte offset of this thread's activation writes (same slot for rows lrow + 64 i)
    const int wofs = lrow * kRowBytes + slot(lrow, lkc) * 16;

    u32x4 RA0[kLoads], RA1[kLoads];
    // NL: activation loads per thread (kLoads, or 1 for sparse tiles); AS / BB: LDS bytes of an
    // activation stage / offset of the weight ring
    auto gloadA = [&](u32x4 *R, int kt, auto nl_tag) {
        constexpr int NL = decltype(nl_tag)::value;
#pragma unroll
        for (int i = 0; i < NL; ++i) R[i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, offA[i], kt * kRowBytes, 0);
    };
    auto lwriteA = [&](const u32x4 *R, int astage, int i0, int n, int AS) {
        unsigned char *base = lds + astage * AS + wofs;
#pragma unroll
        for (int i = i0; i < i0 + n; ++i) *(u32x4 *)(base + i * kLRows * kRowBytes) = R[i];
    };
    auto dmaB = [&](int kt, int bstage, int i0, int n, int BB) {
        unsigned char *dst = lds + BB + bstage * kBStage + wave * (kBN / kWaves) * kRowBytes;
#pragma unroll
        for (int i = i0; i < i0 + n; ++i) dma16(rsB, offB[i], kt * kRowBytes, dst + i * 1024);
    };

    f32x16 acc[2][4];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // 32-row token blocks of this wave that hold a live row
    const int nb_live = max(0, min(4, (rows - wm * 128 + 31) >> 5));
    const int fr = lane & 31, fk = lane >> 5;
    const int nk = K / kBK;  // even: K is a multiple of 128

    auto mainloop = [&](auto nb_tag, auto sp_tag) {
        constexpr int NB = decltype(nb_tag)::value;
        constexpr bool kSp = decltype(sp_tag)::value;  // sparse tile: at most 64 live rows
        constexpr int NR = 2 + NB;  // fragment reads per K step
        constexpr int NM = 2 * NB;  // MFMAs per K step
        constexpr int NL = kSp ? 1 : kLoads;            // activation loads per thread and stage
        constexpr int AS = kSp ? kAStageSp : kAStage;
        constexpr int BB = kSp ? kBBaseSp : kBBase;
        constexpr int NBS = kSp ? kBStagesSp : kBStages;
        constexpr int LA = kSp ? 3 : 2;                 // weight DMA lookahead in stages
        using NLt = std::integral_constant<int, NL>;
        bf16x8 fw[2][2], fx[2][NB > 0 ? NB : 1];
        auto load = [&](int buf, int astage, int bstage, int ks) {
            if constexpr (NB > 0) {
                const u32x4 *sa = (const u32x4 *)(lds + astage * AS);
                const u32x4 *sb = (const u32x4 *)(lds + BB + bstage * kBStage);
                const int kc = ks * 2 + fk;
#pragma unroll
                for (int a = 0; a < 2; ++a) {
                    const int r = wn * 64 + a * 32 + fr;
                    fw[buf][a] = __builtin_bit_cast(bf16x8, sb[r * 8 + slot(r, kc)]);
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int r = wm * 128 + b * 32 + fr;
                    fx[buf][b] = __builtin_bit_cast(bf16x8, sa[r * 8 + slot(r, kc)]);
                }
            }
        };
        auto mfmas = [&](int buf) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
#pragma unroll
                for (int a = 0; a < 2; ++a)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[buf][a], fx[buf][b], acc[a][b], 0, 0, 0);
        };

        // One stage kt: activations in LDS buffer kt & 1 (P), weights in ring slot bs = kt % NBS;
        // its step-0 fragments are already in fw/fx[0].  Issue order per stage (all VMEM, in
        // order): weight DMA of kt+LA at the top, activation loads of kt+3 at step 2.  The weights
        // of kt+1 (DMA issued LA-1 stages earlier) must have landed before the barrier; the VMEM
        // ops issued after them may still be in flight: dense tiles (LA 2) activations kt+2,
        // weights kt+2, activations kt+3; sparse tiles (LA 3) activations kt+1, weights and
        // activations kt+2, weights and activations kt+3, each where that stage exists.
        // kIssue: stages kt+2 (weights) and kt+3 (activations) exist; kNext: stage kt+1 exists.
        auto step = [&](auto p_tag, auto next_tag, auto issue_tag, int kt, int bs) {
            constexpr int P = decltype(p_tag)::value;
            constexpr bool kNext = decltype(next_tag)::value;
            constexpr bool kIssue = decltype(issue_tag)::value;
            u32x4 *Rn = P == 0 ? RA1 : RA0;  // holds the activations of stage kt+1
            const int bs1 = bs + 1 == NBS ? 0 : bs + 1;
            const int bsl = (bs + LA) % NBS;  // slot of the stage the DMA requests
            const bool issue_w = kIssue && (!kSp || kt + 3 < nk);
            if (issue_w) {
                dmaB(kt + LA, bsl, 0, kOpsB / 2, BB);
                __builtin_amdgcn_sched_group_barrier(0x020, kOpsB / 2, 0);
            }
            // K steps 0 and 1: fragments of the next step under the MFMAs, and the activations
            // of stage kt+1 into the free LDS buffer, half under each step (sparse: one write)
            if constexpr (kNext) lwriteA(Rn, P ^ 1, 0, kSp ? 1 : kLoads / 2, AS);
            load(1, P, bs, 1);
            mfmas(0);
            if constexpr (NB > 0) {
                if constexpr (kNext) interleave_x_ds_mfma<0x200, kSp ? 1 : kLoads / 2, NR, NM>();
                else interleave_ds_mfma<NR, NM>();
            }
            if (issue_w) {
                dmaB(kt + LA, bsl, kOpsB / 2, kOpsB / 2, BB);
                __builtin_amdgcn_sched_group_barrier(0x020, kOpsB / 2, 0);
            }
            if constexpr (kNext && !kSp) lwriteA(Rn, P ^ 1, kLoads / 2, kLoads / 2, AS);
            load(0, P, bs, 2);
            mfmas(1);
            if constexpr (NB > 0) {
                if constexpr (kNext && !kSp) interleave_x_ds_mfma<0x200, kLoads / 2, NR, NM>();
                else interleave_ds_mfma<NR, NM>();
            }
            // K step 2: refill the register set with the activations of stage kt+3
            if constexpr (kIssue) {
                if (kt + 3 < nk) gloadA(Rn, kt + 3, NLt{});
            }
            load(1, P, bs, 3);
            mfmas(0);
            if constexpr (NB > 0) interleave_ds_mfma<NR, NM>();
            // K step 3: publish stage kt+1 and load its first fragments under the last MFMAs
            if constexpr (kNext) {
                if constexpr (kSp) {
                    constexpr int G = kOpsB + 1;  // weights + activations of one stage
                    if (kt + 3 < nk) wait_vmcnt<1 + 2 * G>();
                    else if (kt + 2 < nk) wait_vmcnt<1 + G>();
                    else wait_vmcnt<1>();
                } else if constexpr (kIssue) {
                    if (kt + 3 < nk) wait_vmcnt<2 * kLoads + kOpsB>();  // activations kt+2, kt+3; weights kt+2
                    else wait_vmcnt<kLoads + kOpsB>();                 // no activations kt+3 were issued
                } else {
                    wait_vmcnt<0>();
                }
                lds_barrier();
                load(0, P ^ 1, bs1, 0);
            }
            mfmas(1);
            if constexpr (NB > 0 && kNext) interleave_ds_mfma<NR, NM>();
        };
        using T0 = std::integral_constant<int, 0>;
        using T1 = std::integral_constant<int, 1>;
        using Y = std::true_type;
        using F = std::false_type;

        // prologue: stage 0 (weights, activations), then stage 1 (sparse: and the weights of
        // stage 2), in issue order; activations of 0 written, activations of 2 in flight.  The
        // barrier waits for stage 0 only: the later stages land like every later stage.
        dmaB(0, 0, 0, kOpsB, BB);
        asm volatile("" ::: "memory");  // keep the issue order: loads complete in it
        init_offA();
        gloadA(RA0, 0, NLt{});
        asm volatile("" ::: "memory");
        dmaB(1, 1, 0, kOpsB, BB);
        asm volatile("" ::: "memory");
        gloadA(RA1, 1, NLt{});
        asm volatile("" ::: "memory");
        if constexpr (kSp) {
            if (nk > 2) dmaB(2, 2, 0, kOpsB, BB);
            asm volatile("" ::: "memory");
        }
        lwriteA(RA0, 0, 0, NL, AS);
        if (nk > 2) {
            gloadA(RA0, 2, NLt{});
            // dense: weights 1, activations 1 and 2 may be in flight; sparse: also weights 2
            wait_vmcnt<(kSp ? 2 : 1) * kOpsB + 2 * NL>();
        } else {
            wait_vmcnt<kOpsB + NL>();
        }
        lds_barrier();
        load(0, 0, 0, 0);
        int bs = 0;
        int kt = 0;
        for (; kt + 2 < nk; kt += 2) {  // both stages of the pair issue (weights kt+2, kt+3 exist)
            step(T0{}, Y{}, Y{}, kt, bs);
            bs = bs + 1 == NBS ? 0 : bs + 1;
            step(T1{}, Y{}, Y{}, kt + 1, bs);
            bs = bs + 1 == NBS ? 0 : bs + 1;
        }
        // last pair: stage nk-2 has a next stage but nothing to issue; nk-1 is the last
        step(T0{}, Y{}, F{}, nk - 2, bs);
        bs = bs + 1 == NBS ? 0 : bs + 1;
        step(T1{}, F{}, F{}, nk - 1, bs);
    };
    using Dense = std::false_type;
    using Sparse = std::true_type;
    if (rows <= kSpRows) {  // wm = 0 waves hold at most two live 32-row blocks, wm = 1 none
        switch (nb_live) {
            case 2: mainloop(std::integral_constant<int, 2>{}, Sparse{}); break;
            case 1: mainloop(std::integral_constant<int, 1>{}, Sparse{}); break;
            default: mainloop(std::integral_constant<int, 0>{}, Sparse{}); break;
        }
    } else {
        switch (nb_live) {
            case 4: mainloop(std::integral_constant<int, 4>{}, Dense{}); break;
            case 3: mainloop(std::integral_constant<int, 3>{}, Dense{}); break;
            case 2: mainloop(std::integral_constant<int, 2>{}, Dense{}); break;
            case 1: mainloop(std::integral_constant<int, 1>{}, Dense{}); break;
            default: mainloop(std::integral_constant<int, 0>{}, Dense{}); break;
        }
    }

    // ---- epilogue: lane holds token row (lane & 31) of block b and weight rows
    //      m = 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3) of block a.  The bf16 tile goes through
    //      LDS (16-byte chunk c of row r at chunk c ^ (r & 15)), so that every global store
    //      writes whole rows of the tile: direct 8-byte stores from the MFMA layout touch 32
    //      rows per instruction and took ~15% of a GEMM2 tile.
    constexpr int kCols = kSwiGLU ? kBN / 2 : kBN;  // output columns of the tile
    constexpr int kChunks = kCols / 8;              // 16-byte chunks per row: 16 or 32
    auto cofs = [](int r, int c) { return r * (kCols * 2) + ((c ^ (r & 15)) << 4); };
    const int half = lane >> 5;
    lds_barrier();  // every wave is done with the last stage's operands
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const int tr = wm * 128 + b * 32 + (lane & 31);
        if (kSwiGLU) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                float hv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) hv[q] = silu_mul(acc[0][b][g4 * 4 + q], acc[1][b][g4 * 4 + q], clamp);
                u32x2 o;
                o.x = pack2(hv[0], hv[1]);
                o.y = pack2(hv[2], hv[3]);
                *(u32x2 *)(lds + cofs(tr, wn * 4 + g4) + half * 8) = o;  // columns wn*32 + g4*8 + half*4 ..
            }
        } else {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    u32x2 o;
                    o.x = pack2(acc[a][b][g4 * 4 + 0], acc[a][b][g4 * 4 + 1]);
                    o.y = pack2(acc[a][b][g4 * 4 + 2], acc[a][b][g4 * 4 + 3]);
                    *(u32x2 *)(lds + cofs(tr, wn * 8 + a * 4 + g4) + half * 8) = o;  // columns wn*64 + a*32 + ..
                }
        }
    }
    lds_barrier();
    constexpr int kRowsPerOp = 64 / kChunks;  // tile rows one store instruction covers: 4 or 2
    const int sc = lane % kChunks, sr = lane / kChunks;
    const int c0 = nt * kCols + sc * 8;
    if (kSwiGLU || c0 < N) {
#pragma unroll 4
        for (int r0 = wave * kRowsPerOp; r0 < kBM; r0 += kWaves * kRowsPerOp) {
            const int tr = r0 + sr;
            if (tr < rows)
                *(u32x4 *)(C + (int64_t)(row_dst ? row_dst[row_begin + tr] : row_begin + tr) * ldc + c0) =
                    *(const u32x4 *)(lds + cofs(tr, sc));
        }
    }
}

namespace {
template <bool kSwiGLU>
hipError_t launch(const uint16_t *A, const int32_t *row_src, int gather_k, int a_rows, const uint16_t *W,
                  const int32_t *offsets, const int32_t *tiles, const int32_t *n_tiles, int64_t max_tiles, int K,
                  int N, int I, int il, float clamp, uint16_t *C, int ldc, const int32_t *row_dst, hipStream_t s) {
    const int nb_n = (N + kBN - 1) / kBN;
    const TileMap tm = tile_map(nb_n);
    const int64_t blocks = (max_tiles + tm.gm - 1) / tm.gm * tm.per_band;
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<kSwiGLU>, dim3(blocks), dim3(kThreads), 0, s, A, row_src, gather_k,
                       a_rows, W, offsets, tiles, n_tiles, K, N, I, il, clamp, C, ldc, row_dst);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_gemm1_swiglu_bf16(const uint16_t *x_perm, const uint16_t *w1, const int32_t *offsets,
                                    const int32_t *tiles, const int32_t *n_tiles, int64_t max_tiles, int H, int I,
                                    int glu_interleave, float clamp, uint16_t *h, hipStream_t s) {
    return launch<true>(x_perm, nullptr, 1, 0, w1, offsets, tiles, n_tiles, max_tiles, H, 2 * I, I, glu_interleave,
                        clamp, h, I, nullptr, s);
}

hipError_t launch_gemm1_swiglu_gather_bf16(const uint16_t *x, const int32_t *row_src, int T, int k,
                                           const uint16_t *w1, const int32_t *offsets, const int32_t *tiles,
                                           const int32_t *n_tiles, int64_t max_tiles, int H, int I,
                                           int glu_interleave, float clamp, uint16_t *h, hipStream_t s) {
    if (!gather_fits(T, H)) return hipErrorInvalidValue;
    return launch<true>(x, row_src, k, T, w1, offsets, tiles, n_tiles, max_tiles, H, 2 * I, I, glu_interleave, clamp,
                        h, I, nullptr, s);
}

hipError_t launch_gemm2_bf16(const uint16_t *h, const uint16_t *w2, const int32_t *offsets, const int32_t *tiles,
                             const int32_t *n_tiles, int64_t max_tiles, int H, int I, uint16_t *y_perm,
                             const int32_t *row_dst, hipStream_t s) {
    return launch<false>(h, nullptr, 1, 0, w2, offsets, tiles, n_tiles, max_tiles, I, H, I, 0, 0.0f, y_perm, H, row_dst,
                         s);
}

}  // namespace tpg
