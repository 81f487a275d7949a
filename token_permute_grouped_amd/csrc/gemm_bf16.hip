// Grouped expert GEMMs in bf16 on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16).
//
// GEMM1 + SwiGLU (Megatron-LM "Support GEMM + Swiglu fused MLP"; the fused
// kernel of FlashInfer "[SM90] Add W4A8 MegaMoE support"):
//     h[r, c] = silu(g) * u,  g = x_perm[r] . W1_e[gate row of c],  u = x_perm[r] . W1_e[up row of c]
// GEMM2:  y_perm[r, :] = h[r] W2_e^T.
// Rows r of expert e are [offsets[e], offsets[e+1]): one ragged group per expert,
// with no padding of the groups (Megatron-LM's "skip routed expert padding").
//
// Tiling.  A workgroup (4 waves) owns one (m-tile, n-tile) pair of one expert:
// kBM token rows x kBN weight rows, K stepped by kBK = 64.  Both operands are
// K-contiguous in HBM, so each 64-wide K slab of a row is eight 16-byte chunks; a
// slab is staged global -> registers -> LDS (double buffered, one barrier per K
// step) with chunk kc of row r stored at position kc ^ (r & 7), which makes the
// 16-byte fragment reads of the MFMA loop conflict-free.  Each wave computes a
// 64 x 64 sub-tile as 2 x 2 blocks of 32 x 32, issuing the weight fragment as the
// MFMA's first operand so that a lane's 16 accumulators are 4 runs of 4
// consecutive output columns of one token row (8-byte bf16 stores).
//
// SwiGLU fusion.  For GEMM1 the n-tile holds weight rows for 64 output columns
// c0..c0+63 ordered [gate 32 | up 32 | gate 32 | up 32], so a wave's two 32-row
// blocks are the gate and up values of the same 32 columns, in the same lanes,
// and silu(g) * u is formed in registers.  With the interleave-32 layout these
// 128 rows are one contiguous slice of W1; with [gate | up] they are two 64-row
// slices I rows apart.
//
// Ragged tails.  A tile with fewer than kBM live rows loads its last live row in
// place of the missing ones (no out-of-range read) and stores only live rows.
// Workgroups past the device-side tile count exit before any barrier.
#include "moe_internal.h"

namespace tpg {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = kGemmBM;  // token rows per tile
constexpr int kBN = 128;      // weight rows per tile
constexpr int kBK = 64;       // K per LDS stage
constexpr int kThreads = 256;
constexpr int kChunksA = kBM * kBK / 8;  // 16-byte chunks per A stage
constexpr int kChunksB = kBN * kBK / 8;
constexpr int kLoadsA = kChunksA / kThreads;
constexpr int kLoadsB = kChunksB / kThreads;

__device__ __forceinline__ int swz(int row, int kc) { return row * 8 + (kc ^ (row & 7)); }

__device__ __forceinline__ float silu_mul(float g, float u, float clamp) {
    if (clamp > 0.f) {
        g = fminf(fmaxf(g, -clamp), clamp);
        u = fminf(fmaxf(u, -clamp), clamp);
    }
    return g / (1.0f + expf(-g)) * u;
}

__device__ __forceinline__ uint32_t pack2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// stored W1 row of gate (up=false) or up (up=true) column c
__device__ __forceinline__ int64_t w1_row(int c, bool up, int I, int il) {
    if (il == 0) return up ? (int64_t)I + c : c;
    return (int64_t)(c / il) * 2 * il + (up ? il : 0) + c % il;
}

}  // namespace

template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_bf16_kernel(
    const uint16_t *__restrict__ A,        // [S][K] activations in expert-contiguous row order
    const uint16_t *__restrict__ W,        // [E][N][K] expert weights
    const int32_t *__restrict__ offsets,   // [E+1]
    const int32_t *__restrict__ tiles,     // [2 * n_tiles]: expert, first row within the expert
    const int32_t *__restrict__ n_tiles,   // [1]
    int K, int N, int I, int il, float clamp,
    uint16_t *__restrict__ C, int ldc) {   // [S][ldc]
    __shared__ u32x4 lds_a[2][kChunksA];
    __shared__ u32x4 lds_b[2][kChunksB];

    const int nb_n = N / kBN;
    const int mt = blockIdx.x / nb_n;
    const int nt = blockIdx.x % nb_n;
    if (mt >= n_tiles[0]) return;
    const int e = tiles[2 * mt];
    const int row_begin = offsets[e] + tiles[2 * mt + 1];
    const int rows = min(kBM, offsets[e + 1] - row_begin);

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;

    // per-thread source rows of its 16-byte chunks (fixed over K)
    const u32x4 *src_a[kLoadsA];
    const u32x4 *src_b[kLoadsB];
    int dst_a[kLoadsA], dst_b[kLoadsB];
    const uint16_t *We = W + (int64_t)e * N * K;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) {
        const int q = tid + i * kThreads, r = q >> 3, kc = q & 7;
        const int rr = min(r, rows - 1);
        src_a[i] = (const u32x4 *)(A + (int64_t)(row_begin + rr) * K) + kc;
        dst_a[i] = swz(r, kc);
    }
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) {
        const int q = tid + i * kThreads, r = q >> 3, kc = q & 7;
        int64_t wr;
        if (kSwiGLU) {
            const int g = r >> 6, qq = r & 63;
            const int c = nt * (kBN / 2) + g * 32 + (qq & 31);
            wr = w1_row(c, qq >= 32, I, il);
        } else {
            wr = (int64_t)nt * kBN + r;
        }
        src_b[i] = (const u32x4 *)(We + wr * K) + kc;
        dst_b[i] = swz(r, kc);
    }

    f32x16 acc[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    u32x4 ra[kLoadsA], rb[kLoadsB];
    const int nk = K / kBK;
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) ra[i] = src_a[i][0];
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) rb[i] = src_b[i][0];
#pragma unroll
    for (int i = 0; i < kLoadsA; ++i) lds_a[0][dst_a[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < kLoadsB; ++i) lds_b[0][dst_b[i]] = rb[i];
    __syncthreads();

    const int frag_row = lane & 31, frag_kc = lane >> 5;
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) {
            const int off = (kt + 1) * (kBK / 8);  // in 16-byte chunks
#pragma unroll
            for (int i = 0; i < kLoadsA; ++i) ra[i] = src_a[i][off];
#pragma unroll
            for (int i = 0; i < kLoadsB; ++i) rb[i] = src_b[i][off];
        }
#pragma unroll
        for (int ks = 0; ks < kBK / 16; ++ks) {
            bf16x8 fw[2], fx[2];
#pragma unroll
            for (int a = 0; a < 2; ++a)
                fw[a] = __builtin_bit_cast(bf16x8, lds_b[cur][swz(wn * 64 + a * 32 + frag_row, ks * 2 + frag_kc)]);
#pragma unroll
            for (int b = 0; b < 2; ++b)
                fx[b] = __builtin_bit_cast(bf16x8, lds_a[cur][swz(wm * 64 + b * 32 + frag_row, ks * 2 + frag_kc)]);
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int b = 0; b < 2; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[a], fx[b], acc[a][b], 0, 0, 0);
        }
        if (kt + 1 < nk) {
#pragma unroll
            for (int i = 0; i < kLoadsA; ++i) lds_a[cur ^ 1][dst_a[i]] = ra[i];
#pragma unroll
            for (int i = 0; i < kLoadsB; ++i) lds_b[cur ^ 1][dst_b[i]] = rb[i];
        }
        __syncthreads();
    }

    // epilogue: lane holds token row (lane & 31) of block b, weight rows m = 8*(v>>2) + 4*(lane>>5) + (v&3)
    const int half = lane >> 5;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int tr = wm * 64 + b * 32 + (lane & 31);
        if (tr >= rows) continue;
        uint16_t *crow = C + (int64_t)(row_begin + tr) * ldc;
        if (kSwiGLU) {
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int c0 = nt * (kBN / 2) + wn * 32 + g4 * 8 + half * 4;
                float hv[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) hv[j] = silu_mul(acc[0][b][g4 * 4 + j], acc[1][b][g4 * 4 + j], clamp);
                u32x2 o;
                o.x = pack2(hv[0], hv[1]);
                o.y = pack2(hv[2], hv[3]);
                *(u32x2 *)(crow + c0) = o;
            }
        } else {
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c0 = nt * kBN + wn * 64 + a * 32 + g4 * 8 + half * 4;
                    u32x2 o;
                    o.x = pack2(acc[a][b][g4 * 4 + 0], acc[a][b][g4 * 4 + 1]);
                    o.y = pack2(acc[a][b][g4 * 4 + 2], acc[a][b][g4 * 4 + 3]);
                    *(u32x2 *)(crow + c0) = o;
                }
        }
    }
}

hipError_t launch_gemm1_swiglu_bf16(const uint16_t *x_perm, const uint16_t *w1, const int32_t *offsets,
                                    const int32_t *tiles, const int32_t *n_tiles, int64_t max_tiles, int H, int I,
                                    int glu_interleave, float clamp, uint16_t *h, hipStream_t s) {
    const int N = 2 * I;
    const int64_t blocks = max_tiles * (N / kBN);
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<true>, dim3(blocks), dim3(kThreads), 0, s, x_perm, w1, offsets,
                       tiles, n_tiles, H, N, I, glu_interleave, clamp, h, I);
    return hipGetLastError();
}

hipError_t launch_gemm2_bf16(const uint16_t *h, const uint16_t *w2, const int32_t *offsets, const int32_t *tiles,
                             const int32_t *n_tiles, int64_t max_tiles, int H, int I, uint16_t *y_perm,
                             hipStream_t s) {
    const int64_t blocks = max_tiles * (H / kBN);
    hipLaunchKernelGGL(grouped_gemm_bf16_kernel<false>, dim3(blocks), dim3(kThreads), 0, s, h, w2, offsets, tiles,
                       n_tiles, I, H, I, 0, 0.0f, y_perm, H);
    return hipGetLastError();
}

}  // namespace tpg
