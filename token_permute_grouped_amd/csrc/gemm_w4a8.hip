// W4A8 expert FFN: FP8 E4M3 activations (one fp32 scale per 128 columns) times
// NVFP4 weights dequantised to FP8 in-kernel, on FP8 matrix cores
// (v_mfma_f32_32x32x64_f8f6f4 with unit block scales).
//
// Sources: FlashInfer "[SM90] Add W4A8 MegaMoE support" -- the fused kernel's
// NVFP4 -> FP8 dequant, the clamped SwiGLU, and its Usage section (E2M1 codes, one
// E4M3 scale per 16 values along K, FP32 activation scales per 128 channels); the
// split family's note that the second GEMM's activation scales are per 128 like
// the first's; follow-up #6517 point 4 (low-nibble-first packing, 6 * scale <= 448
// so the dequantised value fits E4M3, per-expert global scales).
//
// Three launches per grouped FFN:
//   1. GEMM1 + clamped SwiGLU: h = silu(g) * u in fp32, g, u = gs1_e * sum_kb xs[kb] * (x8 . w8)
//   2. re-quantisation of h per (row, 128 columns): s = amax/448 (1 if 0), q = e4m3(h / s)
//   3. GEMM2: y = gs2_e * sum_kb hs[kb] * (h8 . w8), rounded to bf16
//
// GEMM tiling.  A workgroup (4 waves) owns one expert m-tile of 128 token rows and
// 128 weight rows; wave w computes token block w (32 rows) against all 128 weight
// rows (4 MFMA blocks).  K advances 256 per stage: the workgroup dequantises the
// stage's 128 x 256 weights once into LDS (double buffered, one barrier per stage)
// and every wave reads them from there; activation fragments come straight from
// global memory (they are small and stay in L2).  The MFMA partial of each 128-wide
// K block is kept apart and added to the accumulator times that block's activation
// scale (fp32), so the per-128 scales are applied exactly as the definition states.
// The workload is bound by streaming the packed weights: each weight byte of an
// m-tile is read once.
//
// Dequant.  Eight codes (one dword, low nibble first) and their block scale become
// eight fp8 bytes: v_cvt_scalef32_pk_f32_fp4 (unit scale) gives the e2m1 values, an
// fp32 multiply by the scale is exact, v_med3 saturates to +-448 and
// v_cvt_pk_fp8_f32 rounds to nearest even.
//
// Operand layout of v_mfma_*_32x32x64_f8f6f4 (checked on the device): lane l holds
// row l % 32 and the 32 consecutive K bytes starting at 32 * (l / 32); the output
// layout is that of the 32 x 32 bf16 MFMA.  The weight fragment is the first
// operand, so a lane's accumulators are runs of 4 consecutive output columns of
// one token row.
#include <type_traits>

#include "moe_internal.h"

namespace tpg {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 128;       // token rows per m-tile (4 waves x 32)
constexpr int kBN = 128;       // weight rows per tile
constexpr int kKC = 256;       // K per stage
constexpr int kThreads = 256;
constexpr int kStage = kBN * kKC;  // fp8 bytes of one dequantised stage (32 KB)

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8((int)code, 0); }

// two fp32 values -> two e4m3 bytes (saturating, round to nearest even) into half kHi of `old`
template <bool kHi>
__device__ __forceinline__ uint32_t to_fp8x2(float a, float b, uint32_t old) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// eight packed e2m1 codes (low nibble first) with e4m3 block scale code `sc` -> eight
// e4m3 bytes.  The code is converted at unit scale and multiplied in fp32, which is
// exact (a 2-bit times a 4-bit significand), so the only rounding is the one to e4m3.
// A NaN scale (0x7F / 0xFF) makes all eight the NaN code 0x7F.
__device__ __forceinline__ u32x2 dequant8(uint32_t codes, uint32_t sc) {
    const float scale = e4m3_to_f32(sc & 0xffu);
    f32x2 p[4];
    p[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 0);
    p[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 1);
    p[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 2);
    p[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(codes, 1.0f, 3);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        p[i].x *= scale;
        p[i].y *= scale;
    }
    u32x2 r;
    r.x = to_fp8x2<true>(p[1].x, p[1].y, to_fp8x2<false>(p[0].x, p[0].y, 0u));
    r.y = to_fp8x2<true>(p[3].x, p[3].y, to_fp8x2<false>(p[2].x, p[2].y, 0u));
    if ((sc & 0x7fu) == 0x7fu) r = u32x2{0x7f7f7f7fu, 0x7f7f7f7fu};
    return r;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    return (uint32_t)f32_to_bf16(a) | ((uint32_t)f32_to_bf16(b) << 16);
}

// LDS slot (16-byte granule) of granule g of weight row r: 16 granules per 256-byte row
__device__ __forceinline__ int gslot(int r, int g) { return g ^ (r & 15); }

}  // namespace

template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads) void grouped_gemm_w4a8_kernel(
    const uint8_t *__restrict__ A8,      // [S][K] fp8 activations, expert-contiguous rows
    const float *__restrict__ As,        // [S][K/128] activation scales
    const uint8_t *__restrict__ Wq,      // [E][N][K/2] e2m1 codes, low nibble = even k
    const uint8_t *__restrict__ Wbs,     // [E][N][K/16] e4m3 block scales
    const float *__restrict__ Wgs,       // [E] global scales
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ tiles, const int32_t *__restrict__ n_tiles,
    int K, int N, int I, int il, float clamp,
    float *__restrict__ Hout,            // kSwiGLU: h fp32 [S][I]
    uint16_t *__restrict__ Yout, int ldy) {  // else: y bf16 [S][ldy]
    __shared__ __attribute__((aligned(1024))) unsigned char lds[2 * kStage];

    const int nb_n = N / kBN;
    const int mt = blockIdx.x / nb_n;
    const int nt = blockIdx.x % nb_n;
    if (mt >= n_tiles[0]) return;
    const int e = tiles[2 * mt];
    const int row_begin = offsets[e] + tiles[2 * mt + 1];
    const int rows = min(kBM, offsets[e + 1] - row_begin);

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int kb_n = K / 128;  // scale blocks per row

    // ---- weights: thread t dequantises 128 codes of tile row t/2 (half t%2 of the stage)
    const int wr_local = tid >> 1, whalf = tid & 1;
    int wrow;
    if (kSwiGLU) {  // tile rows [gate 32 | up 32 | gate 32 | up 32] for h columns nt*64 ..
        const int a = wr_local >> 5;
        const int c = nt * (kBN / 2) + (a >> 1) * 32 + (wr_local & 31);
        const bool up = a & 1;
        wrow = il == 0 ? (up ? I + c : c) : (c / il) * 2 * il + (up ? il : 0) + c % il;
    } else {
        wrow = nt * kBN + wr_local;
    }
    const uint8_t *wq = Wq + ((int64_t)e * N + wrow) * (K / 2) + whalf * 64;
    const uint8_t *wbs = Wbs + ((int64_t)e * N + wrow) * (K / 16) + whalf * 8;

    auto dequant_stage = [&](int kc, int buf) {
        const u32x4 *src = (const u32x4 *)(wq + kc * (kKC / 2));
        const u32x2 sc2 = *(const u32x2 *)(wbs + kc * (kKC / 16));
        const uint32_t sc[2] = {sc2.x, sc2.y};
        unsigned char *dst = lds + buf * kStage + wr_local * kKC;
#pragma unroll
        for (int q = 0; q < 4; ++q) {      // 16 bytes = 32 codes = 2 scale blocks
            const u32x4 c = src[q];
            const uint32_t s4 = sc[q >> 1] >> ((q & 1) * 16);
            const u32x2 d0 = dequant8(c.x, s4), d1 = dequant8(c.y, s4);
            const u32x2 d2 = dequant8(c.z, s4 >> 8), d3 = dequant8(c.w, s4 >> 8);
            u32x4 g0, g1;  // 32 fp8 bytes = granules 4q .. 4q+1 of this half
            g0.x = d0.x; g0.y = d0.y; g0.z = d1.x; g0.w = d1.y;
            g1.x = d2.x; g1.y = d2.y; g1.z = d3.x; g1.w = d3.y;
            const int g = whalf * 8 + q * 2;
            *(u32x4 *)(dst + gslot(wr_local, g) * 16) = g0;
            *(u32x4 *)(dst + gslot(wr_local, g + 1) * 16) = g1;
        }
    };

    // ---- activations of this wave's token block, read straight from global memory
    const int tok = wave * 32 + (lane & 31);  // token row within the tile (lane's MFMA column)
    const bool tok_live = tok < rows;
    const uint8_t *arow = A8 + (int64_t)(row_begin + (tok_live ? tok : 0)) * K + (lane >> 5) * 32;
    const float *srow = As + (int64_t)(row_begin + (tok_live ? tok : 0)) * kb_n;

    f32x16 acc[4], part[4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[a][v] = 0.f;

    const int nk = K / kKC;
    const bool wave_live = wave * 32 < rows;
    dequant_stage(0, 0);
    __syncthreads();
    for (int kc = 0; kc < nk; ++kc) {
        const int buf = kc & 1;
        if (kc + 1 < nk) dequant_stage(kc + 1, buf ^ 1);
        if (wave_live) {
            const unsigned char *sw = lds + buf * kStage;
#pragma unroll
            for (int sb = 0; sb < 2; ++sb) {  // two 128-wide scale blocks per stage
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int v = 0; v < 16; ++v) part[a][v] = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {  // two 64-wide MFMA K steps per scale block
                    const int ks = sb * 2 + h;
                    i32x8 xb;
                    {
                        const u32x4 *p = (const u32x4 *)(arow + kc * kKC + ks * 64);
                        u32x4 lo = tok_live ? p[0] : u32x4{0, 0, 0, 0};
                        u32x4 hi = tok_live ? p[1] : u32x4{0, 0, 0, 0};
                        xb = i32x8{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    }
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int r = a * 32 + (lane & 31);
                        const int g = ks * 4 + (lane >> 5) * 2;
                        const u32x4 lo = *(const u32x4 *)(sw + r * kKC + gslot(r, g) * 16);
                        const u32x4 hi = *(const u32x4 *)(sw + r * kKC + gslot(r, g + 1) * 16);
                        const i32x8 wa = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                          (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                        part[a] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, xb, part[a], 0, 0, 0, 127, 0,
                                                                                  127);
                    }
                }
                const float xs = tok_live ? srow[kc * 2 + sb] : 0.f;
#pragma unroll
                for (int a = 0; a < 4; ++a)
#pragma unroll
                    for (int v = 0; v < 16; ++v) acc[a][v] = fmaf(part[a][v], xs, acc[a][v]);
            }
        }
        __syncthreads();
    }

    if (!tok_live) return;
    const float gs = Wgs[e];
    const int half = lane >> 5;
    const int64_t row = row_begin + tok;
    if (kSwiGLU) {
        float *hrow = Hout + row * I;
#pragma unroll
        for (int pr = 0; pr < 2; ++pr)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int c0 = nt * (kBN / 2) + pr * 32 + g4 * 8 + half * 4;
                f32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    float g = gs * acc[2 * pr][g4 * 4 + q], u = gs * acc[2 * pr + 1][g4 * 4 + q];
                    if (clamp > 0.f) {
                        g = fminf(fmaxf(g, -clamp), clamp);
                        u = fminf(fmaxf(u, -clamp), clamp);
                    }
                    o[q] = g / (1.0f + expf(-g)) * u;
                }
                *(f32x4 *)(hrow + c0) = o;
            }
    } else {
        uint16_t *yrow = Yout + row * ldy;
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int c0 = nt * kBN + a * 32 + g4 * 8 + half * 4;
                u32x2 o;
                o.x = pack_bf16x2(gs * acc[a][g4 * 4 + 0], gs * acc[a][g4 * 4 + 1]);
                o.y = pack_bf16x2(gs * acc[a][g4 * 4 + 2], gs * acc[a][g4 * 4 + 3]);
                *(u32x2 *)(yrow + c0) = o;
            }
    }
}

// h fp32 [S][I] -> h8 e4m3 [S][I] + hs fp32 [S][I/128] for the live rows: one wave per
// (row, 128 columns); s = amax / 448 (1 if that is 0), q = e4m3(h / s), decided in fp32.
__global__ __launch_bounds__(256) void requant_fp8_kernel(const float *__restrict__ h, const int32_t *__restrict__ offsets,
                                                          int E, int I, uint8_t *__restrict__ h8,
                                                          float *__restrict__ hs) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nb = I / 128;
    const int64_t row = item / nb;
    const int b = (int)(item % nb);
    if (row >= offsets[E]) return;
    const f32x2 v = *(const f32x2 *)(h + row * I + b * 128 + 2 * lane);
    float m = fmaxf(fabsf(v.x), fabsf(v.y));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float s = m / 448.0f;
    if (s == 0.0f) s = 1.0f;
    const uint32_t q = to_fp8x2<false>(v.x / s, v.y / s, 0u);
    *(uint16_t *)(h8 + row * I + b * 128 + 2 * lane) = (uint16_t)(q & 0xffffu);
    if (lane == 0) hs[row * nb + b] = s;
}

// the dequant of every (e2m1 code c, e4m3 scale s) pair through the GEMMs' device routine,
// with the code in the even-k (low) nibble [0] and in the odd-k (high) nibble [1]
__global__ void w4a8_dequant_table_kernel(uint8_t *out8) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;  // 16 * 256 entries
    if (i >= 16 * 256) return;
    const uint32_t c = (uint32_t)(i >> 8), s = (uint32_t)(i & 255);
    const u32x2 lo = dequant8(c, s);       // code in nibble 0 (k even)
    const u32x2 hi = dequant8(c << 4, s);  // code in nibble 1 (k odd)
    out8[i] = (uint8_t)(lo.x & 0xff);
    out8[16 * 256 + i] = (uint8_t)((hi.x >> 8) & 0xff);
}

hipError_t launch_w4a8_dequant_table(uint8_t *out8, hipStream_t s) {
    hipLaunchKernelGGL(w4a8_dequant_table_kernel, dim3(16), dim3(256), 0, s, out8);
    return hipGetLastError();
}

hipError_t launch_grouped_ffn_w4a8(const uint8_t *x_perm, const float *x_perm_scale, const int32_t *offsets,
                                   const int32_t *tiles, const int32_t *n_tiles, int64_t max_tiles,
                                   const moe_weights &w, const moe_problem &p, float *h32, uint8_t *h8, float *hs,
                                   uint16_t *y_perm, hipStream_t s) {
    const int H = p.H, I = p.I;
    hipLaunchKernelGGL(grouped_gemm_w4a8_kernel<true>, dim3(max_tiles * (2 * I / kBN)), dim3(kThreads), 0, s, x_perm,
                       x_perm_scale, (const uint8_t *)w.w1, (const uint8_t *)w.w1_bscale, w.w1_gscale, offsets, tiles,
                       n_tiles, H, 2 * I, I, p.glu_interleave, p.swiglu_clamp, h32, (uint16_t *)nullptr, 0);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t items = n_slots(p) * (I / 128);
    hipLaunchKernelGGL(requant_fp8_kernel, dim3((items + 3) / 4), dim3(256), 0, s, h32, offsets, p.E, I, h8, hs);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(grouped_gemm_w4a8_kernel<false>, dim3(max_tiles * (H / kBN)), dim3(kThreads), 0, s, h8, hs,
                       (const uint8_t *)w.w2, (const uint8_t *)w.w2_bscale, w.w2_gscale, offsets, tiles, n_tiles, I,
                       H, I, 0, 0.0f, (float *)nullptr, y_perm, H);
    return hipGetLastError();
}

}  // namespace tpg
