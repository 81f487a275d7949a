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
// The GEMMs stream packed weights, which is what bounds them at small token counts.
// Tiling.  A workgroup (4 waves) owns one expert m-tile of up to 64 token rows and
// 128 weight rows; wave w owns 32 weight rows (one MFMA block) and every token of the
// tile.  Weights are never shared between waves, so each wave loads its rows straight
// into registers in the MFMA operand layout (lane l: row l % 32, one contiguous
// 32-code run per 64-wide K step) and dequantises them there.  K advances 256 per
// chunk; weights are loaded three chunks ahead (four register sets).  Activations are
// shared by the four waves: each chunk of the tile's token rows and its activation
// scales are loaded into registers two chunks ahead and written to LDS one chunk
// ahead (two buffers, swizzled).  Every load is an ordinary register load, so the
// compiler's own waits are exact: no wait drains the weight prefetch, and the chunk
// barriers carry no memory fence.
// K is visited so that both halves of a 64-wide MFMA step lie in one 128-wide
// activation-scale block; the partial sum of each block is added to the accumulator
// times that block's activation scale (fp32), as the definition states.
//
// Dequant.  A per-workgroup LDS table holds, for every e4m3 block-scale code, the
// e4m3 codes of the eight e2m1 magnitudes times that scale (rounded to nearest even,
// saturating at +-448; the products are exact in fp32).  Eight packed codes (one
// dword, low nibble first) then become eight e4m3 bytes with two v_perm_b32 table
// selects, a sign xor and two v_perm_b32 interleaves.
//
// Operand layout of v_mfma_*_32x32x64_f8f6f4 (checked on the device): lane l holds
// row l % 32 and the 32 consecutive K bytes starting at 32 * (l / 32); the output
// layout is that of the 32 x 32 bf16 MFMA.  The weight fragment is the first
// operand, so a lane's accumulators are runs of 4 consecutive output columns of
// one token row.
#include "moe_internal.h"

namespace tpg {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = kGemmBMW4A8;  // token rows per m-tile (2 blocks of 32)
constexpr int kBN = 128;          // weight rows per workgroup (4 waves x 32)
constexpr int kKC = 256;          // K per chunk
constexpr int kNBuf = 4;          // weight register sets (weights kNBuf - 1 chunks ahead)
constexpr int kThreads = 256;
constexpr int kActBuf = kBM * kKC;  // bytes of one staged activation chunk (16 KB, two buffers)
static_assert(kBM == 64, "the tile holds at most two 32-token blocks");

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) { return __builtin_amdgcn_cvt_f32_fp8((int)code, 0); }

// two fp32 values -> two e4m3 bytes (saturating, round to nearest even) into half kHi of `old`
template <bool kHi>
__device__ __forceinline__ uint32_t to_fp8x2(float a, float b, uint32_t old) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, kHi);
}

// byte m = e4m3 code of (e2m1 magnitude m) * e4m3(sc), m = 0..7.  A NaN scale gives
// NaN codes with the scale's sign (the code's sign is applied by the xor in dequant8).
__device__ __forceinline__ u32x2 scaled_e2m1_table(uint32_t sc) {
    const float s = e4m3_to_f32(sc & 0xffu);
    u32x2 t;
    t.x = to_fp8x2<true>(1.0f * s, 1.5f * s, to_fp8x2<false>(0.0f * s, 0.5f * s, 0u));
    t.y = to_fp8x2<true>(4.0f * s, 6.0f * s, to_fp8x2<false>(2.0f * s, 3.0f * s, 0u));
    if ((sc & 0x7fu) == 0x7fu) t.x = t.y = (sc & 0x80u) ? 0xffffffffu : 0x7f7f7f7fu;
    return t;
}

// eight e2m1 codes (low nibble first) -> eight e4m3 codes, through the table t of their
// block scale.  v_perm_b32 selector bytes 0..3 pick bytes of the second source, 4..7 of
// the first.
__device__ __forceinline__ u32x2 dequant8(uint32_t x, u32x2 t) {
    const uint32_t me = __builtin_amdgcn_perm(t.y, t.x, x & 0x07070707u);         // codes 0, 2, 4, 6
    const uint32_t mo = __builtin_amdgcn_perm(t.y, t.x, (x >> 4) & 0x07070707u);  // codes 1, 3, 5, 7
    const uint32_t ve = me ^ ((x << 4) & 0x80808080u);
    const uint32_t vo = mo ^ (x & 0x80808080u);
    return u32x2{__builtin_amdgcn_perm(vo, ve, 0x05010400u), __builtin_amdgcn_perm(vo, ve, 0x07030602u)};
}


// LDS slot (16-byte granule) of granule g of staged token row r: 16 granules per row
__device__ __forceinline__ int aslot(int r, int g) { return g ^ (r & 15); }

// LDS barrier without a global-memory fence: register loads stay in flight across it
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

struct W4Args {
    const uint8_t *A8;   // [S][K] fp8 activations, expert-contiguous rows, or with row_src the
                         // token rows [a_rows][K]
    const float *As;     // [S][K/128] activation scales (with row_src: [a_rows][K/128])
    const int32_t *row_src;  // NULL, or [S]: row r reads token row row_src[r] / gather_k
    int gather_k, a_rows;
    const uint8_t *Wq;   // [E][N][K/2] e2m1 codes, low nibble = even k
    const uint8_t *Wbs;  // [E][N][K/16] e4m3 block scales
    const float *Wgs;    // [E] global scales
    int K, N, I, il;
    float clamp;
    float *Hout;         // GEMM1: h fp32 [S][I]
    uint16_t *Yout;      // GEMM2: y bf16 [S][ldy]
    int ldy;
};

// weights of one 256-wide K chunk as one lane loads them (line-coalesced): 16 code bytes of
// each of rows l/8 + 8i (i < 4) at byte 16 (l % 8), and 8 scale bytes of row l/2 at byte
// 8 (l % 2), rows counted within the wave's 32
struct WChunk {
    u32x4 c[4];
    u32x2 s;
};

// per-wave LDS staging of one chunk's weights in rows: 32 code rows of 128 bytes padded to
// 144 (so that 16 consecutive rows read at one column hit 16 distinct bank groups), then
// 32 scale rows of 16 bytes
constexpr int kWRow = 144;
constexpr int kWScales = 32 * kWRow;
constexpr int kWSlot = kWScales + 32 * 16;  // 5120 bytes per chunk and wave

template <bool kSwiGLU, int NTB>
__device__ __forceinline__ void w4a8_tile(const W4Args &g, int e, int row_begin, int rows, int nt,
                                          unsigned char *act, float *xsl, unsigned char *wlds, const u32x2 *lut) {
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = g.K, kb_n = K / 128;
    const int nc = K / kKC;

    // ---- weights.  Each wave streams its own 32 rows, in chunks of 256 K (128 code bytes
    // + 16 scale bytes per row): loads cover whole 128-byte lines (8 lanes per row), and the
    // wave transposes each chunk through its own LDS slot into the MFMA operand layout.
    auto weight_row = [&](int rl) {  // weight matrix row of row rl of this wave
        if (kSwiGLU) {  // waves 0, 1: gate rows of h columns nt*64 + [0, 64); waves 2, 3: the matching up rows
            const bool up = wave >= 2;
            const int c = nt * (kBN / 2) + (wave & 1) * 32 + rl;
            return g.il == 0 ? (up ? g.I + c : c) : (c / g.il) * 2 * g.il + (up ? g.il : 0) + c % g.il;
        }
        return nt * kBN + wave * 32 + rl;
    };
    const __amdgpu_buffer_rsrc_t rsW = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(g.Wq + (int64_t)e * g.N * (K / 2)), (short)0, g.N * (K / 2), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsWs = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(g.Wbs + (int64_t)e * g.N * (K / 16)), (short)0, g.N * (K / 16), 0x00020000);
    uint32_t woff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) woff[i] = (uint32_t)(weight_row((lane >> 3) + 8 * i) * (K / 2) + (lane & 7) * 16);
    const uint32_t wsoff = (uint32_t)(weight_row(lane >> 1) * (K / 16) + (lane & 1) * 8);
    auto load_w = [&](WChunk &w, int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rsW, woff[i], c * (kKC / 2), 0);
        w.s = __builtin_amdgcn_raw_buffer_load_b64(rsWs, wsoff, c * (kKC / 16), 0);
    };
    unsigned char *const wl = wlds + wave * (2 * kWSlot);  // this wave's two staging slots
    auto store_w = [&](const WChunk &w, int slot) {
        unsigned char *d = wl + slot * kWSlot;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)(d + ((lane >> 3) + 8 * i) * kWRow + (lane & 7) * 16) = w.c[i];
        *(u32x2 *)(d + kWScales + (lane >> 1) * 16 + (lane & 1) * 8) = w.s;
    };

    // ---- activations: thread t stages granule t % 16 of token rows t / 16 + 16 i, and thread
    // r < 32 NTB the chunk's two activation scales of token row r.  Raw buffer resources
    // bound the reads (rows past the tile's live rows read as zero), so every lane issues the
    // same unconditional loads and the compiler's wait counts stay exact.  With row_src (the
    // gather fused into GEMM1) a row is read from token row_src[r] / k of x; the row_src loads
    // are issued now, unconditionally (a row past the tile reads the last live row's slot and
    // gets an out-of-range offset), and consumed after the first weight chunk's loads.
    const int sg = tid & 15, sr = tid >> 4;
    const bool gather = g.row_src != nullptr;
    const int srow = min(tid, kBM - 1);
    int src[NTB * 2 + 1] = {};
    if (gather) {
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) src[i] = g.row_src[row_begin + min(sr + 16 * i, rows - 1)];
        src[NTB * 2] = g.row_src[row_begin + min(srow, rows - 1)];
    }
    const __amdgpu_buffer_rsrc_t rsA = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(g.A8 + (gather ? 0 : (int64_t)row_begin * K)), (short)0, gather ? g.a_rows * K : rows * K,
        0x00020000);
    const __amdgpu_buffer_rsrc_t rsS = __builtin_amdgcn_make_buffer_rsrc(
        (void *)(g.As + (gather ? 0 : (int64_t)row_begin * kb_n)), (short)0,
        (gather ? g.a_rows : rows) * kb_n * 4, 0x00020000);
    uint32_t aoff[NTB * 2], soff;
    auto init_aoff = [&]() {
        // token of slot s = t*k + j: s / k in double precision, exact for integers below 2^31
#pragma unroll
        for (int i = 0; i < NTB * 2 + 1; ++i) asm volatile("" : "+v"(src[i])::"memory");
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) {
            const int r = sr + 16 * i;
            const int t = (int)((double)src[i] / (double)g.gather_k);
            aoff[i] = !gather ? (uint32_t)(r * K + sg * 16) : r >= rows ? 0x80000000u : (uint32_t)(t * K + sg * 16);
        }
        const int ts = (int)((double)src[NTB * 2] / (double)g.gather_k);
        soff = !gather ? (uint32_t)(srow * kb_n * 4) : srow >= rows ? 0x80000000u : (uint32_t)(ts * kb_n * 4);
    };
    u32x4 ar[NTB * 2];
    u32x2 ars;
    auto load_a = [&](int c) {
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) ar[i] = __builtin_amdgcn_raw_buffer_load_b128(rsA, aoff[i], c * kKC, 0);
        ars = __builtin_amdgcn_raw_buffer_load_b64(rsS, soff, c * 8, 0);
    };
    auto store_a = [&](int buf) {
        unsigned char *dst = act + buf * kActBuf;
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) {
            const int r = sr + 16 * i;
            *(u32x4 *)(dst + r * kKC + aslot(r, sg) * 16) = ar[i];
        }
        if (tid < NTB * 32) *(u32x2 *)(xsl + buf * (kBM * 2) + tid * 2) = ars;
    };

    f32x16 acc[NTB];
#pragma unroll
    for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[tb][v] = 0.f;

    // lane (row r = l % 32, half h = l / 32) of 64-K step (q, t) takes code bytes
    // [64 q + 32 h + 16 t, +16) of its row and their two scale bytes 8 q + 4 h + 2 t, +1
    auto compute = [&](int buf) {
        const unsigned char *ab = act + buf * kActBuf;
        const float *xr = xsl + buf * (kBM * 2);
        const unsigned char *wr = wl + buf * kWSlot + (lane & 31) * kWRow + half * 32;
        const unsigned char *wsr = wl + buf * kWSlot + kWScales + (lane & 31) * 16 + half * 4;
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float xs[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) xs[tb] = xr[(tb * 32 + (lane & 31)) * 2 + q];
            f32x16 part[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int v = 0; v < 16; ++v) part[tb][v] = 0.f;
            const uint32_t sq = *(const uint32_t *)(wsr + 8 * q);
#pragma unroll
            for (int t = 0; t < 2; ++t) {  // two 64-wide MFMA steps per 128-wide block
                const u32x4 cw = *(const u32x4 *)(wr + 64 * q + 16 * t);
                const uint32_t sc = sq >> (16 * t);
                const u32x2 t0 = lut[sc & 0xffu], t1 = lut[(sc >> 8) & 0xffu];
                const u32x2 d0 = dequant8(cw.x, t0), d1 = dequant8(cw.y, t0);
                const u32x2 d2 = dequant8(cw.z, t1), d3 = dequant8(cw.w, t1);
                const i32x8 wa = {(int)d0.x, (int)d0.y, (int)d1.x, (int)d1.y,
                                  (int)d2.x, (int)d2.y, (int)d3.x, (int)d3.y};
                const int gk = 8 * q + 4 * half + 2 * t;  // granule of this lane's 32 K bytes
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    const int r = tb * 32 + (lane & 31);
                    const u32x4 lo = *(const u32x4 *)(ab + r * kKC + aslot(r, gk) * 16);
                    const u32x4 hi = *(const u32x4 *)(ab + r * kKC + aslot(r, gk + 1) * 16);
                    const i32x8 xb = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    part[tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, xb, part[tb], 0, 0, 0, 127, 0,
                                                                               127);
                }
            }
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tb][v] = fmaf(part[tb][v], xs[tb], acc[tb][v]);
        }
    };

    // ---- main loop.  Chunk c computes from weight set c % 4 and activation buffer c % 2,
    // then writes the staged activations of chunk c + 1 into the other buffer (last read
    // by chunk c - 1, before the previous barrier), loads the activations of chunk c + 2
    // and the weights of chunk c + 3 (into the set of chunk c - 1).  Requests past the
    // last chunk repeat it (cache hits), so every path issues the same loads.
    // The prologue ends like a loop step (activations of the next chunk, then one weight
    // set), so the loads in flight at the loop head follow the same pattern on entry as on
    // the back edge and the compiler's waits there stay exact.
    WChunk w[kNBuf];
    load_w(w[0], 0);
    init_aoff();  // the row_src loads land under the first weight chunk's
    load_a(0);
#pragma unroll
    for (int c = 1; c < kNBuf - 2; ++c) load_w(w[c], min(c, nc - 1));
    store_a(0);
    load_a(min(1, nc - 1));
    load_w(w[kNBuf - 2], min(kNBuf - 2, nc - 1));
    store_w(w[0], 0);
    lds_barrier();  // chunk 0 staged, scale table built
    // Chunk c computes from activation buffer c % 2 and this wave's weight slot c % 2, then
    // stages the weights of chunk c + 1 (set (c + 1) % 4, loaded two steps ago) into the other
    // slot (this wave last read it in chunk c - 1; a wave's LDS accesses stay in order) and
    // the activations of chunk c + 1 into the other buffer (last read in chunk c - 1, before
    // the previous barrier), loads the activations of chunk c + 2 and the weights of chunk
    // c + kNBuf - 1 (into the set of chunk c - 1).  Requests past the last chunk repeat it.
    // Whole groups of four steps: a step past the last chunk skips only its compute (which
    // issues no memory loads), so every path through the loop issues the same loads and
    // the compiler's waits at the loop head see the regular pattern.
    for (int c0 = 0; c0 < nc; c0 += kNBuf) {
#pragma unroll
        for (int sidx = 0; sidx < kNBuf; ++sidx) {
            const int c = c0 + sidx;
            if (c < nc) compute(c & 1);
            store_w(w[(sidx + 1) % kNBuf], (c + 1) & 1);
            store_a((c + 1) & 1);
            load_a(min(c + 2, nc - 1));
            load_w(w[(sidx + kNBuf - 1) % kNBuf], min(c + kNBuf - 1, nc - 1));
            lds_barrier();
        }
    }

    // ---- epilogue (every wave has passed the last chunk's barrier: the buffers are free)
    const float gs = g.Wgs[e];
    if (kSwiGLU) {
        // the up waves hand their accumulators to the gate waves through LDS
        float *xch = (float *)act;  // [2 waves][NTB][16][64]
        if (wave >= 2)
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int v = 0; v < 16; ++v) xch[(((wave - 2) * NTB + tb) * 16 + v) * 64 + lane] = acc[tb][v];
        lds_barrier();
        if (wave < 2) {
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int tok = tb * 32 + (lane & 31);
                if (tok >= rows) continue;
                float *hrow = g.Hout + (int64_t)(row_begin + tok) * g.I;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c0 = nt * (kBN / 2) + wave * 32 + g4 * 8 + half * 4;
                    f32x4 o;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int v = g4 * 4 + q;
                        float gv = gs * acc[tb][v];
                        float uv = gs * xch[((wave * NTB + tb) * 16 + v) * 64 + lane];
                        if (g.clamp > 0.f) {
                            gv = fminf(fmaxf(gv, -g.clamp), g.clamp);
                            uv = fminf(fmaxf(uv, -g.clamp), g.clamp);
                        }
                        o[q] = gv / (1.0f + expf(-gv)) * uv;
                    }
                    *(f32x4 *)(hrow + c0) = o;
                }
            }
        }
    } else {
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb) {
            const int tok = tb * 32 + (lane & 31);
            if (tok >= rows) continue;
            uint16_t *yrow = g.Yout + (int64_t)(row_begin + tok) * g.ldy;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
                const int c0 = nt * kBN + wave * 32 + g4 * 8 + half * 4;
                u32x2 o;
                o.x = pack_bf16x2(gs * acc[tb][g4 * 4 + 0], gs * acc[tb][g4 * 4 + 1]);
                o.y = pack_bf16x2(gs * acc[tb][g4 * 4 + 2], gs * acc[tb][g4 * 4 + 3]);
                *(u32x2 *)(yrow + c0) = o;
            }
        }
    }
}

}  // namespace

template <bool kSwiGLU>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_w4a8_kernel(W4Args g, const int32_t *__restrict__ offsets,
                                                                     const int32_t *__restrict__ tiles,
                                                                     const int32_t *__restrict__ n_tiles) {
    __shared__ __attribute__((aligned(1024))) unsigned char act[2 * kActBuf];
    __shared__ u32x2 lut[256];
    __shared__ float xsl[2 * kBM * 2];  // activation scales of the staged chunks [buf][row][block]
    __shared__ __attribute__((aligned(16))) unsigned char wlds[4 * 2 * kWSlot];  // weight staging, 2 slots per wave

    // Block -> tile.  The tile list holds each expert's m-tiles together.  Expert e's blocks are
    // [first * nb_n, (first + nm) * nb_n); they run in units of G n-tiles, the nm m-tiles of an
    // n-tile G blocks apart: with G = 8 those land on one XCD (block b runs on XCD b mod 8) at
    // the same time, so the weights an expert's second m-tile streams are L2 hits.
    const int nb_n = g.N / kBN;
    const int tq = blockIdx.x / nb_n;  // a tile of the expert this block works for
    if (tq >= n_tiles[0]) return;
    const int e = tiles[2 * tq];
    const int first = tq - tiles[2 * tq + 1] / kBM;
    const int nm = (offsets[e + 1] - offsets[e] + kBM - 1) / kBM;
    const int G = nb_n % 8 == 0 ? 8 : nb_n % 4 == 0 ? 4 : nb_n % 2 == 0 ? 2 : 1;
    const int r = blockIdx.x - first * nb_n, unit = nm * G;
    const int mt = first + (r % unit) / G;
    const int nt = (r / unit) * G + (r % unit) % G;
    const int row_begin = offsets[e] + tiles[2 * mt + 1];
    const int rows = min(kBM, offsets[e + 1] - row_begin);

    lut[threadIdx.x] = scaled_e2m1_table(threadIdx.x);  // read after the first barrier of the tile
    if (rows > 32)
        w4a8_tile<kSwiGLU, 2>(g, e, row_begin, rows, nt, act, xsl, wlds, lut);
    else
        w4a8_tile<kSwiGLU, 1>(g, e, row_begin, rows, nt, act, xsl, wlds, lut);
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

// the dequant of every (e2m1 code, e4m3 scale s) pair through the GEMMs' device routine:
// a dword holding code (c + p) mod 16 at nibble position p = 0..7 (low nibble first) is
// dequantised with scale s, and byte p of the result goes to out8[p][c][s]
__global__ void w4a8_dequant_table_kernel(uint8_t *out8) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;  // 16 * 256 entries
    if (i >= 16 * 256) return;
    const uint32_t c = (uint32_t)(i >> 8), s = (uint32_t)(i & 255);
    uint32_t x = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p) x |= ((c + p) & 15u) << (4 * p);
    const u32x2 d = dequant8(x, scaled_e2m1_table(s));
#pragma unroll
    for (int p = 0; p < 8; ++p) out8[p * 16 * 256 + i] = (uint8_t)(((p < 4 ? d.x : d.y) >> (8 * (p & 3))) & 0xffu);
}

hipError_t launch_w4a8_dequant_table(uint8_t *out8, hipStream_t s) {
    hipLaunchKernelGGL(w4a8_dequant_table_kernel, dim3(16), dim3(256), 0, s, out8);
    return hipGetLastError();
}

hipError_t launch_grouped_ffn_w4a8(const uint8_t *x_perm, const float *x_perm_scale, const int32_t *row_src,
                                   const int32_t *offsets, const int32_t *tiles, const int32_t *n_tiles,
                                   int64_t max_tiles, const moe_weights &w, const moe_problem &p, float *h32,
                                   uint8_t *h8, float *hs, uint16_t *y_perm, hipStream_t s) {
    const int H = p.H, I = p.I;
    if (row_src && !gather_fits_fp8(p.T, H)) return hipErrorInvalidValue;
    W4Args g1{x_perm, x_perm_scale, row_src, p.k, p.T, (const uint8_t *)w.w1, (const uint8_t *)w.w1_bscale,
              w.w1_gscale, H, 2 * I, I, p.glu_interleave, p.swiglu_clamp, h32, nullptr, 0};
    hipLaunchKernelGGL(grouped_gemm_w4a8_kernel<true>, dim3(max_tiles * (2 * I / kBN)), dim3(kThreads), 0, s, g1,
                       offsets, tiles, n_tiles);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t items = n_slots(p) * (I / 128);
    hipLaunchKernelGGL(requant_fp8_kernel, dim3((items + 3) / 4), dim3(256), 0, s, h32, offsets, p.E, I, h8, hs);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    W4Args g2{h8, hs, nullptr, 1, 0, (const uint8_t *)w.w2, (const uint8_t *)w.w2_bscale, w.w2_gscale,
              I, H, I, 0, 0.0f, nullptr, y_perm, H};
    hipLaunchKernelGGL(grouped_gemm_w4a8_kernel<false>, dim3(max_tiles * (H / kBN)), dim3(kThreads), 0, s, g2,
                       offsets, tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace tpg
