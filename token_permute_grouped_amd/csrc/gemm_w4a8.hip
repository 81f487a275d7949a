// W4A8 expert FFN: FP8 E4M3 activations (one fp32 scale per 128 columns) times
// NVFP4 weights dequantised to FP8 in-kernel, on FP8 matrix cores
// (v_mfma_scale_f32_32x32x64_f8f6f4 with unit block scales), or times MXFP4 weights
// (kMX: E2M1 codes with one E8M0 scale per 32 along K) fed to the FP4 matrix cores as
// they are, the E8M0 byte as the instruction's weight block scale.
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
// tile.  Weights are never shared between waves: each wave loads its rows with
// line-coalesced loads (8 lanes per 128-byte line) three 256-wide K chunks ahead (four
// register sets), transposes each chunk through its own LDS slot into the MFMA operand
// layout (lane l: row l % 32, one contiguous 32-code run per 64-wide K step) and
// dequantises it there.  Activations are shared by the four waves: each chunk of the
// tile's token rows and its activation scales are loaded into registers two chunks
// ahead and written to LDS one chunk ahead (two buffers, swizzled).  Every load is an
// ordinary register load, so the compiler's own waits are exact: no wait drains the
// weight prefetch, and the chunk barriers carry no memory fence.  In the forward the
// first GEMM reads its rows straight from the token rows through row_src (the gather
// folded into its loads).  With at most 32 tokens (and K a multiple of 1024) the
// kernel is persistent: each workgroup walks several tiles and fetches the next one's
// first chunks under the current one's last steps (w4a8_tiles, kLoop).
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
// one token row.  With an FP4 first operand (measured with one wave and chosen
// operands): lane l holds 32 codes (16 bytes, low nibble first) of K 32 (l / 32)
// .. +31, its scale byte scales exactly those, and the FP8 second operand then pairs
// its bytes 0-15 with K 16 (l / 32) .. +15 and bytes 16-31 with K 32 + 16 (l / 32)
// .. +15, so the MXFP4 path reads its activation granules in that order.
#include <algorithm>

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
    int gather_k, a_rows;    // rows of A8 / As: T with row_src, else S
    const uint8_t *Wq;   // [E][N][K/2] e2m1 codes, low nibble = even k
    const uint8_t *Wbs;  // [E][N][K/16] e4m3 block scales (MXFP4: [E][N][K/32] e8m0)
    // Bytes between consecutive rows of a 32-row block and between consecutive 256-wide K
    // pieces of one row, for the codes (w_) and the block scales (s_): row-major storage
    // (pitch K/2, step 128) or the tiled layout (pitch 128, step 4096: a block's piece is one
    // contiguous 4 KB run).  A 32-row block occupies the same bytes in both.
    int w_pitch, w_step, s_pitch, s_step;
    const float *Wgs;    // [E] global scales
    int K, N, I, il, E;
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

// One work item of the block -> tile map: expert, first row, live rows, n-tile.
struct W4Tile {
    bool valid;
    int e, row_begin, rows, nt;
};

// Virtual block v -> tile.  The tile list holds each expert's m-tiles together.  Expert e's
// blocks are [first * nb_n, (first + nm) * nb_n); they run in units of G n-tiles, the nm
// m-tiles of an n-tile G blocks apart: with G = 8 those land on one XCD (block b runs on XCD
// b mod 8, and the persistent grid's stride is a multiple of 8) at the same time, so the
// weights an expert's second m-tile streams are L2 hits.
__device__ __forceinline__ W4Tile w4a8_tile_of(int v, int nb_n, const int32_t *__restrict__ offsets,
                                              const int32_t *__restrict__ tiles, int n_mt) {
    W4Tile t{};
    const int tq = v / nb_n;  // a tile of the expert this block works for
    t.valid = tq < n_mt;
    if (!t.valid) return t;
    t.e = tiles[2 * tq];
    const int first = tq - tiles[2 * tq + 1] / kBM;
    const int nm = (offsets[t.e + 1] - offsets[t.e] + kBM - 1) / kBM;
    const int G = nb_n % 8 == 0 ? 8 : nb_n % 4 == 0 ? 4 : nb_n % 2 == 0 ? 2 : 1;
    const int r = v - first * nb_n, unit = nm * G;
    const int mt = first + (r % unit) / G;
    t.nt = (r / unit) * G + (r % unit) % G;
    t.row_begin = offsets[t.e] + tiles[2 * mt + 1];
    t.rows = min(kBM, offsets[t.e + 1] - t.row_begin);
    return t;
}

// The tiles of virtual blocks v0, v0 + stride, ... (kLoop), or of v0 alone.  With kLoop the
// loads a tile's last steps would issue past its last chunk fetch the next tile's first
// chunks instead, so the pipeline runs on across tiles and only the first tile pays for a
// prologue (needs K / kKC to be a multiple of kNBuf, so that every tile starts at the same
// register set and buffer phase).
template <bool kSwiGLU, bool kMX, int NTB, bool kLoop>
__device__ __forceinline__ void w4a8_tiles(const W4Args &g, int v0, int stride, const int32_t *__restrict__ offsets,
                                           const int32_t *__restrict__ tiles, int n_mt, unsigned char *act,
                                           float *xsl, unsigned char *wlds, const u32x2 *lut) {
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = g.K, kb_n = K / 128;
    const int nc = K / kKC;
    const int nb_n = g.N / kBN;
    const int sg = tid & 15, sr = tid >> 4;
    const int srow = min(tid, kBM - 1);
    constexpr int kSB = kMX ? 32 : 16;  // K values per weight block scale
    const bool gather = g.row_src != nullptr;

    // ---- addressing of one tile.  Weights: each wave streams its own 32 rows, in chunks of
    // 256 K (128 code bytes + 16 scale bytes per row); loads cover whole 128-byte lines (8 lanes
    // per row), and the wave transposes each chunk through its own LDS slot into the MFMA
    // operand layout.  Activations: thread t stages granule t % 16 of token rows t / 16 + 16 i,
    // and thread r < 32 NTB the chunk's two activation scales of token row r.  Raw buffer
    // resources bound every read (rows past the tile's live rows read as zero), so every lane
    // issues the same unconditional loads and the compiler's wait counts stay exact.  With
    // row_src (the gather fused into GEMM1) row r is read from token row_src[r] / k of x: the
    // row_src loads are issued first, unconditionally (a row past the tile reads the last live
    // row's slot and gets an out-of-range offset), and consumed later (finish()).
    // Buffer descriptors: per tile (its expert's matrices, its rows), or with kLoop one set
    // over the whole arrays for every tile (the host checks that all byte offsets fit 31 bits),
    // so that a tile's addressing is just the per-lane offsets below.
    struct Rs {
        __amdgpu_buffer_rsrc_t W, Ws, A, S;
    };
    auto make_rs = [&](const W4Tile &t) {
        Rs r;
        const int64_t w0 = kLoop ? 0 : (int64_t)t.e * g.N;  // first weight row the descriptor starts at
        const int64_t nw = kLoop ? (int64_t)g.E * g.N : g.N;
        r.W = __builtin_amdgcn_make_buffer_rsrc((void *)(g.Wq + w0 * (K / 2)), (short)0, (int)(nw * (K / 2)),
                                                0x00020000);
        r.Ws = __builtin_amdgcn_make_buffer_rsrc((void *)(g.Wbs + w0 * (K / kSB)), (short)0, (int)(nw * (K / kSB)),
                                                 0x00020000);
        const bool whole = gather || kLoop;  // rows addressed from the start of the array
        const int64_t a0 = whole ? 0 : t.row_begin;
        const int na = gather ? g.a_rows : kLoop ? g.a_rows : t.rows;
        r.A = __builtin_amdgcn_make_buffer_rsrc((void *)(g.A8 + a0 * K), (short)0, na * K, 0x00020000);
        r.S = __builtin_amdgcn_make_buffer_rsrc((void *)(g.As + a0 * kb_n), (short)0, na * kb_n * 4, 0x00020000);
        return r;
    };
    struct Addr {
        uint32_t woff[4], wsoff, aoff[NTB * 2], soff;
        int src[NTB * 2 + 1];
    };
    auto start_addr = [&](Addr &a, const W4Tile &t) {
        auto weight_row = [&](int rl) {  // weight matrix row of row rl of this wave
            if (kSwiGLU) {  // waves 0, 1: gate rows of h columns nt*64 + [0, 64); waves 2, 3: the matching up rows
                const bool up = wave >= 2;
                const int c = t.nt * (kBN / 2) + (wave & 1) * 32 + rl;
                return g.il == 0 ? (up ? g.I + c : c) : (c / g.il) * 2 * g.il + (up ? g.il : 0) + c % g.il;
            }
            return t.nt * kBN + wave * 32 + rl;
        };
        const int er = kLoop ? t.e * g.N : 0;  // expert's first row within the descriptor
        // a wave's 32 weight rows are one 32-row block of the matrix (weight_row(r) = weight_row(0) + r)
        const int blk = er + weight_row(0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a.woff[i] = (uint32_t)(blk * (K / 2) + ((lane >> 3) + 8 * i) * g.w_pitch + (lane & 7) * 16);
        a.wsoff = (uint32_t)(blk * (K / kSB) + (lane >> 1) * g.s_pitch + (lane & 1) * (kKC / kSB / 2));
#pragma unroll
        for (int i = 0; i < NTB * 2 + 1; ++i) a.src[i] = 0;
        if (gather) {
#pragma unroll
            for (int i = 0; i < NTB * 2; ++i) a.src[i] = g.row_src[t.row_begin + min(sr + 16 * i, t.rows - 1)];
            a.src[NTB * 2] = g.row_src[t.row_begin + min(srow, t.rows - 1)];
        }
    };
    auto finish_addr = [&](Addr &a, const W4Tile &t) {
        // token of slot s = t*k + j: s / k in double precision, exact for integers below 2^31
#pragma unroll
        for (int i = 0; i < NTB * 2 + 1; ++i) asm volatile("" : "+v"(a.src[i])::"memory");
        const int rb = kLoop ? t.row_begin : 0;  // tile's first row within the descriptor (no gather)
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) {
            const int r = sr + 16 * i;
            const int tok = (int)((double)a.src[i] / (double)g.gather_k);
            a.aoff[i] = r >= t.rows ? 0x80000000u : (uint32_t)((gather ? tok : rb + r) * K + sg * 16);
        }
        const int ts = (int)((double)a.src[NTB * 2] / (double)g.gather_k);
        a.soff = srow >= t.rows ? 0x80000000u : (uint32_t)((gather ? ts : rb + srow) * kb_n * 4);
    };

    Rs rs;
    auto load_w = [&](WChunk &w, const Addr &a, int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i) w.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.W, a.woff[i], c * g.w_step, 0);
        if constexpr (kMX)
            w.s = u32x2{__builtin_amdgcn_raw_buffer_load_b32(rs.Ws, a.wsoff, c * g.s_step, 0), 0u};
        else
            w.s = __builtin_amdgcn_raw_buffer_load_b64(rs.Ws, a.wsoff, c * g.s_step, 0);
    };
    unsigned char *const wl = wlds + wave * (2 * kWSlot);  // this wave's two staging slots
    auto store_w = [&](const WChunk &w, int slot) {
        unsigned char *d = wl + slot * kWSlot;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)(d + ((lane >> 3) + 8 * i) * kWRow + (lane & 7) * 16) = w.c[i];
        if constexpr (kMX)
            *(uint32_t *)(d + kWScales + (lane >> 1) * 16 + (lane & 1) * 4) = w.s.x;
        else
            *(u32x2 *)(d + kWScales + (lane >> 1) * 16 + (lane & 1) * 8) = w.s;
    };
    u32x4 ar[NTB * 2];
    u32x2 ars;
    auto load_a = [&](const Addr &a, int c) {
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) ar[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.A, a.aoff[i], c * kKC, 0);
        ars = __builtin_amdgcn_raw_buffer_load_b64(rs.S, a.soff, c * 8, 0);
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
            // block scales of this lane's K runs: NVFP4 e4m3 bytes 8q + 4h + 2t, +1 (one per 16 K),
            // MXFP4 e8m0 byte 4q + 2h + t (one per 32 K)
            const uint32_t sq = kMX ? *(const uint32_t *)(wsr - 4 * half + 4 * q) >> (16 * half)
                                    : *(const uint32_t *)(wsr + 8 * q);
#pragma unroll
            for (int t = 0; t < 2; ++t) {  // two 64-wide MFMA steps per 128-wide block
                const u32x4 cw = *(const u32x4 *)(wr + 64 * q + 16 * t);
                i32x8 wa;
                int wscale = 127;  // e8m0 1.0: the NVFP4 weights are dequantised to fp8 here
                if constexpr (kMX) {  // the e2m1 codes are the MFMA's fp4 operand as they are
                    wa = i32x8{(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
                    wscale = (int)((sq >> (8 * t)) & 0xffu);
                } else {
                    const uint32_t sc = sq >> (16 * t);
                    const u32x2 t0 = lut[sc & 0xffu], t1 = lut[(sc >> 8) & 0xffu];
                    const u32x2 d0 = dequant8(cw.x, t0), d1 = dequant8(cw.y, t0);
                    const u32x2 d2 = dequant8(cw.z, t1), d3 = dequant8(cw.w, t1);
                    wa = i32x8{(int)d0.x, (int)d0.y, (int)d1.x, (int)d1.y, (int)d2.x, (int)d2.y, (int)d3.x, (int)d3.y};
                }
                // activation granules (16 K each) of this lane's 32 fp8 bytes.  Both operands fp8: one
                // contiguous run, the same K as the weight run.  Weights fp4: the instruction pairs
                // the weight run of lane half h (K 32h..32h+31 of the step) with activation bytes
                // 0-15 of half 0 and of half 1, so a lane of half h holds granules h and h + 2 of
                // the step's weight K (measured on the device with one wave and chosen operands)
                const int gk_lo = kMX ? 8 * q + 2 * t + half : 8 * q + 4 * half + 2 * t;
                const int gk_hi = kMX ? gk_lo + 4 : gk_lo + 1;
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    const int r = tb * 32 + (lane & 31);
                    const u32x4 lo = *(const u32x4 *)(ab + r * kKC + aslot(r, gk_lo) * 16);
                    const u32x4 hi = *(const u32x4 *)(ab + r * kKC + aslot(r, gk_hi) * 16);
                    const i32x8 xb = {(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                                      (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
                    // operand formats: weights fp4 e2m1 (4) or fp8 e4m3 (0), activations fp8 e4m3
                    part[tb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wa, xb, part[tb], kMX ? 4 : 0, 0, 0,
                                                                               wscale, 0, 127);
                }
            }
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tb][v] = fmaf(part[tb][v], xs[tb], acc[tb][v]);
        }
    };

    // ---- epilogue of tile t.  xch: LDS the up waves hand their accumulators to the gate waves
    // through (an activation buffer no chunk still needs).
    auto epilogue = [&](const W4Tile &t, float *xch) {
        const float gs = g.Wgs[t.e];
        if (kSwiGLU) {
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
                    if (tok >= t.rows) continue;
                    float *hrow = g.Hout + (int64_t)(t.row_begin + tok) * g.I;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int c0 = t.nt * (kBN / 2) + wave * 32 + g4 * 8 + half * 4;
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
                if (tok >= t.rows) continue;
                uint16_t *yrow = g.Yout + (int64_t)(t.row_begin + tok) * g.ldy;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c0 = t.nt * kBN + wave * 32 + g4 * 8 + half * 4;
                    u32x2 o;
                    o.x = pack_bf16x2(gs * acc[tb][g4 * 4 + 0], gs * acc[tb][g4 * 4 + 1]);
                    o.y = pack_bf16x2(gs * acc[tb][g4 * 4 + 2], gs * acc[tb][g4 * 4 + 3]);
                    *(u32x2 *)(yrow + c0) = o;
                }
            }
        }
    };

    W4Tile cur = w4a8_tile_of(v0, nb_n, offsets, tiles, n_mt);
    if (!cur.valid) return;  // before any barrier: the whole workgroup leaves
    rs = make_rs(cur);
    Addr A;
    start_addr(A, cur);

    // ---- prologue (first tile only).  The row_src loads land under the first weight chunk's.
    // It ends like a loop step (activations of the next chunk, then one weight set), so the
    // loads in flight at the loop head follow the same pattern on entry as on the back edge
    // and the compiler's waits there stay exact.
    WChunk w[kNBuf];
    load_w(w[0], A, 0);
    finish_addr(A, cur);
    load_a(A, 0);
#pragma unroll
    for (int c = 1; c < kNBuf - 2; ++c) load_w(w[c], A, min(c, nc - 1));
    store_a(0);
    load_a(A, min(1, nc - 1));
    load_w(w[kNBuf - 2], A, min(kNBuf - 2, nc - 1));
    store_w(w[0], 0);
    lds_barrier();  // chunk 0 staged, scale table built

    int v = v0;
    for (;;) {
        // the next tile's addressing (kLoop only; otherwise requests past the last chunk repeat
        // it).  Its row_src loads are issued now and consumed at step 2, when every older load in
        // flight is one this tile needs by then anyway; its first request comes at step nc - 2.
        W4Tile nxt{};
        Addr B = A;
        if (kLoop) {
            nxt = w4a8_tile_of(v + stride, nb_n, offsets, tiles, n_mt);
            if (nxt.valid) start_addr(B, nxt);
        }
        const bool go_on = kLoop && nxt.valid;
        // request c of this tile: chunk c below nc, else chunk c - nc of the next tile (or this
        // tile's last chunk again)
        auto req = [&](int c) { return c < nc ? c : go_on ? c - nc : nc - 1; };
#pragma unroll
        for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[tb][q] = 0.f;

        // Chunk c computes from activation buffer c % 2 and this wave's weight slot c % 2, then
        // stages the weights of chunk c + 1 (set (c + 1) % 4, loaded two steps ago) into the other
        // slot (this wave last read it in chunk c - 1; a wave's LDS accesses stay in order) and
        // the activations of chunk c + 1 into the other buffer (last read in chunk c - 1, before
        // the previous barrier), loads the activations of chunk c + 2 and the weights of chunk
        // c + kNBuf - 1 (into the set of chunk c - 1).  Whole groups of four steps: a step past
        // the last chunk (single-tile form with K / kKC not a multiple of four) skips only its
        // compute (which issues no memory loads), so every path through the loop issues the same
        // loads and the compiler's waits at the loop head see the regular pattern.
        for (int c0 = 0; c0 < nc; c0 += kNBuf) {
#pragma unroll
            for (int sidx = 0; sidx < kNBuf; ++sidx) {
                const int c = c0 + sidx;
                if (kLoop && sidx == 2 && c0 == 0 && go_on) finish_addr(B, nxt);
                if (c < nc) compute(c & 1);
                store_w(w[(sidx + 1) % kNBuf], (c + 1) & 1);
                store_a((c + 1) & 1);
                const int ca = req(c + 2), cw = req(c + kNBuf - 1);
                load_a(c + 2 < nc ? A : B, ca);
                load_w(w[(sidx + kNBuf - 1) % kNBuf], c + kNBuf - 1 < nc ? A : B, cw);
                lds_barrier();
            }
        }
        // every wave has passed the last chunk's barrier; buffer nc % 2 holds the next tile's
        // first chunk (kLoop: nc is even), so the exchange uses the other one
        epilogue(cur, (float *)(act + ((nc + 1) & 1) * kActBuf));
        if (!go_on) break;
        lds_barrier();  // the exchange buffer is read before chunk 1 of the next tile is staged in it
        cur = nxt;
        A = B;
        v += stride;
    }
}

}  // namespace

#define TPG_W4A8_LDS                                                                                   \
    __shared__ __attribute__((aligned(1024))) unsigned char act[2 * kActBuf];                          \
    __shared__ u32x2 lut[256];                                                                         \
    __shared__ float xsl[2 * kBM * 2]; /* activation scales of the staged chunks [buf][row][block] */ \
    __shared__ __attribute__((aligned(16))) unsigned char wlds[4 * 2 * kWSlot]; /* 2 slots per wave */ \
    if constexpr (!kMX) lut[threadIdx.x] = scaled_e2m1_table(threadIdx.x); /* read after a tile's first barrier */

// one tile per workgroup; its token-block count from its own rows
template <bool kSwiGLU, bool kMX>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_w4a8_kernel(W4Args g, const int32_t *__restrict__ offsets,
                                                                     const int32_t *__restrict__ tiles,
                                                                     const int32_t *__restrict__ n_tiles) {
    TPG_W4A8_LDS
    const int n_mt = n_tiles[0];
    const W4Tile t = w4a8_tile_of(blockIdx.x, g.N / kBN, offsets, tiles, n_mt);
    if (!t.valid) return;
    if (t.rows > 32)
        w4a8_tiles<kSwiGLU, kMX, 2, false>(g, blockIdx.x, 0, offsets, tiles, n_mt, act, xsl, wlds, lut);
    else
        w4a8_tiles<kSwiGLU, kMX, 1, false>(g, blockIdx.x, 0, offsets, tiles, n_mt, act, xsl, wlds, lut);
}

// persistent (at most 32 rows per tile): workgroup b takes virtual blocks b, b + gridDim.x, ...
template <bool kSwiGLU, bool kMX>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_w4a8_persistent_kernel(
    W4Args g, const int32_t *__restrict__ offsets, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles) {
    TPG_W4A8_LDS
    w4a8_tiles<kSwiGLU, kMX, 1, true>(g, blockIdx.x, gridDim.x, offsets, tiles, n_tiles[0], act, xsl, wlds, lut);
}
#undef TPG_W4A8_LDS

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

namespace {
// Grid and mode of one W4A8 GEMM launch.  With T <= 32 (an expert holds at most T rows, so
// every m-tile fits one 32-row block) and K / kKC a multiple of kNBuf the kernel is
// persistent: two workgroups per CU (the kernel's occupancy) walk the virtual blocks with the
// grid as stride and prefetch each next tile's first chunks under the current one's last
// steps (W4A8 layer, T = 16: 223 -> 214 us per forward).  Above 32 tokens a persistent
// kernel would have to fix two token blocks for every tile (most tiles then hold under 32
// rows at T = 64) and measured slower; there and for other K, one tile per workgroup.
struct W4Launch {
    int64_t grid;
    bool persistent;
};
W4Launch w4_launch(int64_t max_tiles, int N, int K, int E, int a_rows, int T) {
    const int64_t blocks = max_tiles * (N / kBN);
    // the persistent form addresses every expert's codes and every activation row from one
    // descriptor each: their byte offsets must stay below 2^31
    const bool fits = (int64_t)E * N * (K / 2) <= 0x7FFFFFFF && (int64_t)a_rows * K <= 0x7FFFFFFF;
    if (T > 32 || (K / kKC) % kNBuf != 0 || !fits) return {blocks, false};
    int dev = 0, n_cu = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                  hipSuccess || n_cu <= 0)
        return {blocks, false};
    return {std::min<int64_t>(blocks, 2 * (int64_t)n_cu), true};
}

template <bool kSwiGLU, bool kMX>
void launch_w4a8_gemm_as(const W4Launch &l, const W4Args &g, const int32_t *offsets, const int32_t *tiles,
                         const int32_t *n_tiles, hipStream_t s) {
    if (l.persistent)
        hipLaunchKernelGGL((grouped_gemm_w4a8_persistent_kernel<kSwiGLU, kMX>), dim3(l.grid), dim3(kThreads), 0, s, g,
                           offsets, tiles, n_tiles);
    else
        hipLaunchKernelGGL((grouped_gemm_w4a8_kernel<kSwiGLU, kMX>), dim3(l.grid), dim3(kThreads), 0, s, g, offsets,
                           tiles, n_tiles);
}
template <bool kSwiGLU>
void launch_w4a8_gemm(bool mx, const W4Launch &l, const W4Args &g, const int32_t *offsets, const int32_t *tiles,
                      const int32_t *n_tiles, hipStream_t s) {
    if (mx)
        launch_w4a8_gemm_as<kSwiGLU, true>(l, g, offsets, tiles, n_tiles, s);
    else
        launch_w4a8_gemm_as<kSwiGLU, false>(l, g, offsets, tiles, n_tiles, s);
}
}  // namespace

namespace {
// code and scale strides of one matrix stack with K columns in the given layout (see W4Args)
void set_layout(W4Args &g, int K, bool mx, int layout) {
    const int sb = mx ? 32 : 16;  // K values per block scale
    const bool tiled = layout == MOE_W4_LAYOUT_TILED;
    g.w_pitch = tiled ? kKC / 2 : K / 2;
    g.w_step = tiled ? 32 * (kKC / 2) : kKC / 2;
    g.s_pitch = tiled ? kKC / sb : K / sb;
    g.s_step = tiled ? 32 * (kKC / sb) : kKC / sb;
}
}  // namespace

hipError_t launch_grouped_ffn_w4a8(const uint8_t *x_perm, const float *x_perm_scale, const int32_t *row_src,
                                   const int32_t *offsets, const int32_t *tiles, const int32_t *n_tiles,
                                   int64_t max_tiles, const moe_weights &w, const moe_problem &p, float *h32,
                                   uint8_t *h8, float *hs, uint16_t *y_perm, hipStream_t s) {
    const int H = p.H, I = p.I;
    if (row_src && !gather_fits_fp8(p.T, H)) return hipErrorInvalidValue;
    const int S = (int)n_slots(p);
    const bool mx = p.prec == MOE_PREC_W4A8_MX;
    const W4Launch l1 = w4_launch(max_tiles, 2 * I, H, p.E, row_src ? p.T : S, p.T),
                   l2 = w4_launch(max_tiles, H, I, p.E, S, p.T);
    W4Args g1{};
    g1.A8 = x_perm;
    g1.As = x_perm_scale;
    g1.row_src = row_src;
    g1.gather_k = p.k;
    g1.a_rows = row_src ? p.T : S;
    g1.Wq = (const uint8_t *)w.w1;
    g1.Wbs = (const uint8_t *)w.w1_bscale;
    g1.Wgs = w.w1_gscale;
    g1.K = H;
    g1.N = 2 * I;
    g1.I = I;
    g1.il = p.glu_interleave;
    g1.E = p.E;
    g1.clamp = p.swiglu_clamp;
    g1.Hout = h32;
    set_layout(g1, H, mx, w.w4_layout);
    launch_w4a8_gemm<true>(mx, l1, g1, offsets, tiles, n_tiles, s);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t items = n_slots(p) * (I / 128);
    hipLaunchKernelGGL(requant_fp8_kernel, dim3((items + 3) / 4), dim3(256), 0, s, h32, offsets, p.E, I, h8, hs);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    W4Args g2{};
    g2.A8 = h8;
    g2.As = hs;
    g2.gather_k = 1;
    g2.a_rows = S;
    g2.Wq = (const uint8_t *)w.w2;
    g2.Wbs = (const uint8_t *)w.w2_bscale;
    g2.Wgs = w.w2_gscale;
    g2.K = I;
    g2.N = H;
    g2.I = I;
    g2.E = p.E;
    g2.Yout = y_perm;
    g2.ldy = H;
    set_layout(g2, I, mx, w.w4_layout);
    launch_w4a8_gemm<false>(mx, l2, g2, offsets, tiles, n_tiles, s);
    return hipGetLastError();
}

// MOE_W4_LAYOUT_TILED from row-major codes and block scales: one thread per destination unit
// (16 code bytes, or 8 scale bytes); destination unit d of a 32-row block's 256-wide piece c
// holds row r, bytes 16 j (8 j) of that row's piece
__global__ __launch_bounds__(256) void tile_weights_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                           int64_t units, int unit_bytes, int piece_units,
                                                           int row_bytes, int n_pieces) {
    const int64_t d = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (d >= units) return;
    const int j = (int)(d % piece_units);
    const int r = (int)((d / piece_units) % 32);
    const int64_t c = (d / (piece_units * 32)) % n_pieces;
    const int64_t blk = d / ((int64_t)piece_units * 32 * n_pieces);  // expert * (N / 32) + block
    const int64_t from = (blk * 32 + r) * row_bytes + c * (piece_units * unit_bytes) + j * unit_bytes;
    if (unit_bytes == 16)
        *(uint4 *)(dst + d * 16) = *(const uint4 *)(src + from);
    else
        *(uint2 *)(dst + d * 8) = *(const uint2 *)(src + from);
}

hipError_t launch_tile_weights(const uint8_t *codes, const uint8_t *bscale, uint8_t *codes_tiled,
                               uint8_t *bscale_tiled, int E, int N, int K, bool mx, hipStream_t s) {
    const int sb = mx ? 32 : 16, n_pieces = K / kKC;
    const int64_t rows = (int64_t)E * N;
    const int64_t cu = rows * (K / 2) / 16;      // 16-byte code units
    const int64_t su = rows * (K / sb) / 8;      // 8-byte scale units
    hipLaunchKernelGGL(tile_weights_kernel, dim3((cu + 255) / 256), dim3(256), 0, s, codes, codes_tiled, cu, 16,
                       (kKC / 2) / 16, K / 2, n_pieces);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tile_weights_kernel, dim3((su + 255) / 256), dim3(256), 0, s, bscale, bscale_tiled, su, 8,
                       (kKC / sb) / 8, K / sb, n_pieces);
    return hipGetLastError();
}

}  // namespace tpg
