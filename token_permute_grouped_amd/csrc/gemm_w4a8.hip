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
// At decode sizes (w4a8_split_gemm1) GEMM1 runs two workgroups per tile, one per K half,
// writing raw partial sums, and launch 2 adds the halves and applies gs1 and the SwiGLU first
// (requant_swiglu_fp8_kernel): a CU then holds two workgroups' waves, one of which computes
// (NVFP4: dequantises) while the other waits on its loads, and twice the weight bytes in flight.
//
// The GEMMs stream packed weights, which is what bounds them at small token counts.
// Tiling.  A workgroup (4 waves) owns one expert m-tile of up to 64 token rows (an
// expert's last tile up to 96: the tile list lets a remainder of at most 32 rows join
// the tile before it, so that it does not stream the expert's weights once more for a
// few rows) and 128 weight rows; wave w owns 32 weight rows (one MFMA block) and every
// token of the tile.  Weights are never shared between waves: each wave loads its rows
// into a ring of register sets, one 256-wide K chunk per set, as many chunks ahead as the
// ring allows (four sets; fewer where measured faster, see NBUF).  Row-major weights come in line-coalesced loads (8 lanes per
// 128-byte line) and each chunk is transposed, one step before its compute, through the
// wave's own LDS slot into the MFMA operand layout (lane l: row l % 32, one contiguous
// 32-code run per 64-wide K step).  The tiled layout (moe_w4a8_tile_weights) already
// stores every 32-row, 256-wide piece in that operand order, four 1 KB runs in lane
// order, so a wave's loads are contiguous and land in the operand registers as they are
// (kTiled): no LDS transpose.  NVFP4 codes are dequantised as they are read.  Activations are
// shared by the four waves: each chunk of the tile's token rows and its activation scales
// are loaded into registers two chunks ahead and written to LDS one chunk ahead (two
// buffers, swizzled).  Every load is an
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
// selects, a sign xor and two v_perm_b32 interleaves; in the tiled layout the codes
// of a dword are stored so that the table selects already give K order (no
// interleave).  Weight loads are non-temporal: a call reads each weight byte about
// once.
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
#include "route_token.h"
#include "tile_list.h"
#include "w4a8_index.h"

namespace tpg {

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

static_assert(w4::kBM == kGemmBMW4A8, "m-tiles of two 32-token blocks (three for an expert's merged last tile)");

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

// eight e2m1 codes -> eight e4m3 codes, through the table t of their block scale.  kSplit
// false: the codes are packed low nibble first (byte i holds codes 2i and 2i + 1); true: the
// tiled layout's NVFP4 order (byte i holds codes i and i + 4), whose low and high nibbles
// already give the outputs in K order.  v_perm_b32 selector bytes 0..3 pick bytes of the
// second source, 4..7 of the first.
template <bool kSplit = false>
__device__ __forceinline__ u32x2 dequant8(uint32_t x, u32x2 t) {
    const uint32_t me = __builtin_amdgcn_perm(t.y, t.x, x & 0x07070707u);         // low nibbles
    const uint32_t mo = __builtin_amdgcn_perm(t.y, t.x, (x >> 4) & 0x07070707u);  // high nibbles
    const uint32_t ve = me ^ ((x << 4) & 0x80808080u);
    const uint32_t vo = mo ^ (x & 0x80808080u);
    if constexpr (kSplit) return u32x2{ve, vo};
    return u32x2{__builtin_amdgcn_perm(vo, ve, 0x05010400u), __builtin_amdgcn_perm(vo, ve, 0x07030602u)};
}


using w4::kActBuf;
using w4::kBM;
using w4::kBN;
using w4::kKC;
using w4::kNBuf;
using w4::kThreads;
using w4::kWSlot;
using w4::Tile;

// Cache policy of the weight loads: nt (non-temporal, bit 1 of the buffer instruction's cache
// policy on gfx950).  A call reads each weight byte about once, and the lines it would allocate
// only displace others: after a cache flush that leaves the L2 and the last-level cache full of
// dirty lines (a 512 MB write before each call), the W4A8 layer (H 7168, I 2048, E 32, top-8)
// takes 100.9 -> 66.8 us at T=1 (NVFP4), 92.6 -> 58.9 us (MXFP4), 207 -> 143 us at T=16 (MXFP4),
// 284 -> 268 us at T=256 (MXFP4).  Forwards repeated back to back on one layer lose 0-6 % (that
// layer's weights then stay in the 256 MB last-level cache, which a model's many layers do not).
constexpr int kWeightPolicy = 2;

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
    float *Hout;         // GEMM1: h fp32 [S][I]; with split, the partial sums [2 halves][gate, up][S][I]
    int split;           // GEMM1: 1 = one tile per workgroup, workgroup b sums K half b % 2 of tile b / 2 and
                         // writes its partial sums; 2 = each workgroup sums both halves apart and adds them
                         // at the end (the same arithmetic in one workgroup)
    int64_t part_stride;  // with split: S * I (elements between the four partial-sum planes)
    uint16_t *Yout;      // GEMM2: y bf16 [S][ldy]
    int ldy;
    const int32_t *row_dst;  // GEMM2: NULL, or [S]: row r of the tile order goes to y row row_dst[r]
};

// weights of one 256-wide K chunk as one lane loads them (line-coalesced): 16 code bytes of
// each of rows l/8 + 8i (i < 4) at byte 16 (l % 8), and 8 scale bytes of row l/2 at byte
// 8 (l % 2), rows counted within the wave's 32
struct WChunk {
    u32x4 c[4];
    u32x2 s;
};

// Tile order of the multi-launch GEMMs: virtual blocks v0, v0 + stride, ... (the persistent
// form), or v0 alone.  No waits and nothing to signal.
struct StaticSched {
    static constexpr bool kRowDst = true;  // GEMM2 honours W4Args::row_dst
    int v, stride, nb_n, n_mt;
    const int32_t *offsets, *tiles;
    bool merge;  // the tile list merges an expert's last partial tile of at most 32 rows
    __device__ Tile first() { return w4::tile_of(v, nb_n, offsets, tiles, n_mt, merge); }
    __device__ Tile next() {
        v += stride;
        return w4::tile_of(v, nb_n, offsets, tiles, n_mt, merge);
    }
    __device__ void before_act(const Tile &) {}
    __device__ void after_tile(const Tile &) {}
};

// The tiles sc hands out, in its order (kLoop: all of them, one after another; otherwise its
// first only).  With kLoop the loads a tile's last steps would issue past its last chunk fetch
// the next tile's first chunks instead, so the pipeline runs on across tiles and only the first
// tile pays for a prologue (needs K / kKC to be a multiple of kNBuf, so that every tile starts at
// the same register set and buffer phase).  sc.before_act(t) runs (uniformly, in every thread)
// before the first activation load of tile t, sc.after_tile(t) after t's output is written.
template <bool kSwiGLU, bool kMX, int NTB, bool kLoop, class Sched, int kSplit = 0, bool kTiled = false>
__device__ __forceinline__ void w4a8_tiles(const W4Args &g, Sched &sc, unsigned char *act, float *xsl,
                                           unsigned char *wlds, const u32x2 *lut) {
    const int tid = threadIdx.x, lane = tid & 63, half = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int K = g.K, kb_n = K / 128;
    // kSplit (GEMM1 only, the value of g.split): 1 = this workgroup sums K half blockIdx.x % 2 and
    // writes its partial sums; 2 = the two K halves are summed apart and added at the end
    static_assert(kSplit == 0 || (kSwiGLU && NTB == 1), "K splits serve GEMM1 at decode sizes");
    const int nc = (kSplit == 1 ? K / 2 : K) / kKC;               // chunks this workgroup sums
    const int kc0 = kSplit == 1 ? (int)(blockIdx.x & 1) * nc : 0;  // its first chunk
    const int sg = w4::act_gran(tid);
    const int srow = w4::act_scale_row(tid);
    constexpr int kSB = kMX ? 32 : 16;  // K values per weight block scale
    const bool gather = g.row_src != nullptr;

    // ---- addressing of one tile.  Weights: each wave streams its own 32 rows, in chunks of
    // 256 K (128 code bytes + 16 scale bytes per row); row-major weights in loads that cover
    // whole 128-byte lines (8 lanes per row), which the wave transposes through its own LDS slot
    // into the MFMA operand layout, tiled weights in contiguous loads already in that layout (see
    // w4::tiled_code_pos).  Activations: thread t stages granule t % 16 of token rows t / 16 + 16 i,
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
    auto make_rs = [&](const Tile &t) {
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
    auto start_addr = [&](Addr &a, const Tile &t) {
        const int er = kLoop ? t.e * g.N : 0;  // expert's first row within the descriptor
        // a wave's 32 weight rows are one 32-row block of the matrix (weight_row(r) = weight_row(0) + r)
        const int blk = er + w4::weight_row(kSwiGLU, t.nt, wave, 0, g.I, g.il);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a.woff[i] = kTiled ? w4::w_code_off_tiled(blk, K, lane, i) : w4::w_code_off(blk, K, lane, i, g.w_pitch);
        a.wsoff = kTiled ? w4::w_scale_off_tiled(blk, K, kSB, lane) : w4::w_scale_off(blk, K, kSB, lane, g.s_pitch);
#pragma unroll
        for (int i = 0; i < NTB * 2 + 1; ++i) a.src[i] = 0;
        if (gather) {
#pragma unroll
            for (int i = 0; i < NTB * 2; ++i)
                a.src[i] = g.row_src[t.row_begin + min(w4::act_row(tid, i), t.rows - 1)];
            a.src[NTB * 2] = g.row_src[t.row_begin + min(srow, t.rows - 1)];
        }
    };
    auto finish_addr = [&](Addr &a, const Tile &t) {
        // token of slot s = t*k + j: s / k in double precision, exact for integers below 2^31
#pragma unroll
        for (int i = 0; i < NTB * 2 + 1; ++i) asm volatile("" : "+v"(a.src[i])::"memory");
        const int rb = kLoop ? t.row_begin : 0;  // tile's first row within the descriptor (no gather)
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) {
            const int r = w4::act_row(tid, i);
            const int tok = (int)((double)a.src[i] / (double)g.gather_k);
            a.aoff[i] = r >= t.rows ? w4::kDeadOff : w4::a_off(gather ? tok : rb + r, K, sg);
        }
        const int ts = (int)((double)a.src[NTB * 2] / (double)g.gather_k);
        a.soff = srow >= t.rows ? w4::kDeadOff : w4::s_off(gather ? ts : rb + srow, K);
    };

    Rs rs;
    auto load_w = [&](WChunk &w, const Addr &a, int c) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            w.c[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.W, a.woff[i], (kc0 + c) * g.w_step, kWeightPolicy);
        if constexpr (kMX)
            w.s = u32x2{__builtin_amdgcn_raw_buffer_load_b32(rs.Ws, a.wsoff, (kc0 + c) * g.s_step, kWeightPolicy),
                        0u};
        else
            w.s = __builtin_amdgcn_raw_buffer_load_b64(rs.Ws, a.wsoff, (kc0 + c) * g.s_step, kWeightPolicy);
    };
    // this wave's staging slot: a chunk's weights are written after the wave's reads of the
    // previous chunk's, and one wave's LDS accesses complete in order, so one slot serves
    unsigned char *const wl = wlds + wave * kWSlot;
    auto store_w = [&](const WChunk &w) {  // row-major weights only
        unsigned char *d = wl;
#pragma unroll
        for (int i = 0; i < 4; ++i) *(u32x4 *)(d + w4::lds_wcode(lane, i)) = w.c[i];
        if constexpr (kMX)
            *(uint32_t *)(d + w4::lds_wscale(lane, true)) = w.s.x;
        else
            *(u32x2 *)(d + w4::lds_wscale(lane, false)) = w.s;
    };
    u32x4 ar[NTB * 2];
    u32x2 ars;
    auto load_a = [&](const Addr &a, int c) {
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i)
            ar[i] = __builtin_amdgcn_raw_buffer_load_b128(rs.A, a.aoff[i], (kc0 + c) * kKC, 0);
        ars = __builtin_amdgcn_raw_buffer_load_b64(rs.S, a.soff, (kc0 + c) * 8, 0);
    };
    auto store_a = [&](int buf) {
        unsigned char *dst = act + buf * kActBuf;
#pragma unroll
        for (int i = 0; i < NTB * 2; ++i) *(u32x4 *)(dst + w4::lds_act(w4::act_row(tid, i), sg)) = ar[i];
        if (tid < NTB * 32) *(u32x2 *)(xsl + w4::lds_xs(buf, tid, 0)) = ars;
    };

    f32x16 acc[NTB];
    f32x16 acc_lo[kSplit == 2 ? NTB : 1];  // the first K half's sum

    // lane (row r = l % 32, half h = l / 32) of 64-K step (q, t) takes code bytes
    // [64 q + 32 h + 16 t, +16) of its row and their two scale bytes 8 q + 4 h + 2 t, +1: from
    // the wave's staging slot, or (tiled weights) straight from the chunk's registers (code
    // set 2 q + t; scale dword q (NVFP4), or halfword q (MXFP4))
    auto compute = [&](int buf, const WChunk &wc) {
        const unsigned char *ab = act + buf * kActBuf;
        const unsigned char *wr = wl + w4::lds_wread(lane);
        const unsigned char *wsr = wl + w4::lds_wsread(lane);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            float xs[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) xs[tb] = xsl[w4::lds_xs(buf, tb * 32 + (lane & 31), q)];
            f32x16 part[NTB];
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int v = 0; v < 16; ++v) part[tb][v] = 0.f;
            // block scales of this lane's K runs: NVFP4 e4m3 bytes 8q + 4h + 2t, +1 (one per 16 K),
            // MXFP4 e8m0 byte 4q + 2h + t (one per 32 K)
            const uint32_t sq = kTiled ? (kMX ? wc.s.x >> (16 * q) : (q ? wc.s.y : wc.s.x))
                                : kMX ? *(const uint32_t *)(wsr - 4 * half + 4 * q) >> (16 * half)
                                      : *(const uint32_t *)(wsr + 8 * q);
#pragma unroll
            for (int t = 0; t < 2; ++t) {  // two 64-wide MFMA steps per 128-wide block
                const u32x4 cw = kTiled ? wc.c[2 * q + t] : *(const u32x4 *)(wr + 64 * q + 16 * t);
                i32x8 wa;
                int wscale = 127;  // e8m0 1.0: the NVFP4 weights are dequantised to fp8 here
                if constexpr (kMX) {  // the e2m1 codes are the MFMA's fp4 operand as they are
                    wa = i32x8{(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
                    wscale = (int)((sq >> (8 * t)) & 0xffu);
                } else {
                    const uint32_t sc = sq >> (16 * t);
                    const u32x2 t0 = lut[sc & 0xffu], t1 = lut[(sc >> 8) & 0xffu];
                    const u32x2 d0 = dequant8<kTiled>(cw.x, t0), d1 = dequant8<kTiled>(cw.y, t0);
                    const u32x2 d2 = dequant8<kTiled>(cw.z, t1), d3 = dequant8<kTiled>(cw.w, t1);
                    wa = i32x8{(int)d0.x, (int)d0.y, (int)d1.x, (int)d1.y, (int)d2.x, (int)d2.y, (int)d3.x, (int)d3.y};
                }
                // activation granules (16 K each) of this lane's 32 fp8 bytes.  Both operands fp8: one
                // contiguous run, the same K as the weight run.  Weights fp4: the instruction pairs
                // the weight run of lane half h (K 32h..32h+31 of the step) with activation bytes
                // 0-15 of half 0 and of half 1, so a lane of half h holds granules h and h + 2 of
                // the step's weight K (measured on the device with one wave and chosen operands)
                const int gk_lo = w4::gran_lo(kMX, q, t, half), gk_hi = w4::gran_hi(kMX, q, t, half);
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    const int r = tb * 32 + (lane & 31);
                    const u32x4 lo = *(const u32x4 *)(ab + w4::lds_act(r, gk_lo));
                    const u32x4 hi = *(const u32x4 *)(ab + w4::lds_act(r, gk_hi));
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
    auto epilogue = [&](const Tile &t, float *xch) {
        const float gs = g.Wgs[t.e];
        if (kSplit == 1) {
            // raw partial sums of this K half (no global scale, no SwiGLU: requant_swiglu_fp8_kernel
            // adds the halves and applies both): gate waves to plane 2 half, up waves to 2 half + 1,
            // at the h column each accumulator belongs to
            float *plane = g.Hout + (int64_t)(2 * (int)(blockIdx.x & 1) + (wave >> 1)) * g.part_stride;
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb) {
                const int tok = tb * 32 + (lane & 31);
                if (tok >= t.rows) continue;
                float *prow = plane + (int64_t)(t.row_begin + tok) * g.I;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c0 = w4::h_col(t.nt, wave & 1, g4, lane);
                    *(f32x4 *)(prow + c0) = f32x4{acc[tb][g4 * 4], acc[tb][g4 * 4 + 1], acc[tb][g4 * 4 + 2],
                                                  acc[tb][g4 * 4 + 3]};
                }
            }
        } else if (kSwiGLU) {
            if (wave >= 2)
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                    for (int v = 0; v < 16; ++v) xch[w4::lds_xch(wave - 2, NTB, tb, v, lane)] = acc[tb][v];
            lds_barrier();
            if (wave < 2) {
#pragma unroll
                for (int tb = 0; tb < NTB; ++tb) {
                    const int tok = tb * 32 + (lane & 31);
                    if (tok >= t.rows) continue;
                    float *hrow = g.Hout + (int64_t)(t.row_begin + tok) * g.I;
#pragma unroll
                    for (int g4 = 0; g4 < 4; ++g4) {
                        const int c0 = w4::h_col(t.nt, wave, g4, lane);
                        f32x4 o;
#pragma unroll
                        for (int q = 0; q < 4; ++q) {
                            const int v = g4 * 4 + q;
                            float gv = gs * acc[tb][v];
                            float uv = gs * xch[w4::lds_xch(wave, NTB, tb, v, lane)];
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
                const int yr = t.row_begin + tok;
                const int32_t *row_dst = Sched::kRowDst ? g.row_dst : nullptr;
                uint16_t *yrow = g.Yout + (int64_t)(row_dst ? row_dst[yr] : yr) * g.ldy;
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                    const int c0 = w4::y_col(t.nt, wave, g4, lane);
                    u32x2 o;
                    o.x = pack_bf16x2(gs * acc[tb][g4 * 4 + 0], gs * acc[tb][g4 * 4 + 1]);
                    o.y = pack_bf16x2(gs * acc[tb][g4 * 4 + 2], gs * acc[tb][g4 * 4 + 3]);
                    *(u32x2 *)(yrow + c0) = o;
                }
            }
        }
    };

    Tile cur = sc.first();
    if (!cur.valid) return;  // uniform: the whole workgroup leaves (no barrier passed yet)
    rs = make_rs(cur);
    Addr A;
    start_addr(A, cur);

    // ---- prologue (first tile only).  The row_src loads land under the first weight chunk's.
    // It ends like a loop step (activations of the next chunk, then one weight set), so the
    // loads in flight at the loop head follow the same pattern on entry as on the back edge
    // and the compiler's waits there stay exact.
    // weight register sets: kNBuf; for three token blocks (their accumulators take the
    // registers) one fewer.  With tiled weights, whose registers also hold the chunk being
    // computed, the measured best (W4A8 layer, each against the neighbouring counts): two for
    // three token blocks (three: 2-5 % slower at T = 256, NVFP4 spilling), two for one token
    // block outside the persistent form (the K-split GEMM1 at T = 1, one-block tiles above 32
    // tokens: MXFP4 T = 1 -4 %, T = 64 -3 %; the persistent form keeps four: two made MXFP4
    // T = 4 5 % and NVFP4 T = 16 2 % slower), four for two token blocks (three: 2 % slower at
    // T = 128)
    constexpr int NBUF = NTB == 3 ? (kTiled ? 2 : kNBuf - 1) : (NTB == 1 && kTiled && !kLoop) ? 2 : kNBuf;
    static_assert(!kLoop || NBUF == kNBuf, "the persistent form rotates kNBuf sets across tiles");
    WChunk w[NBUF];
    load_w(w[0], A, 0);
    sc.before_act(cur);
    finish_addr(A, cur);
    load_a(A, 0);
#pragma unroll
    for (int c = 1; c < NBUF - 2; ++c) load_w(w[c], A, min(c, nc - 1));
    store_a(0);
    load_a(A, min(1, nc - 1));
    load_w(w[NBUF - 2], A, min(NBUF - 2, nc - 1));
    if constexpr (!kTiled) store_w(w[0]);
    lds_barrier();  // chunk 0 staged, scale table built

    for (;;) {
        // the next tile's addressing (kLoop only; otherwise requests past the last chunk repeat
        // it).  Its row_src loads are issued now and consumed at step 2, when every older load in
        // flight is one this tile needs by then anyway; its first request comes at step nc - 3.
        Tile nxt{};
        Addr B = A;
        if (kLoop) {
            nxt = sc.next();
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

        // Chunk c computes from activation buffer c % 2 and from its weights: this wave's LDS slot
        // (row-major), or register set c % NBUF (tiled).  Then (row-major only) it stages the
        // weights of chunk c + 1 into the slot (this wave read it just now; a wave's LDS accesses
        // stay in order), stages the activations of chunk c + 1 into the other buffer (last read
        // in chunk c - 1, before the previous barrier), loads the activations of chunk c + 2 and
        // the weights of chunk c + NBUF - 1 (into the set of chunk c - 1).  Whole groups of NBUF
        // steps: a step past the last chunk (single-tile form with K / kKC not a multiple of
        // NBUF) skips only its
        // compute (which issues no memory loads), so every path through the loop issues the same
        // loads and the compiler's waits at the loop head see the regular pattern.
        for (int c0 = 0; c0 < nc; c0 += NBUF) {
#pragma unroll
            for (int sidx = 0; sidx < NBUF; ++sidx) {
                const int c = c0 + sidx;
                if (kLoop && c == 2 && go_on) finish_addr(B, nxt);  // before request nc - 2 (nc >= 4)
                if (kSplit == 2 && c == nc / 2) {
#pragma unroll
                    for (int tb = 0; tb < NTB; ++tb) {
                        acc_lo[tb] = acc[tb];
#pragma unroll
                        for (int v = 0; v < 16; ++v) acc[tb][v] = 0.f;
                    }
                }
                if (c < nc) compute(c & 1, w[sidx]);
                if constexpr (!kTiled) {
                    // the staging slot is rewritten below: keep these writes after the reads above
                    // (the lanes of the wave read each other's bytes; its LDS accesses run in order)
                    asm volatile("" ::: "memory");
                    store_w(w[(sidx + 1) % NBUF]);
                }
                store_a((c + 1) & 1);
                const int ca = req(c + 2), cw = req(c + NBUF - 1);
                if (go_on && c + 2 == nc) sc.before_act(nxt);  // the next tile's first activation load
                load_a(c + 2 < nc ? A : B, ca);
                load_w(w[(sidx + NBUF - 1) % NBUF], c + NBUF - 1 < nc ? A : B, cw);
                lds_barrier();
            }
        }
        // every wave has passed the last chunk's barrier; buffer nc % 2 holds the next tile's
        // first chunk (kLoop: nc is even), so the exchange uses the other one
        if (kSplit == 2)
#pragma unroll
            for (int tb = 0; tb < NTB; ++tb)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[tb][v] = acc_lo[tb][v] + acc[tb][v];
        epilogue(cur, (float *)(act + ((nc + 1) & 1) * kActBuf));
        sc.after_tile(cur);
        if (!go_on) break;
        lds_barrier();  // the exchange buffer is read before chunk 1 of the next tile is staged in it
        cur = nxt;
        A = B;
    }
}

}  // namespace

#define TPG_W4A8_LDS                                                                                   \
    __shared__ __attribute__((aligned(1024))) unsigned char act[2 * kActBuf];                          \
    __shared__ u32x2 lut[256];                                                                         \
    __shared__ float xsl[2 * w4::kMaxRows * 2]; /* activation scales of the staged chunks [buf][row][block] */ \
    __shared__ __attribute__((aligned(16))) unsigned char wlds[4 * kWSlot]; /* one slot per wave */ \
    if constexpr (!kMX) lut[threadIdx.x] = scaled_e2m1_table(threadIdx.x); /* read after a tile's first barrier */


template <bool kSwiGLU, bool kMX, bool kTiled>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_w4a8_kernel(W4Args g, const int32_t *__restrict__ offsets,
                                                                     const int32_t *__restrict__ tiles,
                                                                     const int32_t *__restrict__ n_tiles) {
    TPG_W4A8_LDS
    StaticSched sc{g.split == 1 ? (int)(blockIdx.x >> 1) : (int)blockIdx.x, 0, g.N / kBN, n_tiles[0], offsets, tiles,
                   true};
    const Tile t = sc.first();
    if (!t.valid) return;
    if (kSwiGLU && g.split == 1)  // decode sizes: rows of at most 32
        w4a8_tiles<kSwiGLU, kMX, 1, false, StaticSched, kSwiGLU ? 1 : 0, kTiled>(g, sc, act, xsl, wlds, lut);
    else if (t.rows > 2 * 32)
        w4a8_tiles<kSwiGLU, kMX, 3, false, StaticSched, 0, kTiled>(g, sc, act, xsl, wlds, lut);
    else if (t.rows > 32)
        w4a8_tiles<kSwiGLU, kMX, 2, false, StaticSched, 0, kTiled>(g, sc, act, xsl, wlds, lut);
    else
        w4a8_tiles<kSwiGLU, kMX, 1, false, StaticSched, 0, kTiled>(g, sc, act, xsl, wlds, lut);
}

// persistent (at most 32 rows per tile): workgroup b takes virtual blocks b, b + gridDim.x, ...
template <bool kSwiGLU, bool kMX, bool kTiled>
__global__ __launch_bounds__(kThreads, 2) void grouped_gemm_w4a8_persistent_kernel(
    W4Args g, const int32_t *__restrict__ offsets, const int32_t *__restrict__ tiles,
    const int32_t *__restrict__ n_tiles) {
    TPG_W4A8_LDS
    StaticSched sc{(int)blockIdx.x, (int)gridDim.x, g.N / kBN, n_tiles[0], offsets, tiles, true};
    w4a8_tiles<kSwiGLU, kMX, 1, true, StaticSched, 0, kTiled>(g, sc, act, xsl, wlds, lut);
}

// ---------------------------------------------------------------- single-launch small-token forward
//
// The whole W4A8 forward in one persistent launch for up to 256 tokens and 2048 slots, as the
// FlashInfer pull request "[SM90] Add W4A8 MegaMoE support" runs dispatch, both FFN GEMMs, the
// SwiGLU and the top-k reduction in one persistent kernel through 256 tokens per rank (its
// opening description and Usage section).  The work and the arithmetic are those of the
// step-by-step kernels (the same routing and table results, the same GEMM tile pipeline, the
// same re-quantisation and combine arithmetic), so the output is bitwise the same.
//
//   workgroup 0   routes the tokens, builds offsets, row_src, slot_row and the tile list, zeroes
//                 the counters below, then publishes a "go" word; the others wait for it
//   items         GEMM1 tiles, then GEMM2 tiles.  Workgroup b starts with item b; later items
//                 come from one counter (each claimed while the previous item runs)
//   GEMM1 tile    writes its 64 h columns (fp32); of the two tiles that make one 128-column block
//                 of an m-tile, the second to finish re-quantises the block to fp8 and counts it
//                 in the m-tile's ready counter
//   GEMM2 tile    streams its first weight chunks, then waits until its m-tile has all I/128
//                 blocks (no more waiting once every block of every m-tile is done)
//   combine       once every workgroup is past its GEMM tiles, workgroup b combines tokens
//                 b, b + grid, ...; the last workgroup out resets the go word
// No GEMM item waits on an item claimed after it (a GEMM2 tile waits only on GEMM1 tiles, all
// handed out earlier to running workgroups, which never wait), so the GEMM phase completes on
// whatever share of the device the grid gets; every wait is bounded, and a wait that gives up
// sets the error word.  Hand-offs between workgroups: every wave waits for its stores, a
// barrier, one agent-scope release fence (a write-back of the XCD's L2) and a counter update by
// one thread; the consumer polls the counter and takes an agent-scope acquire fence (an
// invalidation of its L1 and L2) before the workgroup reads.

constexpr uint64_t kGoWord = 0x7ff47ff47ff47ff4ull;  // a pattern the workspace holds nowhere else
constexpr int kSpinLimit = 1 << 21;                   // polls (each after a short sleep) before giving up

struct FusedArgs {
    const float *logits;
    const uint8_t *slot_drop;
    int T, E, k;
    int32_t *topk_idx, *offsets, *row_src, *slot_row, *tiles, *n_tiles;
    float *topk_w;
    FusedSync *sync;
    uint32_t *rq_cnt, *mt_ready;
    W4Args g1, g2;      // GEMM1 (x through row_src -> h32), GEMM2 (h8 -> y)
    float *h32;
    uint8_t *h8;
    float *hs;
    uint16_t *y, *out;
    int H, I;
};

__device__ __forceinline__ void fence_release() { __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent"); }
__device__ __forceinline__ void fence_acquire() { __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent"); }
__device__ __forceinline__ uint32_t atomic_add(uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t atomic_get(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every store this wave issued has completed (reached the XCD's L2)
__device__ __forceinline__ void stores_done() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// thread 0: poll until *p >= want (bounded), then the acquire fence for the workgroup (it
// invalidates the caches its waves share); false if the wait gave up
__device__ __forceinline__ bool poll_at_least(const FusedArgs &f, const uint32_t *p, uint32_t want) {
    int n = 0;
    while (atomic_get(p) < want) {
        if (++n > kSpinLimit) {
            __hip_atomic_fetch_or(&f.sync->err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return false;
        }
        __builtin_amdgcn_s_sleep(16);
    }
    fence_acquire();
    return true;
}

// The stores of every wave reach the XCD's L2, then thread 0's release fence writes the L2's
// dirty lines back (one write-back for the whole workgroup) and it adds one to *p.  Returns the
// counter's previous value to every thread (through word, a workgroup-shared int, which every
// thread has read before the call returns); the thread that reads acquire_at takes the acquire
// fence for the workgroup.
__device__ __forceinline__ uint32_t publish_and_count(uint32_t *p, int *word, uint32_t acquire_at = ~0u,
                                                      uint32_t *also = nullptr) {
    stores_done();
    lds_barrier();
    if (threadIdx.x == 0) {
        fence_release();
        const uint32_t old = atomic_add(p, 1u);
        if (also) atomic_add(also, 1u);
        if (old == acquire_at) fence_acquire();
        *word = (int)old;
    }
    lds_barrier();
    const uint32_t v = (uint32_t)*word;
    lds_barrier();
    return v;
}

// Routing of token t by one thread: the same selection (the largest key, the lower id on
// ties) and the same fp32 arithmetic in the same order as route_row, so the same ids and
// weights.  NE >= E keys in registers; exs: per-slot scratch for the unnormalised weights.
template <int NE>
__device__ __forceinline__ void route_thread(const float *__restrict__ logits, const uint8_t *__restrict__ slot_drop,
                                             int t, int E, int k, int32_t *__restrict__ topk_idx,
                                             float *__restrict__ topk_w, int32_t *ids, float *exs) {
    using namespace route_detail;
    const float *l = logits + (int64_t)t * E;
    uint32_t key[NE];
#pragma unroll
    for (int e = 0; e < NE; ++e) key[e] = e < E ? logit_key(l[e]) : 0u;
    float lmax = 0.0f, z = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t bk = 0u;
        int be = 0;
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (key[e] > bk) {
                bk = key[e];
                be = e;
            }
#pragma unroll
        for (int e = 0; e < NE; ++e)
            if (e == be) key[e] = 0u;
        const float lj = key_logit(bk);
        if (j == 0) lmax = lj;
        const float ex = expf(lj - lmax);
        z += ex;
        ids[j] = be;
        exs[j] = ex;
    }
    for (int j = 0; j < k; ++j) {
        const int64_t s = (int64_t)t * k + j;
        const bool dropped = slot_drop != nullptr && slot_drop[s] != 0;
        const int id = dropped ? -1 : ids[j];
        topk_idx[s] = id;
        topk_w[s] = exs[j] / z;
        ids[j] = id;
    }
}

// Routing, tables and tile list of up to 2048 slots in workgroup 0 (256 threads): the same
// results as route_topk + the table kernels.  LDS: sid [2048] ids, exs [2048] scratch, cnt
// [4][256], off [257], run [256], ws8 [8].
__device__ void fused_front_end(const FusedArgs &f, int32_t *sid, float *exs, int (*cnt)[256], int *off, int *run,
                                int *ws8, int *n_mt_out) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int T = f.T, E = f.E, k = f.k, S = T * k;
    auto valid = [E](int32_t x) { return ((unsigned)x < (unsigned)E) ? x : -1; };
    if (T > 16 && E <= 64) {
        // one thread per token (one pass for up to 256 tokens)
        for (int t = tid; t < T; t += kThreads) {
            if (E <= 32)
                route_thread<32>(f.logits, f.slot_drop, t, E, k, f.topk_idx, f.topk_w, sid + t * k, exs + t * k);
            else
                route_thread<64>(f.logits, f.slot_drop, t, E, k, f.topk_idx, f.topk_w, sid + t * k, exs + t * k);
        }
    } else {
        // one 16-lane row per token, four tokens per wave, 16 per pass
        for (int t0 = w * 4; t0 < T; t0 += 16) {
            const int t = t0 + (lane >> 4);
            route_token16(f.logits, f.slot_drop, t < T ? t : T - 1, t < T, E, k, lane & 15, f.topk_idx, f.topk_w,
                          sid + t * k);
        }
    }
    run[tid] = 0;
    __syncthreads();
    for (int s = tid; s < S; s += kThreads) {
        const int x = valid(sid[s]);
        if (x >= 0) atomicAdd(&run[x], 1);
    }
    __syncthreads();
    const int tot = tid < E ? run[tid] : 0;
    int incl = tot, unused = 0, R, unused_total;
    block_incl_sum256(incl, unused, ws8, &R, &unused_total);
    if (tid < E) {
        off[tid] = incl - tot;
        f.offsets[tid] = incl - tot;
        run[tid] = 0;  // rows of expert tid placed by earlier passes
    }
    if (tid == 0) {
        off[E] = R;
        f.offsets[E] = R;
    }
    // stable rank, 256 slots per pass: a slot's rank among equal ids of lower lanes of its wave
    // from 9 ballots, its wave's base from the lower waves' counts and the earlier passes
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int p0 = 0; p0 < S; p0 += kThreads) {
        const int s = p0 + tid;
        const int x = s < S ? valid(sid[s]) : -1;
        const unsigned key = (unsigned)(x + 1);
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = (key >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & lt);
        for (int i = tid; i < 4 * 256; i += kThreads) (&cnt[0][0])[i] = 0;
        __syncthreads();
        if (x >= 0 && rank == 0) cnt[w][x] = __popcll(peers);
        __syncthreads();
        if (tid < E) {
            int b = run[tid];
            for (int ww = 0; ww < 4; ++ww) {
                const int v = cnt[ww][tid];
                cnt[ww][tid] = b;
                b += v;
            }
            run[tid] = b;
        }
        __syncthreads();
        if (s < S) {
            const int r = x >= 0 ? off[x] + cnt[w][x] + rank : -1;
            f.slot_row[s] = r;
            if (r >= 0) f.row_src[r] = s;
        }
        __syncthreads();
    }
    *n_mt_out = build_tile_list(off, E, kBM, 1, f.tiles, f.n_tiles, ws8);
}

// Items of the fused forward: [0, n1) GEMM1 tiles, [n1, n1 + n2) GEMM2 tiles.
struct FusedState {
    int pending;     // thread 0: the item claimed ahead
    int item;        // the current item (uniform)
    bool have;       // item is claimed and not yet started
    int ready_mt;    // GEMM2: the last m-tile seen complete
    bool all_ready;  // GEMM2: every block of every m-tile seen complete
};

template <bool kG1>
struct FusedSched {
    static constexpr bool kRowDst = false;  // the single-launch forward keeps the expert order
    const FusedArgs &f;
    FusedState &st;
    int *word;  // workgroup-shared int
    int n_mt, n1, n2;
    // the item claimed ahead becomes current (to every thread); thread 0 claims the next one
    __device__ int take() {
        if (threadIdx.x == 0) {
            *word = st.pending;
            st.pending = (int)atomic_add(&f.sync->next_item, 1u);
        }
        lds_barrier();
        const int it = *word;
        lds_barrier();  // every thread has read the word before it can be written again
        return it;
    }
    __device__ Tile decode(int it) {
        if (kG1 ? it >= n1 : (it < n1 || it >= n1 + n2)) return Tile{};
        return kG1 ? w4::tile_of(it, 2 * f.I / kBN, f.offsets, f.tiles, n_mt, false)
                   : w4::tile_of(it - n1, f.H / kBN, f.offsets, f.tiles, n_mt, false);
    }
    __device__ Tile first() {
        if (!st.have) {
            // workgroup b starts with item b; the counter starts at the grid size
            st.item = (int)blockIdx.x;
            if (threadIdx.x == 0) st.pending = (int)atomic_add(&f.sync->next_item, 1u);
        }
        st.have = false;
        const Tile t = decode(st.item);
        if (!t.valid) st.have = true;  // handed to the next phase
        return t;
    }
    __device__ Tile next() {
        st.item = take();
        const Tile t = decode(st.item);
        if (!t.valid) st.have = true;
        return t;
    }
    __device__ void before_act(const Tile &t) {
        if (kG1 || st.all_ready || t.mt == st.ready_mt) return;
        if (threadIdx.x == 0) {
            const uint32_t n_cb = f.I / 128;
            const bool ok = poll_at_least(f, f.mt_ready + t.mt * kSyncLine, n_cb);
            *word = ok && atomic_get(&f.sync->rq_total) == (uint32_t)n_mt * n_cb;
        }
        lds_barrier();
        st.all_ready = *word != 0;
        lds_barrier();
        st.ready_mt = t.mt;
    }
    __device__ void after_tile(const Tile &t) {
        if (!kG1) return;  // GEMM2 outputs are published once, after the workgroup's last tile
        const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
        // two GEMM1 tiles (n-tiles 2 cb, 2 cb + 1) make the 128-column block cb of h
        const int cb = t.nt >> 1, n_cb = f.I / 128;
        if (publish_and_count(f.rq_cnt + (t.mt * n_cb + cb) * kSyncLine, word, 1u) != 1) return;
        // the same arithmetic as requant_fp8_kernel, one wave per (row, 128 columns): rows
        // wave, wave + 4, ... of the tile, all loads first
        f32x2 v[kBM / 4];
#pragma unroll
        for (int i = 0; i < kBM / 4; ++i) {
            const int r = wave + 4 * i;
            if (r < t.rows) v[i] = *(const f32x2 *)(f.h32 + (int64_t)(t.row_begin + r) * f.I + cb * 128 + 2 * lane);
        }
#pragma unroll
        for (int i = 0; i < kBM / 4; ++i) {
            const int r = wave + 4 * i;
            if (r >= t.rows) break;
            const int64_t row = t.row_begin + r;
            float m = fmaxf(fabsf(v[i].x), fabsf(v[i].y));
#pragma unroll
            for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
            float s = m / 448.0f;
            if (s == 0.0f) s = 1.0f;
            const uint32_t q = to_fp8x2<false>(v[i].x / s, v[i].y / s, 0u);
            *(uint16_t *)(f.h8 + row * f.I + cb * 128 + 2 * lane) = (uint16_t)(q & 0xffffu);
            if (lane == 0) f.hs[row * n_cb + cb] = s;
        }
        publish_and_count(f.mt_ready + t.mt * kSyncLine, word, ~0u, &f.sync->rq_total);
    }
};

// out[tok] for tokens blockIdx.x, blockIdx.x + gridDim.x, ...: the arithmetic of combine_kernel
// (an fp32 chain over the slots in ascending j, one rounding); the token's rows and weights go
// to LDS first, then every thread loads its chunk of up to 8 slot rows at once.
__device__ void fused_combine(const FusedArgs &f, int *rows_s, float *w_s) {
    const int tid = threadIdx.x, k = f.k, nch = f.H / 8;
    for (int tok = blockIdx.x; tok < f.T; tok += gridDim.x) {
        for (int j = tid; j < k; j += kThreads) {
            rows_s[j] = f.slot_row[(int64_t)tok * k + j];
            w_s[j] = f.topk_w[(int64_t)tok * k + j];
        }
        __syncthreads();
        for (int c = tid; c < nch; c += kThreads) {
            float acc[8] = {};
            for (int j0 = 0; j0 < k; j0 += 8) {
                uint4 v[8];
#pragma unroll
                for (int q = 0; q < 8; ++q) {
                    const int r = j0 + q < k ? rows_s[j0 + q] : -1;
                    v[q] = r >= 0 ? *(const uint4 *)(f.y + (int64_t)r * f.H + c * 8) : make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int q = 0; q < 8; ++q)
                    if (j0 + q < k && rows_s[j0 + q] >= 0) combine_fma8(acc, w_s[j0 + q], v[q]);
            }
            *(uint4 *)(f.out + (int64_t)tok * f.H + c * 8) = combine_pack8(acc);
        }
        __syncthreads();
    }
}

template <bool kMX, int NTB, bool kHalves = false, bool kTiled = false>
__global__ __launch_bounds__(kThreads, 2) void forward_small_w4a8_kernel(FusedArgs f) {
    TPG_W4A8_LDS
    __shared__ int word, n_mt_s;
    const int tid = threadIdx.x;
    FusedSync *sy = f.sync;
    if (blockIdx.x == 0) {
        // front end in the activation buffers (idle until the first GEMM tile)
        int32_t *sid = (int32_t *)act;                        // 2048 slots
        float *exs = (float *)(act + 8192);                    // 2048 slots
        int(*cnt)[256] = (int(*)[256])(act + 16384);          // [4][256]
        int *off = (int *)(act + 20480), *run = off + 260, *ws8 = run + 256;
        fused_front_end(f, sid, exs, cnt, off, run, ws8, &n_mt_s);
        const int n_mt = n_mt_s, n_cb = f.I / 128;
        for (int i = tid; i < n_mt * n_cb; i += kThreads) f.rq_cnt[i * kSyncLine] = 0;
        for (int i = tid; i < n_mt; i += kThreads) f.mt_ready[i * kSyncLine] = 0;
        if (tid == 0) {
            sy->next_item = gridDim.x;  // workgroup b starts with item b
            sy->done = 0;
            sy->err = 0;
            sy->rq_total = 0;
            sy->gemm_done = 0;
        }
        stores_done();
        lds_barrier();
        if (tid == 0) {
            fence_release();
            __hip_atomic_store(&sy->go, kGoWord, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    } else {
        if (tid == 0) {
            int n = 0;
            bool ok = true;
            while (__hip_atomic_load(&sy->go, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != kGoWord) {
                if (++n > kSpinLimit) {
                    ok = false;
                    break;
                }
                __builtin_amdgcn_s_sleep(16);
            }
            fence_acquire();
            word = ok;
            n_mt_s = f.n_tiles[0];
        }
        lds_barrier();
        if (!word) {  // workgroup 0 never published (it cannot have run): do nothing, flag it
            if (tid == 0) __hip_atomic_fetch_or(&sy->err, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
    }
    const int n_mt = n_mt_s;
    FusedState st{0, 0, false, -1, false};
    const int n1 = n_mt * (2 * f.I / kBN), n2 = n_mt * (f.H / kBN);
    {
        FusedSched<true> sc{f, st, &word, n_mt, n1, n2};
        w4a8_tiles<true, kMX, NTB, true, FusedSched<true>, kHalves ? 2 : 0, kTiled>(f.g1, sc, act, xsl, wlds, lut);
    }
    {
        FusedSched<false> sc{f, st, &word, n_mt, n1, n2};
        w4a8_tiles<false, kMX, NTB, true, FusedSched<false>, 0, kTiled>(f.g2, sc, act, xsl, wlds, lut);
    }
    // every workgroup's GEMM2 rows are written before any combine reads them
    publish_and_count(&sy->gemm_done, &word);
    if (tid == 0) poll_at_least(f, &sy->gemm_done, gridDim.x);
    lds_barrier();
    fused_combine(f, (int *)act, (float *)(act + 4096));
    // the last workgroup out resets the go word for the next forward on this workspace
    lds_barrier();
    if (tid == 0 && atomic_add(&sy->done, 1u) == gridDim.x - 1)
        __hip_atomic_store(&sy->go, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

#undef TPG_W4A8_LDS

// h fp32 [S][I] -> h8 e4m3 [S][I] + hs fp32 [S][I/128] for the live rows.  Item i = (row, 128
// columns) starts at float 128 i of h (a row holds I / 128 items).  A half-wave takes one item,
// four columns per lane, and a wave kReqPairs pairs of adjacent items, every load issued before
// any arithmetic; s = amax / 448 (1 if that is 0), q = e4m3(h / s), decided in fp32.  h is read
// once, non-temporal.
constexpr int kReqPairs = 2;
__global__ __launch_bounds__(256) void requant_fp8_kernel(const float *__restrict__ h, const int32_t *__restrict__ offsets,
                                                          int E, int I, uint8_t *__restrict__ h8,
                                                          float *__restrict__ hs) {
    const int lane = threadIdx.x & 63, c = 4 * (lane & 31);
    const int64_t live = (int64_t)offsets[E] * (I / 128);  // items of the live rows
    const int64_t first = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * (2 * kReqPairs) + (lane >> 5);
    f32x4 v[kReqPairs];
#pragma unroll
    for (int u = 0; u < kReqPairs; ++u) {
        const int64_t it = first + 2 * u;
        v[u] = it < live ? __builtin_nontemporal_load((const f32x4 *)(h + it * 128 + c)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kReqPairs; ++u) {
        const int64_t it = first + 2 * u;
        // the reduction stays within each half-wave (both halves run it, live or not)
        float m = fmaxf(fmaxf(fabsf(v[u].x), fabsf(v[u].y)), fmaxf(fabsf(v[u].z), fabsf(v[u].w)));
#pragma unroll
        for (int off = 16; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
        float s = m / 448.0f;
        if (s == 0.0f) s = 1.0f;
        const uint32_t q = to_fp8x2<true>(v[u].z / s, v[u].w / s, to_fp8x2<false>(v[u].x / s, v[u].y / s, 0u));
        if (it < live) {
            *(uint32_t *)(h8 + it * 128 + c) = q;
            if ((lane & 31) == 0) hs[it] = s;
        }
    }
}

// GEMM1 split in two K halves: h = silu(g) * u from the halves' partial sums
// (part [2 halves][gate, up][S][I]; g = gs_e * (gate half 0 + gate half 1), u likewise, clamped,
// then the same SwiGLU expression as the GEMM1 epilogue), then re-quantised as by
// requant_fp8_kernel.  One wave per (row, 128 columns).
__global__ __launch_bounds__(256) void requant_swiglu_fp8_kernel(const float *__restrict__ part, int64_t stride,
                                                                 const int32_t *__restrict__ offsets, int E, int I,
                                                                 const float *__restrict__ gs1, float clamp,
                                                                 uint8_t *__restrict__ h8, float *__restrict__ hs) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nb = I / 128;
    const int64_t row = item / nb;
    const int b = (int)(item % nb);
    if (row >= offsets[E]) return;
    int lo = 0, hi = E - 1;  // the expert of the row: the last e with offsets[e] <= row
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (offsets[mid] <= row) lo = mid;
        else hi = mid - 1;
    }
    const float gs = gs1[lo];
    const int64_t o = row * I + b * 128 + 2 * lane;
    const f32x2 g0 = *(const f32x2 *)(part + o), u0 = *(const f32x2 *)(part + stride + o);
    const f32x2 g1 = *(const f32x2 *)(part + 2 * stride + o), u1 = *(const f32x2 *)(part + 3 * stride + o);
    float h[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        float gv = gs * (g0[j] + g1[j]);
        float uv = gs * (u0[j] + u1[j]);
        if (clamp > 0.f) {
            gv = fminf(fmaxf(gv, -clamp), clamp);
            uv = fminf(fmaxf(uv, -clamp), clamp);
        }
        h[j] = gv / (1.0f + expf(-gv)) * uv;
    }
    float m = fmaxf(fabsf(h[0]), fabsf(h[1]));
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    float sc = m / 448.0f;
    if (sc == 0.0f) sc = 1.0f;
    const uint32_t q = to_fp8x2<false>(h[0] / sc, h[1] / sc, 0u);
    *(uint16_t *)(h8 + o) = (uint16_t)(q & 0xffffu);
    if (lane == 0) hs[row * nb + b] = sc;
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
// kernel would have to fix the token-block count for every tile (most tiles then hold under 32
// rows at T = 64) and measured slower; there and for other K, one tile per workgroup (and
// at decode sizes, two per tile, see w4a8_split_gemm1).
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

template <bool kSwiGLU, bool kMX, bool kTiled>
void launch_w4a8_gemm_as(const W4Launch &l, const W4Args &g, const int32_t *offsets, const int32_t *tiles,
                         const int32_t *n_tiles, hipStream_t s) {
    if (l.persistent)
        hipLaunchKernelGGL((grouped_gemm_w4a8_persistent_kernel<kSwiGLU, kMX, kTiled>), dim3(l.grid), dim3(kThreads), 0,
                           s, g, offsets, tiles, n_tiles);
    else
        hipLaunchKernelGGL((grouped_gemm_w4a8_kernel<kSwiGLU, kMX, kTiled>), dim3(l.grid), dim3(kThreads), 0, s, g,
                           offsets, tiles, n_tiles);
}
// tiled: weights in MOE_W4_LAYOUT_TILED (operand order; NVFP4 codes in its nibble order)
template <bool kSwiGLU>
void launch_w4a8_gemm(bool mx, bool tiled, const W4Launch &l, const W4Args &g, const int32_t *offsets,
                      const int32_t *tiles, const int32_t *n_tiles, hipStream_t s) {
    if (mx && tiled)
        launch_w4a8_gemm_as<kSwiGLU, true, true>(l, g, offsets, tiles, n_tiles, s);
    else if (mx)
        launch_w4a8_gemm_as<kSwiGLU, true, false>(l, g, offsets, tiles, n_tiles, s);
    else if (tiled)
        launch_w4a8_gemm_as<kSwiGLU, false, true>(l, g, offsets, tiles, n_tiles, s);
    else
        launch_w4a8_gemm_as<kSwiGLU, false, false>(l, g, offsets, tiles, n_tiles, s);
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
                                   uint8_t *h8, float *hs, uint16_t *y_perm, const int32_t *row_dst,
                                   hipStream_t s) {
    const int H = p.H, I = p.I;
    if (row_src && !gather_fits_fp8(p.T, H)) return hipErrorInvalidValue;
    const int S = (int)n_slots(p);
    const bool mx = p.prec == MOE_PREC_W4A8_MX;
    const bool tiled = w.w4_layout == MOE_W4_LAYOUT_TILED;
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
    const bool split = w4a8_split_gemm1(p);
    if (split) {  // two workgroups per tile, one per K half, one tile each (rows of at most 32)
        g1.split = 1;
        g1.part_stride = (int64_t)S * I;
        launch_w4a8_gemm<true>(mx, tiled, W4Launch{2 * max_tiles * (2 * I / kBN), false}, g1, offsets, tiles, n_tiles,
                               s);
    } else {
        launch_w4a8_gemm<true>(mx, tiled, l1, g1, offsets, tiles, n_tiles, s);
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const int64_t items = n_slots(p) * (I / 128);
    if (split)
        hipLaunchKernelGGL(requant_swiglu_fp8_kernel, dim3((items + 3) / 4), dim3(256), 0, s, h32, (int64_t)S * I,
                           offsets, p.E, I, w.w1_gscale, p.swiglu_clamp, h8, hs);
    else
        hipLaunchKernelGGL(requant_fp8_kernel, dim3((items + 8 * kReqPairs - 1) / (8 * kReqPairs)), dim3(256), 0, s,
                           h32, offsets, p.E, I, h8, hs);
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
    g2.row_dst = row_dst;
    set_layout(g2, I, mx, w.w4_layout);
    launch_w4a8_gemm<false>(mx, tiled, l2, g2, offsets, tiles, n_tiles, s);
    return hipGetLastError();
}

bool forward_small_w4a8_fits(const moe_problem &p) {
    const int64_t S = n_slots(p), lim = 0x7FFFFFFF;
    return (p.prec == MOE_PREC_W4A8 || p.prec == MOE_PREC_W4A8_MX) && p.T <= 256 && S <= 2048 &&
           p.H % (kKC * kNBuf) == 0 && p.I % (kKC * kNBuf) == 0 && (int64_t)p.E * 2 * p.I * (p.H / 2) <= lim &&
           (int64_t)p.E * p.H * (p.I / 2) <= lim && (int64_t)p.T * p.H <= lim && S * p.I <= lim;
}

namespace {
// one kernel form: its grid is every workgroup resident at once (two per CU: the kernel's LDS and
// register budget); the kernel does not depend on it, but idle waits are shortest then
template <bool kMX, bool kTiled>
hipError_t launch_forward_small_as(const FusedArgs &f, bool halves, bool one_block, int n_cu, hipStream_t s) {
    const void *fn = halves      ? (const void *)forward_small_w4a8_kernel<kMX, 1, true, kTiled>
                     : one_block ? (const void *)forward_small_w4a8_kernel<kMX, 1, false, kTiled>
                                 : (const void *)forward_small_w4a8_kernel<kMX, 2, false, kTiled>;
    int per_cu = 0;
    const hipError_t err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0);
    if (err != hipSuccess) return err;
    const int grid = std::max(1, std::min(per_cu, 2) * n_cu);
    if (halves)
        hipLaunchKernelGGL((forward_small_w4a8_kernel<kMX, 1, true, kTiled>), dim3(grid), dim3(kThreads), 0, s, f);
    else if (one_block)
        hipLaunchKernelGGL((forward_small_w4a8_kernel<kMX, 1, false, kTiled>), dim3(grid), dim3(kThreads), 0, s, f);
    else
        hipLaunchKernelGGL((forward_small_w4a8_kernel<kMX, 2, false, kTiled>), dim3(grid), dim3(kThreads), 0, s, f);
    return hipGetLastError();
}
}  // namespace

hipError_t launch_forward_small_w4a8(const float *logits, const uint8_t *slot_drop, const uint8_t *x,
                                     const float *x_scale, const moe_weights &w, const moe_problem &p,
                                     int64_t max_tiles, FusedSync *sync, int32_t *topk_idx, float *topk_w,
                                     int32_t *offsets, int32_t *row_src, int32_t *slot_row, int32_t *tiles,
                                     int32_t *n_tiles, float *h32, uint8_t *h8, float *hs, uint16_t *y,
                                     uint16_t *out, hipStream_t s) {
    if (!forward_small_w4a8_fits(p)) return hipErrorInvalidValue;
    const bool mx = p.prec == MOE_PREC_W4A8_MX;
    const bool tiled = w.w4_layout == MOE_W4_LAYOUT_TILED;
    const int S = (int)n_slots(p);
    FusedArgs f{};
    f.logits = logits;
    f.slot_drop = slot_drop;
    f.T = p.T;
    f.E = p.E;
    f.k = p.k;
    f.topk_idx = topk_idx;
    f.offsets = offsets;
    f.row_src = row_src;
    f.slot_row = slot_row;
    f.tiles = tiles;
    f.n_tiles = n_tiles;
    f.topk_w = topk_w;
    f.sync = sync;
    f.rq_cnt = (uint32_t *)(sync + 1);  // counters kSyncLine words apart
    f.mt_ready = f.rq_cnt + max_tiles * (p.I / 128) * kSyncLine;
    f.h32 = h32;
    f.h8 = h8;
    f.hs = hs;
    f.y = y;
    f.out = out;
    f.H = p.H;
    f.I = p.I;
    W4Args &g1 = f.g1;
    // where the multi-launch GEMM1 splits K in two workgroups, sum the halves apart here too, so that
    // the output stays bitwise the default forward's
    g1.split = w4a8_split_gemm1(p) ? 2 : 0;
    g1.A8 = x;
    g1.As = x_scale;
    g1.row_src = row_src;
    g1.gather_k = p.k;
    g1.a_rows = p.T;
    g1.Wq = (const uint8_t *)w.w1;
    g1.Wbs = (const uint8_t *)w.w1_bscale;
    g1.Wgs = w.w1_gscale;
    g1.K = p.H;
    g1.N = 2 * p.I;
    g1.I = p.I;
    g1.il = p.glu_interleave;
    g1.E = p.E;
    g1.clamp = p.swiglu_clamp;
    g1.Hout = h32;
    set_layout(g1, p.H, mx, w.w4_layout);
    W4Args &g2 = f.g2;
    g2.A8 = h8;
    g2.As = hs;
    g2.gather_k = 1;
    g2.a_rows = S;
    g2.Wq = (const uint8_t *)w.w2;
    g2.Wbs = (const uint8_t *)w.w2_bscale;
    g2.Wgs = w.w2_gscale;
    g2.K = p.I;
    g2.N = p.H;
    g2.I = p.I;
    g2.E = p.E;
    g2.Yout = y;
    g2.ldy = p.H;
    set_layout(g2, p.I, mx, w.w4_layout);
    int dev = 0, n_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev);
    if (err != hipSuccess) return err;
    const bool one_block = p.T <= 32;  // every m-tile fits one 32-row token block
    const bool halves = g1.split == 2;  // T <= 32 only (one token block)
    if (mx && tiled) return launch_forward_small_as<true, true>(f, halves, one_block, n_cu, s);
    if (mx) return launch_forward_small_as<true, false>(f, halves, one_block, n_cu, s);
    if (tiled) return launch_forward_small_as<false, true>(f, halves, one_block, n_cu, s);
    return launch_forward_small_as<false, false>(f, halves, one_block, n_cu, s);
}

// NVFP4 codes in the tiled layout: the eight codes of a dword, packed low nibble first (byte i
// holds codes 2i and 2i + 1), regrouped so that byte i holds codes i and i + 4; the dequant then
// yields its fp8 bytes in K order without an interleave
__device__ __forceinline__ uint32_t split_nibbles(uint32_t x) {
    const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;  // codes 0, 2, 4, 6 / 1, 3, 5, 7
    const uint32_t first = __builtin_amdgcn_perm(hi, lo, 0x05010400u);   // codes 0, 1, 2, 3
    const uint32_t second = __builtin_amdgcn_perm(hi, lo, 0x07030602u);  // codes 4, 5, 6, 7
    return first | (second << 4);
}

// MOE_W4_LAYOUT_TILED from row-major codes: one thread per 16-byte granule g of row r's 256-wide
// piece c in a 32-row block; it goes to w4::tiled_code_pos(r, g) of that piece (NVFP4 codes with
// split_nibbles applied)
__global__ __launch_bounds__(256) void tile_codes_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                         int64_t units, int row_bytes, int n_pieces, bool split) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int per_row = row_bytes / 16;
    const int64_t row = u / per_row;  // expert * N + row of the matrix
    const int gi = (int)(u % per_row), c = gi / 8, g = gi % 8;
    const int64_t blk = row / 32;
    const int r = (int)(row % 32);
    uint4 v = *(const uint4 *)(src + u * 16);
    if (split) v = make_uint4(split_nibbles(v.x), split_nibbles(v.y), split_nibbles(v.z), split_nibbles(v.w));
    *(uint4 *)(dst + (blk * n_pieces + c) * 4096 + w4::tiled_code_pos(r, g)) = v;
}

// the block scales: one thread per row and piece (16 e4m3 bytes, or 8 e8m0 bytes); byte j goes to
// w4::tiled_scale_pos(r, j, mx) of the piece's scales
__global__ __launch_bounds__(256) void tile_scales_kernel(const uint8_t *__restrict__ src, uint8_t *__restrict__ dst,
                                                          int64_t units, int n_pieces, bool mx) {
    const int64_t u = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (u >= units) return;
    const int per = mx ? kKC / 32 : kKC / 16;  // scale bytes of one row's piece
    const int64_t row = u / n_pieces;
    const int c = (int)(u % n_pieces);
    const int64_t blk = row / 32;
    const int r = (int)(row % 32);
    uint8_t *d = dst + (blk * n_pieces + c) * 32 * per;
    for (int j = 0; j < per; ++j) d[w4::tiled_scale_pos(r, j, mx)] = src[u * per + j];
}

hipError_t launch_tile_weights(const uint8_t *codes, const uint8_t *bscale, uint8_t *codes_tiled,
                               uint8_t *bscale_tiled, int E, int N, int K, bool mx, hipStream_t s) {
    const int n_pieces = K / kKC;
    const int64_t rows = (int64_t)E * N;
    const int64_t cu = rows * (K / 2) / 16;  // 16-byte code granules
    const int64_t su = rows * n_pieces;      // row pieces of scales
    hipLaunchKernelGGL(tile_codes_kernel, dim3((cu + 255) / 256), dim3(256), 0, s, codes, codes_tiled, cu, K / 2,
                       n_pieces, !mx);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(tile_scales_kernel, dim3((su + 255) / 256), dim3(256), 0, s, bscale, bscale_tiled, su, n_pieces,
                       mx);
    return hipGetLastError();
}

}  // namespace tpg
