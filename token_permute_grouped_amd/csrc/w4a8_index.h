// Index arithmetic of the W4A8 expert GEMMs (gemm_w4a8.hip): the tile of a virtual block, the
// weight row a wave streams, the byte offsets of every global load, and the LDS offsets of every
// staging write and operand read.  Plain integer functions, compiled for the device by the
// kernels and for the host by a replay that checks every index against its buffer.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define TPG_HD __host__ __device__ __forceinline__
#else
#define TPG_HD inline
#endif

namespace tpg {
namespace w4 {

constexpr int kBM = 64;            // token rows per m-tile (2 blocks of 32)
constexpr int kMaxRows = 96;       // rows of an expert's last m-tile when a remainder of at most 32
                                   // rows joins it (3 blocks of 32)
constexpr int kBN = 128;           // weight rows per workgroup (4 waves x 32)
constexpr int kKC = 256;           // K per chunk
constexpr int kNBuf = 4;           // weight register sets (weights kNBuf - 1 chunks ahead)
constexpr int kThreads = 256;
constexpr int kActBuf = kMaxRows * kKC;  // bytes of one staged activation chunk (24 KB, two buffers)
// per-wave LDS staging of one chunk's weights in rows: 32 code rows of 128 bytes padded to 144
// (so that 16 consecutive rows read at one column hit 16 distinct bank groups), then 32 scale
// rows of 16 bytes
constexpr int kWRow = 144;
constexpr int kWScales = 32 * kWRow;
constexpr int kWSlot = kWScales + 32 * 16;  // 5120 bytes per chunk and wave

TPG_HD int imin(int a, int b) { return a < b ? a : b; }

// One work item of the block -> tile map: expert, first row, live rows, n-tile, and the m-tile's
// index in the tile list.
struct Tile {
    bool valid;
    int e, row_begin, rows, nt, mt;
};

// n-tiles of one expert m-tile that run side by side (see tile_of)
TPG_HD int tile_group(int nb_n) { return nb_n % 8 == 0 ? 8 : nb_n % 4 == 0 ? 4 : nb_n % 2 == 0 ? 2 : 1; }

// m-tiles of an expert with cnt rows: kBM-row tiles, or with `merge` a last partial tile of at
// most kBM / 2 rows joined to the tile before it (the tile list's by-expert merged form)
TPG_HD int m_tiles(int cnt, bool merge) {
    if (!merge) return (cnt + kBM - 1) / kBM;
    if (cnt <= 0) return 0;
    const int m = cnt / kBM + (cnt % kBM > kBM / 2 ? 1 : 0);
    return m > 0 ? m : 1;
}

// Virtual block v -> tile.  The tile list holds each expert's m-tiles together.  Expert e's
// blocks are [first * nb_n, (first + nm) * nb_n); they run in units of G n-tiles, the nm
// m-tiles of an n-tile G blocks apart: with G = 8 those land on one XCD (block b runs on XCD
// b mod 8, and the persistent grid's stride is a multiple of 8) at the same time, so the
// weights an expert's second m-tile streams are L2 hits.  An expert's last m-tile runs to the
// expert's last row (up to kMaxRows rows with `merge`).
TPG_HD Tile tile_of(int v, int nb_n, const int32_t *offsets, const int32_t *tiles, int n_mt, bool merge) {
    Tile t{};
    const int tq = v / nb_n;  // a tile of the expert this block works for
    t.valid = tq < n_mt;
    if (!t.valid) return t;
    t.e = tiles[2 * tq];
    const int first = tq - tiles[2 * tq + 1] / kBM;
    const int nm = m_tiles(offsets[t.e + 1] - offsets[t.e], merge);
    const int G = tile_group(nb_n);
    const int r = v - first * nb_n, unit = nm * G;
    t.mt = first + (r % unit) / G;
    t.nt = (r / unit) * G + (r % unit) % G;
    t.row_begin = offsets[t.e] + tiles[2 * t.mt + 1];
    t.rows = t.mt == first + nm - 1 ? offsets[t.e + 1] - t.row_begin : kBM;
    return t;
}

// Weight matrix row (within the expert) of row rl < 32 of wave `wave`'s block.  First GEMM
// (swiglu): waves 0, 1 hold the gate rows of h columns nt*64 + [0, 64), waves 2, 3 the matching
// up rows, in [gate | up] order (il = 0) or interleaved in blocks of il; second GEMM: rows
// nt*128 + 32*wave + rl.
TPG_HD int weight_row(bool swiglu, int nt, int wave, int rl, int I, int il) {
    if (swiglu) {
        const bool up = wave >= 2;
        const int c = nt * (kBN / 2) + (wave & 1) * 32 + rl;
        return il == 0 ? (up ? I + c : c) : (c / il) * 2 * il + (up ? il : 0) + c % il;
    }
    return nt * kBN + wave * 32 + rl;
}

// Weight loads of one 256-wide K chunk (chunk c adds c * step): lane l loads 16 code bytes of
// rows l/8 + 8i (i < 4) at byte 16 (l % 8), and the block scales of row l/2 (half l % 2), rows
// counted within the wave's 32-row block whose first row (within the descriptor) is blk.
TPG_HD uint32_t w_code_off(int blk, int K, int lane, int i, int w_pitch) {
    return (uint32_t)(blk * (K / 2) + ((lane >> 3) + 8 * i) * w_pitch + (lane & 7) * 16);
}
TPG_HD uint32_t w_scale_off(int blk, int K, int sb, int lane, int s_pitch) {
    return (uint32_t)(blk * (K / sb) + (lane >> 1) * s_pitch + (lane & 1) * (kKC / sb / 2));
}
// bytes one lane's scale load of a chunk reads (8 e4m3 scales, or 4 e8m0 ones)
TPG_HD int w_scale_bytes(int sb) { return kKC / sb / 2; }

// The tiled layout stores each 32-row block's 256-wide piece in the matrix instruction's operand
// order: lane l = 32 h + r (row r, half h) of 64-K step i = 2 q + t takes the 16 code bytes
// [64 q + 32 h + 16 t, +16) of its row, so the piece is four 1 KB runs, one per step, each in
// lane order; and the block scales of those codes in lane order (8 bytes per lane for NVFP4:
// row bytes 4 h .. 4 h + 3 and 8 + 4 h .. 8 + 4 h + 3; 4 for MXFP4: row bytes 2 h, 2 h + 1,
// 4 + 2 h, 5 + 2 h).  A wave then loads its operands with contiguous 16-byte (codes) and 8- or
// 4-byte (scales) loads per lane, with no transposition through LDS.
// Position within the piece of 16-byte code granule g of row r:
TPG_HD int tiled_code_pos(int r, int g) {
    const int q = g >> 2, h = (g >> 1) & 1, t = g & 1;
    return (2 * q + t) * 1024 + (32 * h + r) * 16;
}
// Position within the piece's scales of scale byte j of row r (16 per row for NVFP4, 8 for MXFP4)
TPG_HD int tiled_scale_pos(int r, int j, bool mx) {
    if (mx) {  // j = 4 q + 2 h + u
        const int q = j >> 2, h = (j >> 1) & 1, u = j & 1;
        return (32 * h + r) * 4 + 2 * q + u;
    }
    const int q = j >> 3, h = (j >> 2) & 1, u = j & 3;  // j = 8 q + 4 h + u
    return (32 * h + r) * 8 + 4 * q + u;
}
// Loads of one chunk from the tiled layout (chunk c adds c * 4096 for the codes, c * 32 times
// the row's scale bytes per piece for the scales): lane l's codes of step i, its scales
TPG_HD uint32_t w_code_off_tiled(int blk, int K, int lane, int i) {
    return (uint32_t)(blk * (K / 2) + i * 1024 + lane * 16);
}
TPG_HD uint32_t w_scale_off_tiled(int blk, int K, int sb, int lane) {
    return (uint32_t)(blk * (K / sb) + lane * w_scale_bytes(sb));
}

// Activation staging: thread tid stages granule tid % 16 (16 bytes) of tile rows tid / 16 + 16 i
// (i < 2 NTB), and thread tid < 32 NTB the chunk's two activation scales of tile row
// min(tid, kMaxRows - 1).  Row rr of the source (the token row when gathering, else the row within the
// descriptor): bytes rr * K + g * 16 (+ c * kKC for chunk c), scales rr * (K/128) * 4 (+ c * 8).
TPG_HD int act_row(int tid, int i) { return (tid >> 4) + 16 * i; }
TPG_HD int act_gran(int tid) { return tid & 15; }
TPG_HD int act_scale_row(int tid) { return imin(tid, kMaxRows - 1); }
TPG_HD uint32_t a_off(int rr, int K, int g) { return (uint32_t)(rr * K + g * 16); }
TPG_HD uint32_t s_off(int rr, int K) { return (uint32_t)(rr * (K / 128) * 4); }
// offset given to a row past the tile's live rows: beyond every descriptor, so it reads zero
constexpr uint32_t kDeadOff = 0x80000000u;

// LDS byte offsets.  Activation chunk buffer: granule g of staged row r (swizzled, 16 per row).
TPG_HD int aslot(int r, int g) { return g ^ (r & 15); }
TPG_HD int lds_act(int r, int g) { return r * kKC + aslot(r, g) * 16; }
// a wave's weight staging slot: code bytes of lane l's i-th load, its scale bytes
TPG_HD int lds_wcode(int lane, int i) { return ((lane >> 3) + 8 * i) * kWRow + (lane & 7) * 16; }
TPG_HD int lds_wscale(int lane, bool mx) { return kWScales + (lane >> 1) * 16 + (lane & 1) * (mx ? 4 : 8); }
// operand reads of lane l (row l % 32, half h = l / 32) in 64-K step (q, t): 16 code bytes at
// lds_wread(l) + 64 q + 16 t, scale bytes from lds_wsread(l) (4 bytes at + 8 q for NVFP4; the
// dword at - 4 h + 4 q for MXFP4)
TPG_HD int lds_wread(int lane) { return (lane & 31) * kWRow + (lane >> 5) * 32; }
TPG_HD int lds_wsread(int lane) { return kWScales + (lane & 31) * 16 + (lane >> 5) * 4; }
// activation scale of tile row r, block q of the chunk (float index into [2][kMaxRows][2])
TPG_HD int lds_xs(int buf, int r, int q) { return buf * (kMaxRows * 2) + r * 2 + q; }
// SwiGLU hand-over: accumulator v of token block tb of up wave 2 + wu, lane l (float index)
TPG_HD int lds_xch(int wu, int NTB, int tb, int v, int lane) { return ((wu * NTB + tb) * 16 + v) * 64 + lane; }
// activation granules of lane half h in 64-K step (q, t) of a chunk: the fp8 operand's bytes
// 0-15 and 16-31 (MXFP4 weights pair granules h and h + 2 of the step, see the kernel header)
TPG_HD int gran_lo(bool mx, int q, int t, int h) { return mx ? 8 * q + 2 * t + h : 8 * q + 4 * h + 2 * t; }
TPG_HD int gran_hi(bool mx, int q, int t, int h) { return mx ? gran_lo(mx, q, t, h) + 4 : gran_lo(mx, q, t, h) + 1; }

// Epilogue output columns of lane l, 4-column group g4: first GEMM h columns (of I),
// second GEMM y columns (of N)
TPG_HD int h_col(int nt, int wave, int g4, int lane) { return nt * (kBN / 2) + wave * 32 + g4 * 8 + (lane >> 5) * 4; }
TPG_HD int y_col(int nt, int wave, int g4, int lane) { return nt * kBN + wave * 32 + g4 * 8 + (lane >> 5) * 4; }

}  // namespace w4
}  // namespace tpg
