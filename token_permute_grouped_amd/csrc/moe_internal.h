// Internal declarations shared by the HIP translation units of libtpg_moe.so.
// Every kernel is written for gfx950 (CDNA4, wave64).
#pragma once
#include <algorithm>

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace tpg {

constexpr int kWave = 64;

// ---------------------------------------------------------------- workspace layout
// One layout for every entry point, computed on the host from the problem only
// (never from the routing), so a workspace allocated once serves every call of that
// shape.  Offsets are 256-byte aligned.
// Hand-off words of the single-launch small-token forward (the first bytes of a W4A8 workspace),
// each in a 128-byte line of its own, followed by its counters, one per line too:
// rq_cnt [max_tiles][I/128], mt_ready [max_tiles].
constexpr int kSyncLine = 32;  // uint32 per 128-byte line
struct FusedSync {
    uint64_t go;  // set while a forward runs (after its tables are built), 0 after
    uint32_t pad0[kSyncLine - 2];
    uint32_t next_item;  // item claims
    uint32_t pad1[kSyncLine - 1];
    uint32_t done;  // workgroups finished
    uint32_t pad2[kSyncLine - 1];
    uint32_t err;  // nonzero: a bounded wait gave up
    uint32_t pad3[kSyncLine - 1];
    uint32_t rq_total;  // 128-column blocks of h re-quantised
    uint32_t pad4[kSyncLine - 1];
    uint32_t gemm_done;  // workgroups past their last GEMM tile
    uint32_t pad5[kSyncLine - 1];
};

struct WsLayout {
    size_t fsync;         // W4A8: FusedSync + counters (always at offset 0)
    size_t chunk_counts;  // int32 [n_chunks][E]   permutation: per-chunk histograms
    size_t tiles;         // int32 [2 * max_tiles]  grouped GEMMs: (expert, first row) per m-tile
    size_t n_tiles;       // int32 [4]              grouped GEMMs: tile count, full-tile count
    size_t h;             // bf16 [S][I]  or (W4A8) fp8 [S][I]
    size_t h_scale;       // W4A8: fp32 [S][I/128]
    size_t h32;           // W4A8: fp32 [S][I] (SwiGLU output before re-quantisation); with the GEMM1
                          // K split, its partial sums [2 halves][gate, up][S][I]
    size_t topk_idx;      // forward only: int32 [T][k]
    size_t topk_w;        // forward only: fp32 [T][k]
    size_t offsets;       // forward only: int32 [E+1]
    size_t row_src;       // forward only: int32 [S]
    size_t slot_row;      // forward only: int32 [S]
    size_t x_perm;        // forward only: bf16/fp8 [S][H]
    size_t x_perm_scale;  // forward only: fp32 [S][H/128]
    size_t y_perm;        // forward only: bf16 [S][H]
    size_t permute_end, ffn_end, forward_end;
};

// rows of the permutation processed by one workgroup of the table kernels
constexpr int kChunk = 1024;
// M tile (rows of one expert per workgroup) of the bf16 and of the W4A8 grouped GEMMs
constexpr int kGemmBM = 256;
constexpr int kGemmBMW4A8 = 64;

inline int64_t n_slots(const moe_problem &p) { return (int64_t)p.T * p.k; }
inline int64_t n_chunks(const moe_problem &p) { return (n_slots(p) + kChunk - 1) / kChunk; }
inline int gemm_bm(const moe_problem &p) { return p.prec == MOE_PREC_BF16 ? kGemmBM : kGemmBMW4A8; }
// upper bound of sum_e ceil(count_e / bm) over any routing (also of the merged W4A8 tile count)
inline int64_t max_m_tiles(const moe_problem &p) { return (n_slots(p) + gemm_bm(p) - 1) / gemm_bm(p) + p.E; }
// W4A8 GEMM1 split in two halves of K (two workgroups per tile): at most 256 GEMM1 tiles whatever
// the routing (each tile would otherwise stream its weights on a CU of its own, one wave per SIMD,
// with the NVFP4 dequant unhidden and few bytes in flight), K a multiple of 512.  Deterministic:
// the halves' partial sums are added by the re-quantisation (h32 holds the four partial planes:
// 4 x S x I floats).
inline bool w4a8_split_gemm1(const moe_problem &p) {
    const int64_t experts = std::min<int64_t>(p.E, (int64_t)p.T * p.k);
    return p.prec != MOE_PREC_BF16 && experts * (2 * (int64_t)p.I / 128) <= 256 && p.H % 512 == 0 && p.T <= 32;
}
// tile list order (build_tile_list's by_expert): bf16 full tiles first; W4A8 by expert, an expert's
// last partial tile of at most 32 rows merged into the tile before it (a 96-row tile at most)
inline int tile_order(const moe_problem &p) { return p.prec == MOE_PREC_BF16 ? 0 : 2; }

WsLayout ws_layout(const moe_problem &p);

// ---------------------------------------------------------------- launchers (enqueue only)
hipError_t launch_route_topk(const float *logits, const uint8_t *slot_drop, int T, int E, int k, int32_t *topk_idx,
                             float *topk_w, hipStream_t s);

hipError_t launch_tables(const int32_t *topk_idx, int T, int k, int E, int32_t *chunk_counts, int32_t *offsets,
                         int32_t *row_src, int32_t *slot_row, int bm, int by_expert, int32_t *tiles,
                         int32_t *n_tiles, hipStream_t s);

hipError_t launch_permute(const void *x, const float *x_scale, const int32_t *slot_row, int T, int k, int H,
                          int elem_bytes, void *x_perm, float *x_perm_scale, hipStream_t s);

// GEMM m-tile list in order by_expert (see build_tile_list and tile_order)
hipError_t launch_build_tiles(const int32_t *offsets, int E, int bm, int by_expert, int32_t *tiles,
                              int32_t *n_tiles, hipStream_t s);

// routing + tables + tile list in one workgroup, for at most kChunk slots
hipError_t launch_frontend_small(const float *logits, const uint8_t *slot_drop, int T, int E, int k, int bm,
                                 int by_expert, int32_t *topk_idx, float *topk_w, int32_t *offsets,
                                 int32_t *row_src, int32_t *slot_row, int32_t *tiles, int32_t *n_tiles,
                                 hipStream_t s);

hipError_t launch_gemm1_swiglu_bf16(const uint16_t *x_perm, const uint16_t *w1, const int32_t *offsets,
                                    const int32_t *tiles, const int32_t *n_tiles, int64_t max_tiles, int H, int I,
                                    int glu_interleave, float clamp, uint16_t *h, hipStream_t s);

// GEMM1 + SwiGLU reading its activation rows from the token rows x [T][H] through row_src
// (the gather fused into the tile loads); needs gather_fits(T, H)
inline bool gather_fits(int64_t T, int64_t H) { return T * H * 2 <= 0x7FFFFFFF; }
inline bool gather_fits_fp8(int64_t T, int64_t H) { return T * H <= 0x7FFFFFFF; }
// moe_forward skips the separate row gather and runs GEMM1 on x (and x_scale) through row_src
inline bool fused_gather(const moe_problem &p) {
    return p.prec == MOE_PREC_BF16 ? gather_fits(p.T, p.H) : gather_fits_fp8(p.T, p.H);
}
hipError_t launch_gemm1_swiglu_gather_bf16(const uint16_t *x, const int32_t *row_src, int T, int k,
                                           const uint16_t *w1, const int32_t *offsets, const int32_t *tiles,
                                           const int32_t *n_tiles, int64_t max_tiles, int H, int I,
                                           int glu_interleave, float clamp, uint16_t *h, hipStream_t s);

// row_dst NULL: y row r in the expert-major order; else y row row_dst[r] (the scatter epilogue:
// row_src as row_dst puts every row at its slot t*k + j)
hipError_t launch_gemm2_bf16(const uint16_t *h, const uint16_t *w2, const int32_t *offsets, const int32_t *tiles,
                             const int32_t *n_tiles, int64_t max_tiles, int H, int I, uint16_t *y_perm,
                             const int32_t *row_dst, hipStream_t s);

// row_src NULL: x_perm / x_perm_scale are the expert-ordered rows; else x / x_scale token rows
// read through row_src (the gather fused into GEMM1; needs gather_fits_fp8(T, H)).  row_dst as
// for launch_gemm2_bf16.
hipError_t launch_grouped_ffn_w4a8(const uint8_t *x_perm, const float *x_perm_scale, const int32_t *row_src,
                                   const int32_t *offsets, const int32_t *tiles, const int32_t *n_tiles,
                                   int64_t max_tiles, const moe_weights &w, const moe_problem &p, float *h32,
                                   uint8_t *h8, float *hs, uint16_t *y_perm, const int32_t *row_dst,
                                   hipStream_t s);

// slot_order false: slot s = t*k + j reads y row slot_row[s]; true: y row s (the scatter
// epilogue's layout).  Either way a slot with slot_row[s] < 0 is dropped.
hipError_t launch_combine(const uint16_t *y_perm, const int32_t *slot_row, const float *topk_w, int T, int k, int H,
                          bool slot_order, uint16_t *out, hipStream_t s);

// The whole W4A8 forward in one launch (up to 256 tokens and 2048 slots, H and I multiples of
// 1024, every byte offset below 2^31): routing, tables, both GEMMs with the SwiGLU and the
// re-quantisation, and the combine.  Buffers are the forward's workspace regions.
bool forward_small_w4a8_fits(const moe_problem &p);
hipError_t launch_forward_small_w4a8(const float *logits, const uint8_t *slot_drop, const uint8_t *x,
                                     const float *x_scale, const moe_weights &w, const moe_problem &p,
                                     int64_t max_tiles, FusedSync *sync, int32_t *topk_idx, float *topk_w,
                                     int32_t *offsets, int32_t *row_src, int32_t *slot_row, int32_t *tiles,
                                     int32_t *n_tiles, float *h32, uint8_t *h8, float *hs, uint16_t *y,
                                     uint16_t *out, hipStream_t s);

hipError_t launch_w4a8_dequant_table(uint8_t *out8, hipStream_t s);

hipError_t launch_tile_weights(const uint8_t *codes, const uint8_t *bscale, uint8_t *codes_tiled,
                               uint8_t *bscale_tiled, int E, int N, int K, bool mx, hipStream_t s);

// ---------------------------------------------------------------- device helpers
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// two floats -> two bf16 (round to nearest even) packed in one word, a in the low half: one
// v_cvt_pk_bf16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// One step of the combine's fp32 chain for 8 consecutive columns: acc[i] = fma(w, y[i], acc[i])
// with y eight bf16 values (used by the combine kernel and by the single-launch forward, so both
// give the same bits).
__device__ __forceinline__ void combine_fma8(float *acc, float w, const uint4 &v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, __uint_as_float(u[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, __uint_as_float(u[q] & 0xffff0000u), acc[2 * q + 1]);
    }
}

// eight fp32 values -> eight bf16 (round to nearest even) in 16 bytes
__device__ __forceinline__ uint4 combine_pack8(const float *a) {
    uint4 o;
    o.x = pack_bf16x2(a[0], a[1]);
    o.y = pack_bf16x2(a[2], a[3]);
    o.z = pack_bf16x2(a[4], a[5]);
    o.w = pack_bf16x2(a[6], a[7]);
    return o;
}

// Streamed-out rows (written once, not read again by the kernel that writes them) are stored
// through a buffer resource over the row with the sc1 cache-policy bit: a device-scope store,
// written through the XCD's L2 rather than left there as a dirty line.  Measured on the row
// gather and on the combine: equal or faster on every workload (the gather on a 101 MB output
// 32 -> 18 us, the combine on the skewed layer 199 -> 190 us); the GEMM epilogues, whose
// output tiles share the L2 with reused operands, measured slower with it and keep plain stores.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(void *row, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(row, (short)0, bytes, 0x00020000);
}
__device__ __forceinline__ void store16_through(__amdgpu_buffer_rsrc_t r, uint32_t byte_off, const uint4 &v) {
    typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
    constexpr int kSc1 = 16;  // cache-policy bits of a buffer store: sc0 = 1, nt = 2, sc1 = 16
    __builtin_amdgcn_raw_buffer_store_b128((u32x4_t){v.x, v.y, v.z, v.w}, r, byte_off, 0, kSc1);
}

}  // namespace tpg
