// The GEMM m-tile list, built on the device from the expert offsets (used by the table
// kernels and by the single-launch small-token forward).
#pragma once
#include "wave_ops.h"

namespace tpg {

// m-tiles of an expert with cnt rows when a last partial tile of at most bm / 2 rows joins the
// tile before it (so the last tile holds up to 1.5 bm rows)
__host__ __device__ inline int merged_m_tiles(int cnt, int bm) {
    if (cnt <= 0) return 0;
    const int m = cnt / bm + (cnt % bm > bm / 2 ? 1 : 0);
    return m > 0 ? m : 1;
}

// GEMM tile list from offsets (LDS or global, E+1 entries): tiles[2i] = expert, tiles[2i+1] =
// first row of the tile within the expert (tiles of bm rows); n_tiles[0] = count, n_tiles[1] =
// tiles before the partial section.  by_expert = 0: full tiles first (expert by expert), then each
// expert's partial last tile.  1: every expert's tiles together in row order (n_tiles[1] = count).
// 2: as 1, with a last partial tile of at most bm / 2 rows merged into the tile before it
// (merged_m_tiles), and the experts whose last tile is such a merged one (the longest-running
// tiles) first, so that their workgroups start in the first round.  Thread e < E handles expert e;
// every thread of the workgroup must call it (it holds a barrier); ws is 8 ints of LDS (see
// block_incl_sum256).  Returns the tile count (in every thread).
__device__ __forceinline__ int build_tile_list(const int32_t *off, int E, int bm, int by_expert, int32_t *__restrict__ tiles,
                                int32_t *__restrict__ n_tiles, int *ws) {
    const int e = threadIdx.x;
    int full = 0, part = 0;
    if (e < E) {
        const int cnt = off[e + 1] - off[e];
        if (by_expert == 2) {
            const int m = merged_m_tiles(cnt, bm);
            const bool merged_last = cnt - (m - 1) * bm > bm;
            full = merged_last ? m : 0;  // the "full" section holds the experts with a merged last tile
            part = merged_last ? 0 : m;
        } else {
            full = by_expert ? (cnt + bm - 1) / bm : cnt / bm;
            part = !by_expert && (cnt % bm) ? 1 : 0;
        }
    }
    int sf = full, sp = part, total_full, total_part;
    block_incl_sum256(sf, sp, ws, &total_full, &total_part);
    if (by_expert == 2) {
        if (e < E) {
            const int m = full + part;
            const int f0 = full ? sf - full : total_full + sp - part;
            for (int i = 0; i < m; ++i) {
                tiles[2 * (f0 + i)] = e;
                tiles[2 * (f0 + i) + 1] = i * bm;
            }
        }
        if (e == 0) n_tiles[0] = n_tiles[1] = total_full + total_part;
        return total_full + total_part;
    }
    if (e < E) {
        const int f0 = sf - full;
        for (int m = 0; m < full; ++m) {
            tiles[2 * (f0 + m)] = e;
            tiles[2 * (f0 + m) + 1] = m * bm;
        }
        if (part) {
            const int pos = total_full + sp - 1;
            tiles[2 * pos] = e;
            tiles[2 * pos + 1] = full * bm;
        }
    }
    if (e == 0) {
        n_tiles[0] = total_full + total_part;
        n_tiles[1] = total_full;
    }
    return total_full + total_part;
}

}  // namespace tpg
