// Permutation tables: a stable counting sort of the T*k (token, slot) pairs by
// expert id, giving expert-contiguous rows (Megatron-LM "add permute fusion into
// hybrid ep": tokens are permuted into expert order before the experts and
// unpermuted in the combine).  Rows of one expert keep ascending slot id
// s = t*k + j, so the result is a pure function of topk_idx and bit-exact.
//
// Three launches, no atomics outside LDS and nothing order-dependent:
//   1. chunk_hist  one workgroup per chunk of kChunk slots: LDS histogram -> chunk_counts[c][e]
//   2. scan        one workgroup of 1024 threads: the chunks are split into up to 16 parts per
//                  expert, a thread sums one (expert, part) with all its loads in flight, then
//                  per expert an exclusive prefix over parts and chunks (in place), an
//                  exclusive prefix over experts -> offsets[E+1]; in the forward the same launch
//                  also writes the GEMM tile list
//   3. rank        one workgroup per chunk, one wave per quarter chunk: per-wave LDS bases,
//                  then 64 slots at a time, a slot's rank among equal ids of lower lanes
//                  comes from 9 ballots (one per bit of id+1) and a popcount.
// The GEMM tile list (expert, m-tile) is built from offsets by build_tile_list (in the scan
// launch of the forward, or by build_tiles on its own).
//
// For up to kChunk slots the forward runs all of this (and the routing) in one workgroup
// instead: frontend_small, with the expert ids kept in LDS between the steps.  At small
// token counts the five launches it replaces cost more than their work.  Up to 2048 slots the
// three table launches are one (tables_small, after the router).
#include <algorithm>

#include "route_token.h"
#include "tile_list.h"

namespace tpg {

namespace {
constexpr int kWavesPerChunk = 4;
constexpr int kSub = kChunk / kWavesPerChunk;  // slots per wave in the rank kernel

__device__ __forceinline__ int valid_id(int32_t x, int E) { return ((unsigned)x < (unsigned)E) ? x : -1; }
}  // namespace

__global__ __launch_bounds__(256) void chunk_hist_kernel(const int32_t *__restrict__ idx, int64_t S, int E,
                                                         int32_t *__restrict__ chunk_counts) {
    __shared__ int h[256];
    for (int e = threadIdx.x; e < E; e += 256) h[e] = 0;
    __syncthreads();
    const int64_t base = (int64_t)blockIdx.x * kChunk;
    for (int i = threadIdx.x; i < kChunk; i += 256) {
        const int64_t s = base + i;
        if (s < S) {
            const int x = valid_id(idx[s], E);
            if (x >= 0) atomicAdd(&h[x], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += 256) chunk_counts[(int64_t)blockIdx.x * E + e] = h[e];
}

constexpr int kScanThreads = 1024;
constexpr int kScanBatch = 8;  // loads in flight per thread
// parts the chunk column of one expert is split into: at most 16 (the per-expert walk over the
// parts is serial), at least kScanBatch chunks each, and E * parts <= kScanThreads
inline int scan_parts(int64_t nch, int E) {
    const int64_t by_len = (nch + kScanBatch - 1) / kScanBatch;
    return (int)std::max<int64_t>(1, std::min<int64_t>({16, kScanThreads / E, by_len}));
}

__global__ __launch_bounds__(kScanThreads) void scan_kernel(int32_t *__restrict__ chunk_counts, int64_t nch, int E,
                                                            int P, int32_t *__restrict__ offsets, int bm,
                                                            int by_expert, int32_t *__restrict__ tiles,
                                                            int32_t *__restrict__ n_tiles) {
    __shared__ int part_base[kScanThreads];  // [part][E]: part sums, then exclusive bases
    __shared__ int off[257], ws[8];
    const int tid = threadIdx.x;
    const int e = tid % E, part = tid / E;
    const bool act = part < P;
    const int64_t cpp = (nch + P - 1) / P;  // chunks per part
    const int64_t c0 = act ? std::min<int64_t>(nch, part * cpp) : 0;
    const int64_t c1 = act ? std::min<int64_t>(nch, c0 + cpp) : 0;
    int32_t *col = chunk_counts + e;
    int sum = 0;
    for (int64_t c = c0; c < c1; c += kScanBatch) {
        int v[kScanBatch];
#pragma unroll
        for (int q = 0; q < kScanBatch; ++q) v[q] = c + q < c1 ? col[(c + q) * E] : 0;
#pragma unroll
        for (int q = 0; q < kScanBatch; ++q) sum += v[q];
    }
    if (act) part_base[part * E + e] = sum;
    __syncthreads();
    int etot = 0;  // expert tid's total
    if (tid < E)
        for (int pp = 0; pp < P; ++pp) {
            const int v = part_base[pp * E + tid];
            part_base[pp * E + tid] = etot;
            etot += v;
        }
    // exclusive prefix over experts (the barrier inside also publishes the part bases)
    int incl = etot, unused = 0, total, unused_total;
    block_incl_sum256(incl, unused, ws, &total, &unused_total);
    // exclusive prefix over chunks, in place: the part's base plus the running sum within it
    if (act) {
        int run = part_base[part * E + e];
        for (int64_t c = c0; c < c1; c += kScanBatch) {
            int v[kScanBatch];
#pragma unroll
            for (int q = 0; q < kScanBatch; ++q) v[q] = c + q < c1 ? col[(c + q) * E] : 0;
#pragma unroll
            for (int q = 0; q < kScanBatch; ++q) {
                if (c + q < c1) col[(c + q) * E] = run;
                run += v[q];
            }
        }
    }
    if (tid < E) {
        offsets[tid] = incl - etot;
        off[tid] = incl - etot;
    }
    if (tid == 0) {
        offsets[E] = total;
        off[E] = total;
    }
    if (tiles == nullptr) return;  // uniform
    __syncthreads();
    build_tile_list(off, E, bm, by_expert, tiles, n_tiles, ws);
}

__global__ __launch_bounds__(256) void rank_kernel(const int32_t *__restrict__ idx, int64_t S, int E,
                                                   const int32_t *__restrict__ chunk_prefix,
                                                   const int32_t *__restrict__ offsets,
                                                   int32_t *__restrict__ row_src, int32_t *__restrict__ slot_row) {
    __shared__ int cnt[kWavesPerChunk][256];
    const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int64_t c = blockIdx.x;
    for (int i = threadIdx.x; i < kWavesPerChunk * 256; i += 256) (&cnt[0][0])[i] = 0;
    __syncthreads();

    const int64_t sub = c * kChunk + (int64_t)w * kSub;
    for (int it = 0; it < kSub / 64; ++it) {
        const int64_t s = sub + it * 64 + lane;
        const int x = s < S ? valid_id(idx[s], E) : -1;
        if (x >= 0) atomicAdd(&cnt[w][x], 1);
    }
    __syncthreads();
    // per-wave base of every expert = offsets[e] + rows of e in earlier chunks + earlier waves
    for (int e = threadIdx.x; e < E; e += 256) {
        int b = offsets[e] + chunk_prefix[c * E + e];
        for (int ww = 0; ww < kWavesPerChunk; ++ww) {
            const int v = cnt[ww][e];
            cnt[ww][e] = b;
            b += v;
        }
    }
    __syncthreads();

    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int it = 0; it < kSub / 64; ++it) {
        const int64_t s = sub + it * 64 + lane;
        const int x = s < S ? valid_id(idx[s], E) : -1;
        const unsigned key = (unsigned)(x + 1);  // 0 .. 256
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = (key >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & lt);
        int r = -1;
        if (x >= 0) r = cnt[w][x] + rank;
        // every lane has read its base; the lowest lane of each group advances it
        __builtin_amdgcn_wave_barrier();
        if (x >= 0 && rank == 0) cnt[w][x] += __popcll(peers);
        __builtin_amdgcn_wave_barrier();
        if (s < S) {
            slot_row[s] = r;
            if (r >= 0) row_src[r] = (int32_t)s;
        }
    }
    // rows past the live count R hold -1 (this chunk's share of [R, S))
    const int64_t R = offsets[E];
    for (int i = threadIdx.x; i < kChunk; i += 256) {
        const int64_t s = c * kChunk + i;
        if (s < S && s >= R) row_src[s] = -1;
    }
}

__global__ __launch_bounds__(256) void build_tiles_kernel(const int32_t *__restrict__ offsets, int E, int bm,
                                                          int by_expert, int32_t *__restrict__ tiles,
                                                          int32_t *__restrict__ n_tiles) {
    __shared__ int ws[8];
    build_tile_list(offsets, E, bm, by_expert, tiles, n_tiles, ws);
}

// Routing, tables and tile list of at most kChunk slots in one workgroup of 16 waves: the same
// results as route_topk + chunk_hist + scan + rank + build_tiles.  Slot s is thread s.
constexpr int kFrontWaves = kChunk / kWave;  // 16
constexpr int kTablesPasses = 2;                        // tables_small_kernel: slots per thread
constexpr int kTablesSlots = kTablesPasses * kChunk;    // its largest slot count (2048)
__global__ __launch_bounds__(kChunk) void frontend_small_kernel(
    const float *__restrict__ logits, const uint8_t *__restrict__ slot_drop, int T, int E, int k, int bm, int by_expert,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t *__restrict__ offsets,
    int32_t *__restrict__ row_src, int32_t *__restrict__ slot_row, int32_t *__restrict__ tiles,
    int32_t *__restrict__ n_tiles) {
    __shared__ int32_t sid[kChunk];          // expert id (or -1) of every slot
    __shared__ int cnt[kFrontWaves][256];    // per-wave counts, then per-wave bases
    __shared__ int off[257];
    __shared__ int ws[8];                    // block prefix-sum scratch
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int S = T * k;

    // routing: one 16-lane row per token, four tokens per wave
    for (int t0 = w * 4; t0 < T; t0 += kFrontWaves * 4) {
        const int t = t0 + (lane >> 4);
        route_token16(logits, slot_drop, t < T ? t : T - 1, t < T, E, k, lane & 15, topk_idx, topk_w, sid + t * k);
    }
    for (int i = tid; i < kFrontWaves * 256; i += kChunk) (&cnt[0][0])[i] = 0;
    __syncthreads();

    // per-wave histograms
    const int x = tid < S ? valid_id(sid[tid], E) : -1;
    if (x >= 0) atomicAdd(&cnt[w][x], 1);
    __syncthreads();

    // per expert: exclusive bases over the waves and the total; exclusive scan over experts
    int tot = 0;
    if (tid < 256)
        for (int ww = 0; ww < kFrontWaves; ++ww) {
            const int v = cnt[ww][tid];
            cnt[ww][tid] = tot;
            tot += v;
        }
    int incl = tot, unused = 0, R_all, unused_total;
    block_incl_sum256(incl, unused, ws, &R_all, &unused_total);
    if (tid < E) {
        off[tid] = incl - tot;
        offsets[tid] = incl - tot;
    }
    if (tid == 0) {
        off[E] = R_all;
        offsets[E] = R_all;
    }
    __syncthreads();

    // rank of the slot among equal ids of lower lanes: 9 ballots (one per bit of id+1)
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const unsigned key = (unsigned)(x + 1);
    uint64_t peers = ~0ull;
#pragma unroll
    for (int b = 0; b < 9; ++b) {
        const bool bit = (key >> b) & 1u;
        const uint64_t bal = __ballot(bit);
        peers &= bit ? bal : ~bal;
    }
    const int rank = __popcll(peers & lt);
    const int R = off[E];
    if (tid < S) {
        const int r = x >= 0 ? off[x] + cnt[w][x] + rank : -1;
        slot_row[tid] = r;
        if (r >= 0) row_src[r] = tid;
        if (tid >= R) row_src[tid] = -1;  // rows past the live count (r < R never lands here)
    }

    // GEMM tile list
    build_tile_list(off, E, bm, by_expert, tiles, n_tiles, ws);
}

// Tables (and, given tiles, the tile list) of at most kTablesSlots slots in one workgroup of 16
// waves, after the router: the same results as chunk_hist + scan + rank, in one launch instead
// of three.  Slot s is thread s % kChunk of pass s / kChunk; the passes, and the waves within a
// pass, take an expert's rows in slot order, so the order stays stable.  (Routing stays with
// route_topk's many workgroups: routing 256 tokens inside one workgroup measured as slow as the
// separate launches.)
__global__ __launch_bounds__(kChunk) void tables_small_kernel(const int32_t *__restrict__ idx, int S, int E, int bm,
                                                              int by_expert, int32_t *__restrict__ offsets,
                                                              int32_t *__restrict__ row_src,
                                                              int32_t *__restrict__ slot_row,
                                                              int32_t *__restrict__ tiles,
                                                              int32_t *__restrict__ n_tiles) {
    __shared__ int cnt[kTablesPasses * kFrontWaves][256];  // per (pass, wave) counts, then bases
    __shared__ int off[257];
    __shared__ int ws[8];  // block prefix-sum scratch
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    int x[kTablesPasses];
#pragma unroll
    for (int p = 0; p < kTablesPasses; ++p) {
        const int slot = p * kChunk + tid;
        x[p] = slot < S ? valid_id(idx[slot], E) : -1;
    }
    for (int i = tid; i < kTablesPasses * kFrontWaves * 256; i += kChunk) (&cnt[0][0])[i] = 0;
    __syncthreads();
#pragma unroll
    for (int p = 0; p < kTablesPasses; ++p)
        if (x[p] >= 0) atomicAdd(&cnt[p * kFrontWaves + w][x[p]], 1);
    __syncthreads();

    // per expert: exclusive bases over the (pass, wave) groups in slot order and the total;
    // exclusive scan over experts
    int tot = 0;
    if (tid < 256)
        for (int g = 0; g < kTablesPasses * kFrontWaves; ++g) {
            const int v = cnt[g][tid];
            cnt[g][tid] = tot;
            tot += v;
        }
    int incl = tot, unused = 0, R_all, unused_total;
    block_incl_sum256(incl, unused, ws, &R_all, &unused_total);
    if (tid < E) {
        off[tid] = incl - tot;
        offsets[tid] = incl - tot;
    }
    if (tid == 0) {
        off[E] = R_all;
        offsets[E] = R_all;
    }
    __syncthreads();

    // rank of the slot among equal ids of lower lanes of its pass: 9 ballots (one per bit of id+1)
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int R = off[E];
#pragma unroll
    for (int p = 0; p < kTablesPasses; ++p) {
        const unsigned key = (unsigned)(x[p] + 1);
        uint64_t peers = ~0ull;
#pragma unroll
        for (int b = 0; b < 9; ++b) {
            const bool bit = (key >> b) & 1u;
            const uint64_t bal = __ballot(bit);
            peers &= bit ? bal : ~bal;
        }
        const int rank = __popcll(peers & lt);
        const int slot = p * kChunk + tid;
        if (slot < S) {
            const int r = x[p] >= 0 ? off[x[p]] + cnt[p * kFrontWaves + w][x[p]] + rank : -1;
            slot_row[slot] = r;
            if (r >= 0) row_src[r] = slot;
            if (slot >= R) row_src[slot] = -1;  // rows past the live count (r < R never lands here)
        }
    }
    if (tiles == nullptr) return;  // uniform
    build_tile_list(off, E, bm, by_expert, tiles, n_tiles, ws);
}

hipError_t launch_frontend_small(const float *logits, const uint8_t *slot_drop, int T, int E, int k, int bm,
                                 int by_expert, int32_t *topk_idx, float *topk_w, int32_t *offsets,
                                 int32_t *row_src, int32_t *slot_row, int32_t *tiles, int32_t *n_tiles,
                                 hipStream_t s) {
    if (T > 256 || (int64_t)T * k > kChunk) return hipErrorInvalidValue;  // the LDS tables' sizes
    hipLaunchKernelGGL(frontend_small_kernel, dim3(1), dim3(kChunk), 0, s, logits, slot_drop, T, E, k, bm, by_expert,
                       topk_idx, topk_w, offsets, row_src, slot_row, tiles, n_tiles);
    return hipGetLastError();
}

hipError_t launch_tables(const int32_t *topk_idx, int T, int k, int E, int32_t *chunk_counts, int32_t *offsets,
                         int32_t *row_src, int32_t *slot_row, int bm, int by_expert, int32_t *tiles,
                         int32_t *n_tiles, hipStream_t s) {
    const int64_t S = (int64_t)T * k;
    if (S <= kTablesSlots) {
        hipLaunchKernelGGL(tables_small_kernel, dim3(1), dim3(kChunk), 0, s, topk_idx, (int)S, E, bm, by_expert, offsets,
                           row_src, slot_row, tiles, n_tiles);
        return hipGetLastError();
    }
    const int64_t nch = (S + kChunk - 1) / kChunk;
    hipLaunchKernelGGL(chunk_hist_kernel, dim3(nch), dim3(256), 0, s, topk_idx, S, E, chunk_counts);
    hipLaunchKernelGGL(scan_kernel, dim3(1), dim3(kScanThreads), 0, s, chunk_counts, nch, E, scan_parts(nch, E),
                       offsets, bm, by_expert, tiles, n_tiles);
    hipLaunchKernelGGL(rank_kernel, dim3(nch), dim3(256), 0, s, topk_idx, S, E, chunk_counts, offsets, row_src,
                       slot_row);
    return hipGetLastError();
}

hipError_t launch_build_tiles(const int32_t *offsets, int E, int bm, int by_expert, int32_t *tiles,
                              int32_t *n_tiles, hipStream_t s) {
    hipLaunchKernelGGL(build_tiles_kernel, dim3(1), dim3(256), 0, s, offsets, E, bm, by_expert, tiles, n_tiles);
    return hipGetLastError();
}

}  // namespace tpg
