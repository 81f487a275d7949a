// Routing of one token by one wave (wave64), shared by the router kernel and the fused
// front end: softmax over E logits, top-k, renormalised over the k chosen.
//
// FlashInfer "[SM90] Add W4A8 MegaMoE support", Usage section: the fused MoE takes
// per-token expert ids (-1 masks a route) and fp32 routing weights.  Selection compares
// the fp32 logits directly (softmax is strictly increasing), so the chosen ids are
// exact; equal logits go to the lower expert id and slots are ordered by descending
// logit.  The weight of slot j is exp(l_j - l_max) / sum_i exp(l_i - l_max) over the k
// chosen, which is the full softmax renormalised over the top k.
//
// A token is routed by one row of 16 lanes (a DPP row), four tokens per wave64: lane i of the
// row holds experts i, i+16, i+32, ...  Each of the k rounds is a row-wide maximum of a 32-bit
// key (the logit's bits mapped so that unsigned order is float order, -0 folded onto +0) and a
// row-wide minimum of the ids holding it (equal logits -> lower id), four DPP steps each
// (quad_perm, row_half_mirror, row_mirror), so the rows never exchange data.  Every lane of the
// row learns each round's winner, so the normaliser is summed in slot order identically in
// every lane; lane i keeps slots i, i + 16, ... (two of them for k <= 32, sixteen for k up to
// 256).  If `ids` is not null, the slots' expert ids (or -1) are also stored at ids[j] (e.g. in
// LDS).
#pragma once
#include "wave_ops.h"

namespace tpg {
namespace route_detail {

// unsigned order of the key = numeric order of the (finite) float; -0 and +0 share a key; no
// finite or infinite value maps to 0
__device__ __forceinline__ uint32_t logit_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key & 0x7fffffffu) : ~key);
}

// maximum / minimum over the 16 lanes of each row, returned to every lane of the row
__device__ __forceinline__ uint32_t row_max(uint32_t x) {
    using namespace wave;
    x = max(x, dpp<kQuadSwap1, 0xf>(x, 0u));
    x = max(x, dpp<kQuadSwap2, 0xf>(x, 0u));
    x = max(x, dpp<kRowHalfMirror, 0xf>(x, 0u));
    return max(x, dpp<kRowMirror, 0xf>(x, 0u));
}
__device__ __forceinline__ uint32_t row_min(uint32_t x) {
    using namespace wave;
    x = min(x, dpp<kQuadSwap1, 0xf>(x, ~0u));
    x = min(x, dpp<kQuadSwap2, 0xf>(x, ~0u));
    x = min(x, dpp<kRowHalfMirror, 0xf>(x, ~0u));
    return min(x, dpp<kRowMirror, 0xf>(x, ~0u));
}

// V: experts per lane (16 V >= E); J: slots per lane (16 J >= k).  t is a valid token for every
// row; only rows with `valid` store.
template <int V, int J>
__device__ __forceinline__ void route_row(const float *__restrict__ logits, const uint8_t *__restrict__ slot_drop,
                                          int64_t t, bool valid, int E, int k, int i,
                                          int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int32_t *ids) {
    const float *l = logits + t * E;
    uint32_t key[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        const int e = i + 16 * q;
        key[q] = e < E ? logit_key(l[e]) : 0u;  // 0: no expert (or already taken)
    }
    int id[J];
    float exs[J];
#pragma unroll
    for (int h = 0; h < J; ++h) {
        id[h] = -1;
        exs[h] = 0.0f;
    }
    float lmax = 0.0f, z = 0.0f;
    for (int j = 0; j < k; ++j) {
        // this lane's best remaining expert: ids grow with q, so strict '>' keeps the lower id
        uint32_t bk = 0u;
        int bq = 0;
#pragma unroll
        for (int q = 0; q < V; ++q)
            if (key[q] > bk) {
                bk = key[q];
                bq = q;
            }
        const uint32_t m = row_max(bk);  // > 0: k <= E experts are live
        const int win = (int)row_min(bk == m ? (uint32_t)(i + 16 * bq) : ~0u);
        if ((win & 15) == i) {
#pragma unroll
            for (int q = 0; q < V; ++q)
                if (q == (win >> 4)) key[q] = 0u;
        }
        const float lj = key_logit(m);
        if (j == 0) lmax = lj;
        // renormalised softmax weights: exp(l_j - l_max) summed over the chosen slots in order
        const float ex = expf(lj - lmax);
        z += ex;
#pragma unroll
        for (int h = 0; h < J; ++h)
            if (j == i + 16 * h) {
                id[h] = win;
                exs[h] = ex;
            }
    }
    if (!valid) return;
#pragma unroll
    for (int h = 0; h < J; ++h) {
        const int j = i + 16 * h;
        if (j < k) {
            const int64_t s = t * k + j;
            const bool dropped = slot_drop != nullptr && slot_drop[s] != 0;
            const int sid = dropped ? -1 : id[h];
            topk_idx[s] = sid;
            topk_w[s] = exs[h] / z;
            if (ids) ids[j] = sid;
        }
    }
}

}  // namespace route_detail

// Routes token t with the 16-lane row this lane belongs to (i = lane within the row).  All
// 64 lanes of the wave must call it with the same E and k.
__device__ __forceinline__ void route_token16(const float *__restrict__ logits, const uint8_t *__restrict__ slot_drop,
                                              int64_t t, bool valid, int E, int k, int i,
                                              int32_t *__restrict__ topk_idx, float *__restrict__ topk_w,
                                              int32_t *ids) {
    using namespace route_detail;
    if (k > 32) {  // k <= E, so E > 32
        if (E <= 64)
            route_row<4, 16>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
        else if (E <= 128)
            route_row<8, 16>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
        else
            route_row<16, 16>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
    } else if (E <= 16) {
        route_row<1, 2>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
    } else if (E <= 32) {
        route_row<2, 2>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
    } else if (E <= 64) {
        route_row<4, 2>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
    } else if (E <= 128) {
        route_row<8, 2>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
    } else {
        route_row<16, 2>(logits, slot_drop, t, valid, E, k, i, topk_idx, topk_w, ids);
    }
}

}  // namespace tpg
