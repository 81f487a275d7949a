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
// Lane l holds experts l, l+64, l+128, l+192.  Each of the k rounds is one wave-wide maximum
// of a 32-bit key (the logit's bits mapped so that unsigned order is float order, -0 folded
// onto +0) over DPP row operations, then a ballot of the lanes holding it; only equal logits in
// several lanes take a second (minimum-id) reduction.  Every lane learns each round's winner,
// so the normaliser is summed in slot order by every lane alike and lane j keeps slot j.  If
// `ids` is not null, lane j < k also stores the slot's expert id (or -1) at ids[j] (e.g. in LDS).
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

}  // namespace route_detail

__device__ __forceinline__ void route_token(const float *__restrict__ logits, const uint8_t *__restrict__ slot_drop,
                                            int64_t t, int E, int k, int lane, int32_t *__restrict__ topk_idx,
                                            float *__restrict__ topk_w, int32_t *ids) {
    using namespace route_detail;
    const float *l = logits + t * E;
    uint32_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        key[q] = e < E ? logit_key(l[e]) : 0u;  // 0: no expert (or already taken)
    }
    int my_id = -1;
    float my_ex = 0.0f, lmax = 0.0f, z = 0.0f;
    for (int j = 0; j < k; ++j) {
        // this lane's best remaining expert: ids grow with q, so strict '>' keeps the lower id
        uint32_t bk = 0u;
        int bq = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (key[q] > bk) {
                bk = key[q];
                bq = q;
            }
        const uint32_t m = wave::max_u32(bk);  // > 0: k <= E experts are live
        const uint64_t holders = __ballot(bk == m);
        int win;
        if ((holders & (holders - 1)) == 0) {  // one lane holds the largest logit
            const int wl = __builtin_ctzll(holders);
            win = wl + 64 * __builtin_amdgcn_readlane(bq, wl);
        } else {  // equal logits in several lanes: the lowest id among them
            win = (int)wave::min_u32(bk == m ? (uint32_t)(lane + 64 * bq) : ~0u);
        }
        if (lane == (win & 63)) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (q == (win >> 6)) key[q] = 0u;
        }
        const float lj = key_logit(m);
        if (j == 0) lmax = lj;
        // renormalised softmax weights: exp(l_j - l_max) summed over the chosen slots in order
        const float ex = expf(lj - lmax);
        z += ex;
        if (lane == j) {
            my_id = win;
            my_ex = ex;
        }
    }
    if (lane < k) {
        const int64_t s = t * k + lane;
        const bool dropped = slot_drop != nullptr && slot_drop[s] != 0;
        topk_idx[s] = dropped ? -1 : my_id;
        topk_w[s] = my_ex / z;
        if (ids) ids[lane] = dropped ? -1 : my_id;
    }
}

}  // namespace tpg
