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
// Lane l holds experts l, l+64, l+128, l+192; each of the k rounds is a wave-wide argmax
// (butterfly over 64 lanes); lane j keeps slot j.  If `ids` is not null, lane j < k also
// stores the slot's expert id (or -1) at ids[j] (e.g. in LDS).
#pragma once

#include "moe_internal.h"

namespace tpg {

__device__ __forceinline__ void route_token(const float *__restrict__ logits, const uint8_t *__restrict__ slot_drop,
                                            int64_t t, int E, int k, int lane, int32_t *__restrict__ topk_idx,
                                            float *__restrict__ topk_w, int32_t *ids) {
    const float *l = logits + t * E;
    float v[4];
    bool live[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int e = lane + 64 * q;
        live[q] = e < E;
        v[q] = live[q] ? l[e] : 0.0f;
    }

    int my_id = -1;
    float my_logit = 0.0f, lmax = 0.0f;
    for (int j = 0; j < k; ++j) {
        // best remaining expert of this lane (ids grow with q, so strict '>' keeps the lower id)
        float bv = 0.0f;
        int bi = 0x7fffffff;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (live[q] && (bi == 0x7fffffff || v[q] > bv)) {
                bv = v[q];
                bi = lane + 64 * q;
            }
        // wave argmax: larger logit wins, equal logits -> lower id
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float ov = __shfl_xor(bv, off);
            const int oi = __shfl_xor(bi, off);
            const bool take = (oi != 0x7fffffff) && (bi == 0x7fffffff || ov > bv || (ov == bv && oi < bi));
            if (take) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & 63) == lane) {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (bi == lane + 64 * q) live[q] = false;
        }
        if (j == 0) lmax = bv;
        if (lane == j) {
            my_id = bi;
            my_logit = bv;
        }
    }

    // renormalised softmax weights of the k chosen; every lane gets the same sum
    float ex = lane < k ? expf(my_logit - lmax) : 0.0f;
    float z = ex;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) z += __shfl_xor(z, off);
    if (lane < k) {
        const int64_t s = t * k + lane;
        const bool dropped = slot_drop != nullptr && slot_drop[s] != 0;
        topk_idx[s] = dropped ? -1 : my_id;
        topk_w[s] = ex / z;
        if (ids) ids[lane] = dropped ? -1 : my_id;
    }
}

}  // namespace tpg
