// Unpermute + combine: out[t] = bf16( sum_j w[t][j] * y_perm[slot_row[t*k+j]] ).
//
// The top-k reduction that ends the fused MoE of FlashInfer "[SM90] Add W4A8
// MegaMoE support", with the unpermute folded in as Megatron-LM "add permute
// fusion into hybrid ep" folds it into the combine.  Each output element is an
// fp32 fused multiply-add chain over the token's slots in ascending j, skipping
// dropped slots (-1), then one round-to-nearest-even to bf16: no atomics, so the
// result is bitwise reproducible.  One wave per token; every y row is read once
// with 16-byte loads, up to eight rows in flight per lane.
#include "moe_internal.h"

namespace tpg {

namespace {
__device__ __forceinline__ void fma8(float *acc, float w, const uint4 &v) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] = fmaf(w, __uint_as_float(u[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = fmaf(w, __uint_as_float(u[q] & 0xffff0000u), acc[2 * q + 1]);
    }
}
}  // namespace

__global__ __launch_bounds__(256) void combine_kernel(const uint4 *__restrict__ y_perm,
                                                      const int32_t *__restrict__ slot_row,
                                                      const float *__restrict__ topk_w, int T, int k, int row_vec,
                                                      uint4 *__restrict__ out) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int32_t *rows = slot_row + t * k;  // wave-uniform: scalar loads
    const float *w = topk_w + t * k;
    for (int c = lane; c < row_vec; c += 64) {
        float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        for (int j0 = 0; j0 < k; j0 += 8) {
            uint4 v[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = j0 + q;
                const int32_t r = j < k ? rows[j] : -1;
                v[q] = r >= 0 ? y_perm[(int64_t)r * row_vec + c] : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = j0 + q;
                if (j < k && rows[j] >= 0) fma8(acc, w[j], v[q]);
            }
        }
        uint4 o;
        o.x = (uint32_t)f32_to_bf16(acc[0]) | ((uint32_t)f32_to_bf16(acc[1]) << 16);
        o.y = (uint32_t)f32_to_bf16(acc[2]) | ((uint32_t)f32_to_bf16(acc[3]) << 16);
        o.z = (uint32_t)f32_to_bf16(acc[4]) | ((uint32_t)f32_to_bf16(acc[5]) << 16);
        o.w = (uint32_t)f32_to_bf16(acc[6]) | ((uint32_t)f32_to_bf16(acc[7]) << 16);
        out[t * row_vec + c] = o;
    }
}

hipError_t launch_combine(const uint16_t *y_perm, const int32_t *slot_row, const float *topk_w, int T, int k, int H,
                          uint16_t *out, hipStream_t s) {
    const int row_vec = H / 8;
    hipLaunchKernelGGL(combine_kernel, dim3((T + 3) / 4), dim3(256), 0, s, (const uint4 *)y_perm, slot_row, topk_w,
                       T, k, row_vec, (uint4 *)out);
    return hipGetLastError();
}

}  // namespace tpg
