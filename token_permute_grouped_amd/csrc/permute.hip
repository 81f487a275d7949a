// Permute (row gather into expert-contiguous order): x_perm[slot_row[t*k+j]] = x[t].
//
// Megatron-LM "add permute fusion into hybrid ep" moves each token row into the
// expert-major order the grouped GEMMs read.  Here the copy is driven from the
// token side: a wave reads x[t] once (16-byte loads, fully coalesced) and writes
// it to each of its k destination rows, so HBM sees exactly T*H reads and R*H
// writes, never a re-read of a token row.  On the W4A8 path the per-128 fp32
// activation scales travel with their row.
#include "moe_internal.h"

namespace tpg {

__global__ __launch_bounds__(256) void permute_kernel(const uint4 *__restrict__ x, const float *__restrict__ x_scale,
                                                      const int32_t *__restrict__ slot_row, int T, int k,
                                                      int row_vec, int n_scale, uint4 *__restrict__ x_perm,
                                                      float *__restrict__ x_perm_scale) {
    const int lane = threadIdx.x & 63;
    const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    const int32_t *rows = slot_row + t * k;  // wave-uniform: scalar loads

    const uint4 *src = x + t * row_vec;
    int c = lane;
    for (; c + 3 * 64 < row_vec; c += 4 * 64) {
        const uint4 v0 = src[c], v1 = src[c + 64], v2 = src[c + 128], v3 = src[c + 192];
        for (int j = 0; j < k; ++j) {
            if (rows[j] < 0) continue;
            uint4 *dst = x_perm + (int64_t)rows[j] * row_vec;
            dst[c] = v0;
            dst[c + 64] = v1;
            dst[c + 128] = v2;
            dst[c + 192] = v3;
        }
    }
    for (; c < row_vec; c += 64) {
        const uint4 v = src[c];
        for (int j = 0; j < k; ++j)
            if (rows[j] >= 0) x_perm[(int64_t)rows[j] * row_vec + c] = v;
    }
    if (n_scale > 0) {
        for (int q = lane; q < n_scale; q += 64) {
            const float sc = x_scale[t * n_scale + q];
            for (int j = 0; j < k; ++j)
                if (rows[j] >= 0) x_perm_scale[(int64_t)rows[j] * n_scale + q] = sc;
        }
    }
}

hipError_t launch_permute(const void *x, const float *x_scale, const int32_t *slot_row, int T, int k, int H,
                          int elem_bytes, void *x_perm, float *x_perm_scale, hipStream_t s) {
    const int row_vec = H * elem_bytes / 16;  // H is a multiple of 128
    const int n_scale = x_scale ? H / 128 : 0;
    hipLaunchKernelGGL(permute_kernel, dim3((T + 3) / 4), dim3(256), 0, s, (const uint4 *)x, x_scale, slot_row, T, k,
                       row_vec, n_scale, (uint4 *)x_perm, x_perm_scale);
    return hipGetLastError();
}

}  // namespace tpg
