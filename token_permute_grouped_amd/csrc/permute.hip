// Permute (row gather into expert-contiguous order): x_perm[slot_row[t*k+j]] = x[t].
//
// Megatron-LM "add permute fusion into hybrid ep" moves each token row into the
// expert-major order the grouped GEMMs read.  Here the copy is driven from the
// token side: a wave reads a piece of x[t] once (16-byte loads, fully coalesced) and
// writes it to each of the token's k destination rows, so HBM sees exactly T*H reads
// and R*H writes, never a re-read of a token row.  On the W4A8 path the per-128 fp32
// activation scales travel with their row.  The destination rows are stored write-through
// (device scope, see store16_through).
#include "moe_internal.h"

namespace tpg {

// One wave per (token, column block of up to 4 x 64 sixteen-byte chunks): a lane issues
// all of its loads before any store, so a row costs one load round trip however wide it
// is (a 7 KB fp8 row took four dependent round trips when one wave walked the whole row).
constexpr int kBlockVec = 4 * 64;

__global__ __launch_bounds__(256) void permute_kernel(const uint4 *__restrict__ x, const float *__restrict__ x_scale,
                                                      const int32_t *__restrict__ slot_row, int T, int k,
                                                      int row_vec, int n_blk, int n_scale, uint4 *__restrict__ x_perm,
                                                      float *__restrict__ x_perm_scale) {
    const int lane = threadIdx.x & 63;
    const int64_t w = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t t = w / n_blk;
    if (t >= T) return;
    const int blk = (int)(w - t * n_blk);
    const int32_t *rows = slot_row + t * k;  // wave-uniform: scalar loads

    const uint4 *src = x + t * row_vec;
    const int c0 = blk * kBlockVec + lane;
    uint4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
        if (c0 + 64 * q < row_vec) v[q] = src[c0 + 64 * q];
    for (int j = 0; j < k; ++j) {
        if (rows[j] < 0) continue;
        const __amdgpu_buffer_rsrc_t dst = row_rsrc(x_perm + (int64_t)rows[j] * row_vec, row_vec * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q)
            if (c0 + 64 * q < row_vec) store16_through(dst, (c0 + 64 * q) * 16, v[q]);
    }
    if (blk == 0 && n_scale > 0) {
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
    const int n_blk = (row_vec + kBlockVec - 1) / kBlockVec;
    const int n_scale = x_scale ? H / 128 : 0;
    const int64_t waves = (int64_t)T * n_blk;
    hipLaunchKernelGGL(permute_kernel, dim3((waves + 3) / 4), dim3(256), 0, s, (const uint4 *)x, x_scale, slot_row, T,
                       k, row_vec, n_blk, n_scale, (uint4 *)x_perm, x_perm_scale);
    return hipGetLastError();
}

}  // namespace tpg
