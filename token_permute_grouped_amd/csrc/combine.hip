// Unpermute + combine: out[t] = bf16( sum_j w[t][j] * y_perm[slot_row[t*k+j]] ), or with the
// scatter epilogue's layout (GEMM2 stored every row at its slot) y[t*k+j] for the slots with
// slot_row[t*k+j] >= 0: a token's k rows are then one contiguous run.
//
// The top-k reduction that ends the fused MoE of FlashInfer "[SM90] Add W4A8
// MegaMoE support", with the unpermute folded in as Megatron-LM "add permute
// fusion into hybrid ep" folds it into the combine.  Each output element is an
// fp32 fused multiply-add chain over the token's slots in ascending j, skipping
// dropped slots (-1), then one round-to-nearest-even to bf16: no atomics, so the
// result is bitwise reproducible.
//
// One workgroup per token, as many threads as the row has 16-byte chunks (64 to 512): each
// thread owns chunks blockDim.x apart and issues the loads of all its slots before any
// arithmetic, so a token's k rows (k * H * 2 bytes, each row read exactly once) are in flight
// together.  A row of 256 chunks (H = 2048) on 256 threads rather than 512 half-idle ones: mid
// layer 24.7 -> 23.8 us.
// The y rows are read with non-temporal loads: they are never read again, so they
// need not displace reusable lines in the caches.  Measured on the skewed workload
// (H = 4096, k = 8): 6.1 TB/s, against 5.2 TB/s with 256 threads and ordinary loads.
// The output rows are stored write-through (device scope, see store16_through).
#include <algorithm>

#include "moe_internal.h"

namespace tpg {

namespace {
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint4 load_once(const uint4 *p) {
    const u32x4 v = __builtin_nontemporal_load((const u32x4 *)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

constexpr int kThreads = 512;
}  // namespace

__global__ __launch_bounds__(kThreads) void combine_kernel(const uint4 *__restrict__ y_perm,
                                                           const int32_t *__restrict__ slot_row,
                                                           const float *__restrict__ topk_w, int T, int k,
                                                           int row_vec, bool slot_order,
                                                           uint4 *__restrict__ out) {
    const int64_t t = blockIdx.x;
    const int32_t *rows = slot_row + t * k;  // uniform: scalar loads
    const float *w = topk_w + t * k;
    const int nt = blockDim.x;
    for (int c0 = threadIdx.x; c0 < row_vec; c0 += 2 * nt) {
        const int c1 = c0 + nt;
        const bool two = c1 < row_vec;
        float acc[2][8] = {};
        for (int j0 = 0; j0 < k; j0 += 8) {
            uint4 v[2][8];
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = j0 + q;
                const int32_t r = j < k ? rows[j] : -1;
                const uint4 *yr = y_perm + (slot_order ? t * k + j : (int64_t)r) * row_vec;
                v[0][q] = r >= 0 ? load_once(yr + c0) : make_uint4(0, 0, 0, 0);
                v[1][q] = (r >= 0 && two) ? load_once(yr + c1) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int q = 0; q < 8; ++q) {
                const int j = j0 + q;
                if (j < k && rows[j] >= 0) {
                    combine_fma8(acc[0], w[j], v[0][q]);
                    combine_fma8(acc[1], w[j], v[1][q]);
                }
            }
        }
        const __amdgpu_buffer_rsrc_t dst = row_rsrc(out + t * row_vec, row_vec * 16);
        store16_through(dst, c0 * 16, combine_pack8(acc[0]));
        if (two) store16_through(dst, c1 * 16, combine_pack8(acc[1]));
    }
}

hipError_t launch_combine(const uint16_t *y_perm, const int32_t *slot_row, const float *topk_w, int T, int k, int H,
                          bool slot_order, uint16_t *out, hipStream_t s) {
    const int row_vec = H / 8;
    // one 16-byte chunk per thread (two above 512 chunks): as many threads as the row has chunks
    const int threads = std::min(kThreads, std::max(64, (row_vec + 63) / 64 * 64));
    hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(threads), 0, s, (const uint4 *)y_perm, slot_row, topk_w, T, k,
                       row_vec, slot_order, (uint4 *)out);
    return hipGetLastError();
}

}  // namespace tpg
