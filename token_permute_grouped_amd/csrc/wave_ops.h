// Wave64 cross-lane operations over DPP row operations (no LDS traffic), and a 256-entry
// workgroup prefix sum built on them.
//
// DPP source of lane i: quad_perm / row_shr / row_half_mirror / row_mirror stay within a row
// of 16 lanes; row_bcast15 / row_bcast31 carry lane 15 / 31 into later rows (the rows that
// row_mask enables).  Lanes with no source, and rows outside row_mask, keep `fill`.  Every
// function here must be called by all 64 lanes of the wave.
#pragma once
#include "moe_internal.h"

namespace tpg {
namespace wave {

constexpr int kQuadSwap1 = 0xb1, kQuadSwap2 = 0x4e, kRowShr1 = 0x111, kRowShr2 = 0x112, kRowShr4 = 0x114,
              kRowShr8 = 0x118, kRowHalfMirror = 0x141, kRowMirror = 0x140, kRowBcast15 = 0x142,
              kRowBcast31 = 0x143;

template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp(uint32_t x, uint32_t fill) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)fill, (int)x, kCtrl, kRowMask, 0xf, false);
}

// maximum / minimum of x over the 64 lanes, returned to every lane
__device__ __forceinline__ uint32_t max_u32(uint32_t x) {
    x = max(x, dpp<kQuadSwap1, 0xf>(x, 0u));
    x = max(x, dpp<kQuadSwap2, 0xf>(x, 0u));
    x = max(x, dpp<kRowHalfMirror, 0xf>(x, 0u));  // every lane: the maximum of its 8-lane half row
    x = max(x, dpp<kRowMirror, 0xf>(x, 0u));      // every lane: the maximum of its 16-lane row
    x = max(x, dpp<kRowBcast15, 0xa>(x, 0u));     // rows 1 and 3: rows 0-1 and 2-3
    x = max(x, dpp<kRowBcast31, 0xc>(x, 0u));     // rows 2 and 3: rows 0-3 (lane 63)
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}
__device__ __forceinline__ uint32_t min_u32(uint32_t x) {
    x = min(x, dpp<kQuadSwap1, 0xf>(x, ~0u));
    x = min(x, dpp<kQuadSwap2, 0xf>(x, ~0u));
    x = min(x, dpp<kRowHalfMirror, 0xf>(x, ~0u));
    x = min(x, dpp<kRowMirror, 0xf>(x, ~0u));
    x = min(x, dpp<kRowBcast15, 0xa>(x, ~0u));
    x = min(x, dpp<kRowBcast31, 0xc>(x, ~0u));
    return (uint32_t)__builtin_amdgcn_readlane((int)x, 63);
}

// inclusive prefix sum over the lanes: lane i gets x_0 + ... + x_i
__device__ __forceinline__ int incl_sum(int v) {
    uint32_t x = (uint32_t)v;
    x += dpp<kRowShr1, 0xf>(x, 0u);
    x += dpp<kRowShr2, 0xf>(x, 0u);
    x += dpp<kRowShr4, 0xf>(x, 0u);
    x += dpp<kRowShr8, 0xf>(x, 0u);   // every lane: the prefix within its row of 16
    x += dpp<kRowBcast15, 0xa>(x, 0u);  // rows 1 and 3 add the last lane of rows 0 and 2
    x += dpp<kRowBcast31, 0xc>(x, 0u);  // rows 2 and 3 add lane 31 (rows 0-1)
    return (int)x;
}

}  // namespace wave

// Inclusive prefix sums of a and b over threads 0..255 of the workgroup (threads 256 and up
// pass and get unspecified values).  Every thread of the workgroup must call it: it holds one
// barrier.  ws is 8 ints of LDS that nothing may write again before the workgroup's next
// barrier.  *total_a / *total_b receive the sums over all 256 threads.
__device__ __forceinline__ void block_incl_sum256(int &a, int &b, int *ws, int *total_a, int *total_b) {
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    a = wave::incl_sum(a);
    b = wave::incl_sum(b);
    if (w < 4 && lane == 63) {
        ws[w] = a;
        ws[4 + w] = b;
    }
    __syncthreads();
    int ta = 0, tb = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (i < w) {
            a += ws[i];
            b += ws[4 + i];
        }
        ta += ws[i];
        tb += ws[4 + i];
    }
    *total_a = ta;
    *total_b = tb;
}

}  // namespace tpg
