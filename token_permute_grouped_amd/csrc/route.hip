// Router: one 16-lane row per token (the per-token body is route_token16, route_token.h).
#include "route_token.h"

namespace tpg {

// four tokens per wave (one per 16-lane row), 16 per workgroup
__global__ __launch_bounds__(256) void route_topk_kernel(const float *__restrict__ logits,
                                                         const uint8_t *__restrict__ slot_drop, int T, int E, int k,
                                                         int32_t *__restrict__ topk_idx,
                                                         float *__restrict__ topk_w) {
    const int lane = threadIdx.x & 63;
    const int64_t t0 = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 6) * 4;  // first token of this wave
    if (t0 >= T) return;  // whole wave leaves together
    const int64_t t = t0 + (lane >> 4);
    route_token16(logits, slot_drop, t < T ? t : T - 1, t < T, E, k, lane & 15, topk_idx, topk_w, nullptr);
}

hipError_t launch_route_topk(const float *logits, const uint8_t *slot_drop, int T, int E, int k, int32_t *topk_idx,
                             float *topk_w, hipStream_t s) {
    const int blocks = (T + 15) / 16;
    hipLaunchKernelGGL(route_topk_kernel, dim3(blocks), dim3(256), 0, s, logits, slot_drop, T, E, k, topk_idx,
                       topk_w);
    return hipGetLastError();
}
}  // namespace tpg
