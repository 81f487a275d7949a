// W4A8 expert FFN: FP8 E4M3 activations (one fp32 scale per 128 columns) times
// NVFP4 weights dequantised to FP8 in-kernel, on FP8 matrix cores.
//
// FlashInfer "[SM90] Add W4A8 MegaMoE support": the fused kernel's NVFP4 -> FP8
// dequant and its Usage section (E2M1 codes, one E4M3 scale per 16 values, FP32
// activation scales per 128 channels); follow-up #6517 point 4 (low-nibble-first
// packing, 6 * scale <= 448 so the dequantised value fits E4M3, per-expert global
// scales).
#include "moe_internal.h"

namespace tpg {

namespace w4a8 {

// E2M1 magnitude of a 3-bit code: 0, 0.5, 1, 1.5, 2, 3, 4, 6
__device__ __forceinline__ float e2m1_mag(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    return e == 0 ? 0.5f * (float)m : __uint_as_float((e + 126u) << 23) * (1.0f + 0.5f * (float)m);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// one weight: e2m1(code) * e4m3(scale), rounded to nearest-even E4M3, saturating at +-448
__device__ __forceinline__ uint32_t fp4_to_fp8(uint32_t code4, uint32_t scale8) {
    float v = e2m1_mag(code4 & 7u) * e4m3_to_f32(scale8);
    v = (code4 & 8u) ? -v : v;
    v = fminf(fmaxf(v, -448.0f), 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, v, 0, false) & 0xffu;
}

}  // namespace w4a8

__global__ void w4a8_dequant_table_kernel(uint8_t *out8) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;  // 16 * 256 entries
    if (i < 16 * 256) out8[i] = (uint8_t)w4a8::fp4_to_fp8((uint32_t)(i >> 8), (uint32_t)(i & 255));
}

hipError_t launch_w4a8_dequant_table(uint8_t *out8, hipStream_t s) {
    hipLaunchKernelGGL(w4a8_dequant_table_kernel, dim3(16), dim3(256), 0, s, out8);
    return hipGetLastError();
}

hipError_t launch_grouped_ffn_w4a8(const uint8_t *, const float *, const int32_t *, const int32_t *, const int32_t *,
                                   int64_t, const moe_weights &, const moe_problem &, uint8_t *, float *, uint16_t *,
                                   hipStream_t) {
    return hipErrorNotSupported;
}

}  // namespace tpg
