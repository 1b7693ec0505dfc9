// Combine (chenxutan.com/d/1930 section 3.1 step 5): y[t] = bf16( sum over slots
// j = 0..k-1 of stage[t*k + j] ), each staging row already holding
// bf16(topk_weight[t,j] * Linear2 output). Slots whose expert id is outside [0, E) were
// never written and add nothing. The sum runs in fp32 in slot order, so the result does
// not depend on which workgroup finished first (no atomics).
#include "moe_internal.h"

namespace moe {
namespace {

__device__ inline uint16_t f32_to_bf16_rne(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// One thread per 8 output columns (16 bytes) of one token.
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ stage,
                                                      const int32_t* __restrict__ topk_idx,
                                                      int T, int k, int E, int H,
                                                      uint16_t* __restrict__ y) {
    const int per_row = H / 8;
    const size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (idx >= (size_t)T * per_row) return;
    const int t = (int)(idx / per_row);
    const int c8 = (int)(idx % per_row);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int j = 0; j < k; ++j) {
        const int e = topk_idx[(size_t)t * k + j];
        if (e < 0 || e >= E) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(stage + ((size_t)t * k + j) * H + c8 * 8);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            acc[2 * q] += __uint_as_float(w[q] << 16);
            acc[2 * q + 1] += __uint_as_float(w[q] & 0xffff0000u);
        }
    }
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    *reinterpret_cast<uint4*>(y + (size_t)t * H + c8 * 8) = o;
}

}  // namespace

hipError_t launch_combine(const uint16_t* stage, const int32_t* topk_idx, int T, int k, int E,
                          int H, uint16_t* y, hipStream_t stream) {
    const size_t n = (size_t)T * (H / 8);
    if (n == 0) return hipSuccess;
    combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(stage, topk_idx, T, k, E, H, y);
    return hipGetLastError();
}

}  // namespace moe
