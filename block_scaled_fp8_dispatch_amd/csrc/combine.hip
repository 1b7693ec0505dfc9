// Combine (chenxutan.com/d/1930 section 3.1 step 5): y[t] = bf16( sum over slots
// j = 0..k-1 of topk_weight[t,j] * stage[t*k + j] ), each staging row holding the bf16
// rounding of its slot's Linear2 output. Slots whose expert id is outside [0, E) were never
// written and add nothing. The sum runs in fp32 in slot order, one fused multiply-add per
// slot, so the result does not depend on which workgroup finished first (no atomics).
#include "moe_internal.h"

namespace moe {
namespace {

__device__ inline uint16_t f32_to_bf16_rne(float v) {
    uint32_t b = __float_as_uint(v);
    if ((b & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
    b += 0x7fffu + ((b >> 16) & 1u);
    return (uint16_t)(b >> 16);
}

// acc += wt * (8 staged bf16 values), one fused multiply-add (single rounding) per value
__device__ inline void add_bf16x8(float (&acc)[8], const uint4 v, float wt) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        acc[2 * q] = __builtin_fmaf(wt, __uint_as_float(w[q] << 16), acc[2 * q]);
        acc[2 * q + 1] = __builtin_fmaf(wt, __uint_as_float(w[q] & 0xffff0000u), acc[2 * q + 1]);
    }
}

__device__ inline uint4 pack_bf16x8(const float (&acc)[8]) {
    uint4 o;
    o.x = f32_to_bf16_rne(acc[0]) | ((uint32_t)f32_to_bf16_rne(acc[1]) << 16);
    o.y = f32_to_bf16_rne(acc[2]) | ((uint32_t)f32_to_bf16_rne(acc[3]) << 16);
    o.z = f32_to_bf16_rne(acc[4]) | ((uint32_t)f32_to_bf16_rne(acc[5]) << 16);
    o.w = f32_to_bf16_rne(acc[6]) | ((uint32_t)f32_to_bf16_rne(acc[7]) << 16);
    return o;
}

// The stage is read once and y is not read again here: both go through non-temporal
// accesses, which keep them from displacing cached data (c4, a 3.76 GB stage: 826 -> 661 us).
__device__ inline uint4 load_nt(const uint16_t* p) {
    const uint32_t* q = reinterpret_cast<const uint32_t*>(p);
    return make_uint4(__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                      __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3));
}

__device__ inline void store_nt(uint16_t* p, const uint4 v) {
    uint32_t* q = reinterpret_cast<uint32_t*>(p);
    __builtin_nontemporal_store(v.x, q);
    __builtin_nontemporal_store(v.y, q + 1);
    __builtin_nontemporal_store(v.z, q + 2);
    __builtin_nontemporal_store(v.w, q + 3);
}

// One thread per 8 output columns (16 bytes) of one token. KMAX > 0: k <= KMAX, and the
// loads of all the token's slots are issued before the sums (which still run in slot
// order); KMAX = 0: any k, one slot at a time.
template <int KMAX>
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ stage,
                                                      const int32_t* __restrict__ topk_idx,
                                                      const float* __restrict__ topk_weights,
                                                      int T, int k, int E, int H,
                                                      uint16_t* __restrict__ y) {
    const int per_row = H / 8;
    const size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (idx >= (size_t)T * per_row) return;
    const int t = (int)(idx / per_row);
    const int c8 = (int)(idx % per_row);
    const uint16_t* src = stage + (size_t)t * k * H + c8 * 8;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if constexpr (KMAX > 0) {
        uint4 v[KMAX];
        float w[KMAX];
#pragma unroll
        for (int j = 0; j < KMAX; ++j) {
            const int e = j < k ? topk_idx[(size_t)t * k + j] : -1;
            const bool ok = e >= 0 && e < E;
            v[j] = ok ? load_nt(src + (size_t)j * H) : make_uint4(0u, 0u, 0u, 0u);
            w[j] = ok ? topk_weights[(size_t)t * k + j] : 0.f;   // a skipped slot adds +0
        }
#pragma unroll
        for (int j = 0; j < KMAX; ++j) add_bf16x8(acc, v[j], w[j]);
    } else {
        for (int j = 0; j < k; ++j) {
            const int e = topk_idx[(size_t)t * k + j];
            if (e < 0 || e >= E) continue;
            add_bf16x8(acc, load_nt(src + (size_t)j * H), topk_weights[(size_t)t * k + j]);
        }
    }
    store_nt(y + (size_t)t * H + c8 * 8, pack_bf16x8(acc));
}

}  // namespace

hipError_t launch_combine(const uint16_t* stage, const int32_t* topk_idx, const float* topk_weights,
                          int T, int k, int E, int H, uint16_t* y, hipStream_t stream) {
    const size_t n = (size_t)T * (H / 8);
    if (n == 0) return hipSuccess;
    const unsigned grid = (unsigned)((n + 255) / 256);
    if (k <= 2)
        combine_kernel<2><<<grid, 256, 0, stream>>>(stage, topk_idx, topk_weights, T, k, E, H, y);
    else if (k <= 4)
        combine_kernel<4><<<grid, 256, 0, stream>>>(stage, topk_idx, topk_weights, T, k, E, H, y);
    else if (k <= 8)
        combine_kernel<8><<<grid, 256, 0, stream>>>(stage, topk_idx, topk_weights, T, k, E, H, y);
    else
        combine_kernel<0><<<grid, 256, 0, stream>>>(stage, topk_idx, topk_weights, T, k, E, H, y);
    return hipGetLastError();
}

}  // namespace moe
