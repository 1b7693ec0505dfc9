// FP8 cast of bf16 activation rows: e4m3 codes plus one UE8M0 scale per 1x128 block
// (chenxutan.com/d/1930 section 9.2: the activation is cast to FP8 codes and scale factors
// before the MoE call; section 11.1: a block's scale follows its largest magnitude).
//
// Per block: s = the least integer with amax <= 448 * 2^s (amax = 0: s = 0), byte =
// max(s + 127, 0), code = e4m3 of x * 2^-(byte - 127), round to nearest even. bf16 -> fp32
// and the power-of-two product are exact, so nothing rounds before the decision. Scale
// bytes of the last 32-bit word past the row's last block are 0.
//
// Memory-bound: one wave per (row, 512-column chunk); lane l holds columns 8l .. 8l+7 of
// the chunk (one 16-byte load, one 8-byte store), so the 16 lanes of a DPP row hold one
// 128-column block and its amax is a 16-lane DPP max.
#include "moe_internal.h"

namespace moe {
namespace {

constexpr int kCastThreads = 256;

// UE8M0 byte of a block whose largest magnitude has fp32 bit pattern `bits` (sign clear)
__device__ inline uint32_t cast_scale_byte(uint32_t bits) {
    if (bits == 0) return 127u;
    const int ex = (int)(bits >> 23);                 // 0 for a subnormal amax
    const uint32_t mant = bits & 0x7fffffu;
    const int b = ex - 8 + (mant > 0x600000u ? 1 : 0);   // 448 = 1.75 * 2^8
    return b < 0 ? 0u : (uint32_t)b;                  // subnormal amax: s <= -133, byte 0
}

__global__ __launch_bounds__(kCastThreads) void cast_fp8_kernel(const uint16_t* __restrict__ x,
                                                                int cols, int chunks,
                                                                uint8_t* __restrict__ q,
                                                                uint8_t* __restrict__ sf,
                                                                int sf_stride, size_t n_waves) {
    const size_t wid = blockIdx.x * (size_t)(kCastThreads / 64) + (threadIdx.x >> 6);
    if (wid >= n_waves) return;
    const int lane = threadIdx.x & 63;
    const size_t row = wid / chunks;
    const int ch = (int)(wid % chunks);
    const int c0 = ch * 512 + lane * 8;
    const bool active = c0 < cols;                    // cols % 128 == 0: whole DPP rows
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (active) v = *reinterpret_cast<const uint4*>(x + row * cols + c0);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float f[8];
    uint32_t m = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = w[i] << 16, hi = w[i] & 0xffff0000u;
        f[2 * i] = __uint_as_float(lo);
        f[2 * i + 1] = __uint_as_float(hi);
        m = max(m, max(lo & 0x7fffffffu, hi & 0x7fffffffu));
    }
    // largest magnitude over the 16 lanes of the DPP row (non-negative floats order like
    // their bit patterns): swap neighbours, swap pairs, mirror each half row, mirror the row
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0xB1, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x4E, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x141, 0xF, 0xF, false));
    m = max(m, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)m, 0x140, 0xF, 0xF, false));
    const uint32_t byte = cast_scale_byte(m);
    const float mul = __uint_as_float((254u - byte) << 23);   // 2^-(byte - 127); byte <= 247
    if (active) {
        int p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[0] * mul, f[1] * mul, 0, false);
        p0 = __builtin_amdgcn_cvt_pk_fp8_f32(f[2] * mul, f[3] * mul, p0, true);
        int p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[4] * mul, f[5] * mul, 0, false);
        p1 = __builtin_amdgcn_cvt_pk_fp8_f32(f[6] * mul, f[7] * mul, p1, true);
        *reinterpret_cast<uint2*>(q + row * cols + c0) = make_uint2((uint32_t)p0, (uint32_t)p1);
    }
    if ((lane & 15) == 0)
        sf[row * sf_stride + ch * 4 + (lane >> 4)] = active ? (uint8_t)byte : (uint8_t)0;
}

}  // namespace

hipError_t launch_cast_fp8(const uint16_t* x, int rows, int cols, uint8_t* q, uint8_t* sf,
                           hipStream_t stream) {
    const int chunks = cdiv(cols, 512);
    const size_t n_waves = (size_t)rows * chunks;
    if (n_waves == 0) return hipSuccess;
    const size_t blocks = (n_waves + kCastThreads / 64 - 1) / (kCastThreads / 64);
    cast_fp8_kernel<<<(unsigned)blocks, kCastThreads, 0, stream>>>(x, cols, chunks, q, sf,
                                                                  4 * chunks, n_waves);
    return hipGetLastError();
}

}  // namespace moe
