// Weight transform: FP4 E2M1 nibbles and their UE8M0 scales reordered into the layout the
// grouped-GEMM kernels consume (the pages' transform_weights_for_mega_moe,
// chenxutan.com/d/1930 section 3.3: weights are converted once, before any forward).
//
// gfx950's v_mfma_scale_f32_16x16x128_f8f6f4 with an FP4 B operand takes, in lane
// l = 16*g + j, the 32 consecutive K values [32g, 32g+32) of column j as 16 bytes (low
// nibble first), and one UE8M0 scale per lane for column j's 32-block g; the 32-bit scale
// register can hold four such bytes, selected per instruction. The packed layout stores
// every 16-column x 128-K fragment as 64 lanes x 16 bytes in lane order, so a fragment is
// one 1 KB contiguous read, and the scales of four successive K steps as one 32-bit word
// per lane (byte s = K step 4*kb + s).
//
//   W1 data   [E][I/128][H/128][16 frag][64 lane][16 B]   frag 0..7 gate, 8..15 up rows of
//                                                         one 128-wide block of I
// W1's output rows are interleaved inside each 128-block: lane column j of gate fragment f
// (and of up fragment 8 + f) is row 64*(f/4) + 4*j + f%4 of the block. A wave that owns gate
// fragments 4w..4w+3 (or 2w, 2w+1) then holds 4 (or 2) consecutive h columns per lane, which
// it stores as one word. The rows of a dot product are independent, so any order is valid;
// this one serves both wave layouts of the Linear1 kernel.
// W2's output rows are interleaved the same way inside each 256-row tile: lane column j of
// fragment f is row 128*(f/8) + 8*j + f%8, so a wave owning fragments 8w..8w+7 (or
// 4w..4w+3) holds 8 (or 4) consecutive output columns per lane.
//   W1 scales [E][I/128][ceil(H/512)][16][64] u32
//   W2 data   [E][ceil(H/256)][I/128][16][64][16 B]       256 rows of H per column tile
//   W2 scales [E][ceil(H/256)][ceil(I/512)][16][64] u32
// Every byte of the input lands in exactly one place; scale bytes of K steps past the
// end of K are zero. When H is an odd multiple of 128, W2's last column tile is completed
// with 128 zero rows (data and scale bytes 0), as B of the plain GEMMs below.
//
// The plain GEMMs' B ([G][N][K], section 4.3 of the same page) takes the W2 layout with N
// in place of H; when N is not a multiple of 256 the last column tile is completed with
// zero rows (data and scale bytes 0).
#include "moe_internal.h"

namespace moe {
namespace {

// W1 row (of 2I) held by lane column lane%16 of fragment f in column tile nt
__device__ inline int l1_row(int f, int lane, int nt, int I) {
    const int ff = f & 7;
    return (f < 8 ? 0 : I) + nt * 128 + 64 * (ff >> 2) + 4 * (lane & 15) + (ff & 3);
}

// W2 row (of H) held by lane column lane%16 of fragment f in column tile nt
__device__ inline int l2_row(int f, int lane, int nt) {
    return nt * 256 + 128 * (f >> 3) + 8 * (lane & 15) + (f & 7);
}

// One thread per 16-byte chunk of packed data.
__global__ __launch_bounds__(256) void pack_data_kernel(
    const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, size_t n_chunks,
    int rows_per_expert, int src_row_bytes, int nks, int n_tiles, int l1_gate_up, int I) {
    // rows at or past rows_per_expert (the zero padding of a last partial tile) are zeros
    const size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (idx >= n_chunks) return;
    const int lane = (int)(idx & 63);
    const int f = (int)((idx >> 6) & 15);
    size_t rest = idx >> 10;
    const int ks = (int)(rest % nks);
    rest /= nks;
    const int nt = (int)(rest % n_tiles);
    const int e = (int)(rest / n_tiles);
    const int row = l1_gate_up ? l1_row(f, lane, nt, I) : l2_row(f, lane, nt);
    if (row >= rows_per_expert) {
        *reinterpret_cast<uint4*>(dst + idx * 16) = make_uint4(0, 0, 0, 0);
        return;
    }
    const uint8_t* s = src + ((size_t)e * rows_per_expert + row) * src_row_bytes + ks * 64 +
                       (lane >> 4) * 16;
    *reinterpret_cast<uint4*>(dst + idx * 16) = *reinterpret_cast<const uint4*>(s);
}

// One thread per 32-bit scale word.
__global__ __launch_bounds__(256) void pack_scale_kernel(
    const uint8_t* __restrict__ src_sf, uint32_t* __restrict__ dst, size_t n_words,
    int rows_per_expert, int sf_row_bytes, int nks, int nkb, int n_tiles, int l1_gate_up, int I) {
    const size_t idx = blockIdx.x * (size_t)blockDim.x + threadIdx.x;
    if (idx >= n_words) return;
    const int lane = (int)(idx & 63);
    const int f = (int)((idx >> 6) & 15);
    size_t rest = idx >> 10;
    const int kb = (int)(rest % nkb);
    rest /= nkb;
    const int nt = (int)(rest % n_tiles);
    const int e = (int)(rest / n_tiles);
    const int row = l1_gate_up ? l1_row(f, lane, nt, I) : l2_row(f, lane, nt);
    if (row >= rows_per_expert) {
        dst[idx] = 0;
        return;
    }
    const uint8_t* s = src_sf + ((size_t)e * rows_per_expert + row) * sf_row_bytes;
    uint32_t w = 0;
    for (int b = 0; b < 4; ++b) {
        const int ks = kb * 4 + b;
        if (ks < nks) w |= (uint32_t)s[ks * 4 + (lane >> 4)] << (8 * b);
    }
    dst[idx] = w;
}

}  // namespace

PackedLayout packed_layout(const moe_shape_t& s) {
    PackedLayout L{};
    const size_t E = s.num_experts, H = s.hidden, I = s.intermediate;
    const size_t nks1 = H / 128, nkb1 = (H + 511) / 512, nb1 = I / 128;
    const size_t nks2 = I / 128, nkb2 = (I + 511) / 512, nt2 = (H + 255) / 256;
    L.w1d_ntile = nks1 * kBTileBytes;
    L.w1d_expert = nb1 * L.w1d_ntile;
    L.w1s_ntile = nkb1 * kBScaleBlockBytes;
    L.w1s_expert = nb1 * L.w1s_ntile;
    L.w2d_ntile = nks2 * kBTileBytes;
    L.w2d_expert = nt2 * L.w2d_ntile;
    L.w2s_ntile = nkb2 * kBScaleBlockBytes;
    L.w2s_expert = nt2 * L.w2s_ntile;
    size_t off = 0;
    L.w1d = off; off = align_up(off + E * L.w1d_expert, 256);
    L.w1s = off; off = align_up(off + E * L.w1s_expert, 256);
    L.w2d = off; off = align_up(off + E * L.w2d_expert, 256);
    L.w2s = off; off = align_up(off + E * L.w2s_expert, 256);
    L.total = off;
    return L;
}

hipError_t launch_pack(const moe_shape_t& s, const PackedLayout& L, const uint8_t* w1,
                       const uint8_t* w1_sf, const uint8_t* w2, const uint8_t* w2_sf,
                       uint8_t* packed, hipStream_t stream) {
    const int E = s.num_experts, H = s.hidden, I = s.intermediate;
    const int nks1 = H / 128, nkb1 = cdiv(H, 512), nb1 = I / 128;
    const int nks2 = I / 128, nkb2 = cdiv(I, 512), nt2 = cdiv(H, 256);
    const int T = 256;
    {
        const size_t n = (size_t)E * nb1 * nks1 * 1024;
        pack_data_kernel<<<(unsigned)((n + T - 1) / T), T, 0, stream>>>(
            w1, packed + L.w1d, n, 2 * I, H / 2, nks1, nb1, 1, I);
        const size_t m = (size_t)E * nb1 * nkb1 * 1024;
        pack_scale_kernel<<<(unsigned)((m + T - 1) / T), T, 0, stream>>>(
            w1_sf, reinterpret_cast<uint32_t*>(packed + L.w1s), m, 2 * I, H / 32, nks1, nkb1, nb1,
            1, I);
    }
    {
        const size_t n = (size_t)E * nt2 * nks2 * 1024;
        pack_data_kernel<<<(unsigned)((n + T - 1) / T), T, 0, stream>>>(
            w2, packed + L.w2d, n, H, I / 2, nks2, nt2, 0, I);
        const size_t m = (size_t)E * nt2 * nkb2 * 1024;
        pack_scale_kernel<<<(unsigned)((m + T - 1) / T), T, 0, stream>>>(
            w2_sf, reinterpret_cast<uint32_t*>(packed + L.w2s), m, H, I / 32, nks2, nkb2, nt2, 0,
            I);
    }
    return hipGetLastError();
}

PackedBLayout packed_b_layout(int G, int N, int K) {
    PackedBLayout L{};
    L.n_tiles = cdiv(N, 256);
    const size_t nks = K / 128, nkb = cdiv(K, 512);
    L.d_ntile = nks * kBTileBytes;
    L.d_group = L.n_tiles * L.d_ntile;
    L.s_ntile = nkb * kBScaleBlockBytes;
    L.s_group = L.n_tiles * L.s_ntile;
    size_t off = 0;
    L.data = off; off = align_up(off + (size_t)G * L.d_group, 256);
    L.scales = off; off = align_up(off + (size_t)G * L.s_group, 256);
    L.total = off;
    return L;
}

hipError_t launch_pack_b(int G, int N, int K, const PackedBLayout& L, const uint8_t* b,
                         const uint8_t* b_sf, uint8_t* packed, hipStream_t stream) {
    const int nks = K / 128, nkb = cdiv(K, 512), nt = L.n_tiles;
    const int T = 256;
    const size_t n = (size_t)G * nt * nks * 1024;
    pack_data_kernel<<<(unsigned)((n + T - 1) / T), T, 0, stream>>>(b, packed + L.data, n, N, K / 2,
                                                                     nks, nt, 0, 0);
    const size_t m = (size_t)G * nt * nkb * 1024;
    pack_scale_kernel<<<(unsigned)((m + T - 1) / T), T, 0, stream>>>(
        b_sf, reinterpret_cast<uint32_t*>(packed + L.scales), m, N, K / 32, nks, nkb, nt, 0, 0);
    return hipGetLastError();
}

}  // namespace moe
