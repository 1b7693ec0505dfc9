// Internal declarations shared by the HIP sources of the MoE library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "moe.h"

namespace moe {

// Routing processes the flattened (token, slot) list in chunks of this many slots per
// workgroup; each chunk's per-expert histogram is one row of the block-count table. (2048
// against 4096: twice the workgroups for the count and the scatter, each with half the
// rounds; c3 -1 %, c4 -0.3 %, c2 unchanged; 1024 was no better.)
constexpr int kRouteChunk = 2048;
constexpr int kRouteThreads = 256;
// Output columns of one grouped-GEMM tile: Linear1 = 128 gate + 128 up columns of one
// 128-wide block of the intermediate; Linear2 = 256 hidden columns.
constexpr int kBN = 256;
// One K step of the main loop (one 16x16x128 scaled MFMA along K).
constexpr int kBK = 128;
// Bytes of one packed B fragment: 16 columns x 128 K of FP4 = 64 lanes x 16 bytes.
constexpr int kFragBytes = 1024;
// Bytes of the packed B data of one (tile, K step): 16 fragments.
constexpr int kBTileBytes = 16 * kFragBytes;
// Bytes of the packed B scales of one (tile, 512-K block): 16 fragments x 64 lanes x 4.
constexpr int kBScaleBlockBytes = 16 * 64 * 4;

// Rows of a half tile: with 256-row tiles, an expert's last tile that holds at most this
// many rows is listed after all full tiles (meta[3] = number of full tiles) and runs as one
// 128-row tile in the second launch of the 256-row class.
constexpr int kHalfTileRows = 128;

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Word index of the blocked UE8M0 scales of the dispatched activations (xg_sf) and of h
// (h_sf): padded rows in blocks of hblk rows (a multiple of 64), `words` 32-bit words per
// row (word w holds the bytes of 128-column blocks 4w .. 4w+3). Block b stores its rows'
// word 0, then word 1, ...; within each 64-row group, row 16f + i (f < 4, i < 16) sits at
// position 4i + f, so that a GEMM lane reads the words of rows i, 16+i, 32+i, 48+i (its
// four 16-row fragments) as one 16-byte load.
__host__ __device__ inline uint32_t blocked_scale_word(uint32_t p, uint32_t w, uint32_t words, uint32_t hblk) {
    const uint32_t r = p % hblk;
    const uint32_t pos = (r & ~63u) | ((r & 15u) << 2) | ((r >> 4) & 3u);
    return ((p / hblk) * words + w) * hblk + pos;
}
inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// Offsets of the four regions of the packed weight buffer.
struct PackedLayout {
    size_t w1d, w1s, w2d, w2s, total;
    size_t w1d_expert, w1d_ntile;   // bytes per expert, per 128-column block of I
    size_t w1s_expert, w1s_ntile;
    size_t w2d_expert, w2d_ntile;   // per 256-column block of H
    size_t w2s_expert, w2s_ntile;
};

PackedLayout packed_layout(const moe_shape_t& s);

// Routing kernels (route.hip)
hipError_t launch_route(const int32_t* topk_idx, int num_slots, int E, int block_m,
                        int32_t* blk_counts, int32_t* meta, int32_t* counts, int32_t* offsets,
                        int32_t* perm, int32_t* inv, int32_t* tile_expert, int32_t* tile_row0,
                        int max_tiles, hipStream_t stream);

// Weight transform (pack.hip)
hipError_t launch_pack(const moe_shape_t& s, const PackedLayout& L,
                       const uint8_t* w1, const uint8_t* w1_sf, const uint8_t* w2,
                       const uint8_t* w2_sf, uint8_t* packed, hipStream_t stream);

// Grouped GEMMs (gemm.hip)
struct GemmArgs {
    // A operand: rows of FP8 codes with per-1x128 UE8M0 scales
    const uint8_t* a;          // A rows: blocked (h8, or the dispatched x) or x itself
    int a_blocked;             // 1: A blocked like h8; 0 (Linear1 only): rows of x
                               // gathered through perm
    const uint8_t* a_sf;       // Linear1/2: the blocked scale copy (xg_sf, h_sf), except
                               // Linear1 with 64-row tiles and no dispatch copy: x_sf, rows
                               // named by perm; plain GEMM: scale rows named by perm
    int a_stride;              // bytes per A row (= K)
    int a_sf_stride;           // scale bytes per A row (4*ceil(K/512))
    int K;                     // reduction length (multiple of 128)
    int topk;                  // a_blocked == 0: slot -> token = slot / topk
    const int32_t* perm;       // per padded row: slot (MoE) or A/D row (plain GEMM); -1 padding
    const int32_t* meta;       // meta[0] = M tiles in use, meta[3] = full tiles among them
    const int32_t* tile_expert;
    const int32_t* tile_row0;
    int n_tiles;               // column tiles per M tile
    int max_tiles;
    // Tail split (256-row tiles only): when the last round of tiles (split_round workgroups
    // run at once) is at most half full, its tiles are left to a second launch that runs
    // each as two 128-row halves (tail = 1). 0 disables it.
    int split_round;
    int tail;
    int host_tiles;            // M tiles in use when the host knows them (dense GEMM), else -1
    int max_half;              // most half tiles the tile list can hold (one per group), 0: none
    int dense_rows;            // plain GEMM only: > 0 = dense rows 0..dense_rows-1, no row list
    // B operand: packed weights
    const uint8_t* b;
    const uint32_t* b_sf;
    size_t b_expert, b_ntile;        // bytes
    size_t bs_expert, bs_ntile;      // 32-bit words
    // h8 is stored in blocks of hblk rows x 128 columns, [P_pad/hblk][I/128][hblk][128]: the
    // block a Linear1 tile writes is the A block one Linear2 K step reads, contiguous
    int hblk;
    // Linear1 outputs
    uint8_t* h8;
    uint8_t* h_sf;
    int h_stride;              // = I
    int h_sf_stride;
    // Linear2 outputs (plain GEMM: stage = D, out_cols = N, the row stride of D)
    uint16_t* stage;
    const float* topk_weights;
    int out_cols;              // = H
    uint32_t out_bytes;        // bytes of `stage` when below 4 GiB (32-bit store offsets), else 0
    // Split-K of the plain GEMM: `splits` workgroups per output tile, each over ks_split K
    // steps (a multiple of 4), FP32 partials [tile][split][BM][256]
    int splits;
    int ks_split;
    float* partial;
};

hipError_t launch_linear1(int block_m, const GemmArgs& a, hipStream_t stream);
hipError_t launch_linear2(int block_m, const GemmArgs& a, hipStream_t stream);
// Plain FP8 x FP4 GEMM over a row list: D[perm[p]] = bf16(A[perm[p]] . B_g^T)
hipError_t launch_gemm_plain(int block_m, const GemmArgs& a, hipStream_t stream);
// The same with K split over a.splits workgroups per tile (block_m 64 or 128), then the
// in-order reduction of the FP32 partials
hipError_t launch_gemm_splitk(int block_m, const GemmArgs& a, hipStream_t stream);

// Packed B of the plain GEMMs ([G][N][K] FP4, the W2 layout): N padded to 256-row tiles
// with zero rows
struct PackedBLayout {
    size_t data, scales, total;          // byte offsets
    size_t d_group, d_ntile;             // bytes
    size_t s_group, s_ntile;             // bytes
    int n_tiles;
};
PackedBLayout packed_b_layout(int G, int N, int K);
hipError_t launch_pack_b(int G, int N, int K, const PackedBLayout& L, const uint8_t* b,
                         const uint8_t* b_sf, uint8_t* packed, hipStream_t stream);

// Row list and tile list of the masked plain GEMM without a routing pass (route.hip): group
// g's rows g*max_m + i, i < clamp(masked_m[g], 0, max_m), each group padded to BM rows.
hipError_t launch_gemm_layout(int G, int max_m, const int32_t* masked_m, int block_m,
                              int pad_rows_cap, int32_t* perm, int32_t* tile_expert,
                              int32_t* tile_row0, int32_t* meta, hipStream_t stream);

// FP8 cast of bf16 rows (cast.hip)
hipError_t launch_cast_fp8(const uint16_t* x, int rows, int cols, uint8_t* q, uint8_t* sf,
                           hipStream_t stream);

// Dispatch copy (route.hip): the x row (when xg is not null) and the scale row of each
// padded row's token into the blocked A layout of Linear1 and the blocked scale layout
// (zero on padding rows)
hipError_t launch_gather(const uint8_t* x, const uint8_t* x_sf, const int32_t* perm,
                         const int32_t* meta, int k, int H, int sfs, int hblk, int max_rows,
                         uint8_t* xg, uint8_t* xg_sf, hipStream_t stream);

// Combine (combine.hip)
hipError_t launch_combine(const uint16_t* stage, const int32_t* topk_idx, const float* topk_weights,
                          int T, int k, int E, int H, uint16_t* y, hipStream_t stream);

}  // namespace moe
