/*
 * fp8_fp4_gemm.h -- C ABI of the FP8 x FP4 block-scaled GEMMs and of the FP8 activation
 * cast, in the same library as the MoE forward (libmoe.so, MI355X / gfx950).
 *
 * The operations (pages cited by address and section):
 *   moe_fp8_fp4_gemm       chenxutan.com/d/1930 section 4.3: D = A . B^T with FP8
 *                          activations A [M, K] and their block scales, FP4 weights B
 *                          [N, K] packed two per byte with UE8M0 scales, bf16 D [M, N];
 *                          section 4.2: FP32 accumulation.
 *   moe_m_grouped_fp8_fp4_gemm_contiguous
 *                          juejin.cn/post/7631516744872673307 "MoE模型专属优化" and
 *                          zevenfang.github.io 2026/04/23 section 二: M-axis grouped GEMM
 *                          over a contiguous layout, the rows of all groups back to back,
 *                          each row multiplied by the B of its group.
 *   moe_m_grouped_fp8_fp4_gemm_masked
 *                          the same two passages: the masked grouped GEMM used for decoding
 *                          under graph capture, where each group's row count lives only in
 *                          device memory.
 *   moe_cast_to_fp8        chenxutan.com/d/1930 section 9.2 (the bf16 activation is cast to
 *                          FP8 codes and scale factors before the MoE call) and 11.1 (a
 *                          block's scale follows its largest magnitude).
 *
 * Formats: those of moe.h. A is OCP e4m3fn, one byte per element, rows of K bytes; A's
 * scales are UE8M0 bytes per 1x128 block along K, 4*ceil(K/512) bytes per row (byte j of
 * 32-bit word w = block 4w+j; bytes past K/128 are ignored). B is E2M1, element 2i in the
 * low nibble of byte i, [G][N][K/2]; its scales are UE8M0 per 1x32 block along K,
 * [G][N][K/32]. D is bf16: the FP32 sum of the products, rounded to nearest even.
 *
 * Shapes: K a positive multiple of 128; N a multiple of 16 and at least 16;
 * G (groups) in [1, MOE_MAX_EXPERTS]; the rows of A times K below 2^32.
 *
 * Memory, errors and streams as in moe.h: device pointers, 16-byte aligned, owned by the
 * caller (the library allocates nothing); host-detectable problems return a negative
 * MOE_ERR_* status before any launch; every call is asynchronous on `stream`. Calls that
 * share a workspace must not overlap.
 */
#ifndef MOE_FP8_FP4_GEMM_H
#define MOE_FP8_FP4_GEMM_H

#include "moe.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Bytes of the packed B buffer for `groups` matrices of N x K (N padded to 256-row tiles
 * with zero rows, FP4 data and scales in the kernels' fragment order). 0 if unsupported. */
size_t moe_gemm_packed_b_bytes(int32_t groups, int32_t n, int32_t k);

/* Pack B once (the GEMM's weight transform, as moe_prepare_weights is the forward's):
 *   b     u8 [groups][n][k/2]  E2M1 pairs        b_sf  u8 [groups][n][k/32]  UE8M0
 *   packed  out, packed_bytes >= moe_gemm_packed_b_bytes(groups, n, k).
 * Reads b and b_sf only. */
int moe_gemm_prepare_b(int32_t groups, int32_t n, int32_t k, const uint8_t* b,
                       const uint8_t* b_sf, void* packed, size_t packed_bytes,
                       hipStream_t stream);

/* Workspace bytes of a GEMM call whose A has up to `max_rows` rows in `groups` groups
 * (dense: m rows, 1 group; contiguous: m rows; masked: groups * max_m rows). Holds the row
 * list and tile list of the call and a fixed 16 MiB area for the FP32 partial sums of a
 * dense GEMM whose K is split over several workgroups (used when its output has fewer than
 * 128 tiles of up to 128 x 256; the split sums are added in a fixed order, so results are
 * deterministic). 0 if unsupported. The contents need no initialisation. */
size_t moe_gemm_workspace_bytes(int32_t max_rows, int32_t groups);

/* Dense GEMM: d[r, :] = bf16(A[r, :] . B^T) for r < m, with B = packed group 0.
 *   d     u16 [m][n] bf16 out (row stride n)
 *   a     u8 [m][k] e4m3;  a_sf  u8 [m][4*ceil(k/512)]
 * Decode-sized outputs split K over several workgroups (see moe_gemm_workspace_bytes).
 * m = 0 launches nothing and returns MOE_OK. */
int moe_fp8_fp4_gemm(uint16_t* d, const uint8_t* a, const uint8_t* a_sf, int32_t m, int32_t n,
                     int32_t k, const void* packed_b, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* M-grouped GEMM, contiguous layout: row r of A is multiplied by B[group_of_row[r]].
 *   group_of_row  i32 [m] device; -1 marks a padding row. Rows whose id is outside
 *                 [-1, groups) are skipped like padding. D rows of skipped rows are not
 *                 written. Rows of one group need not be adjacent or aligned; they are
 *                 grouped on the device (stable in row order) before the GEMM runs.
 *   d u16 [m][n], a u8 [m][k], a_sf u8 [m][4*ceil(k/512)] as in moe_fp8_fp4_gemm. */
int moe_m_grouped_fp8_fp4_gemm_contiguous(uint16_t* d, const uint8_t* a, const uint8_t* a_sf,
                                          const int32_t* group_of_row, int32_t m,
                                          int32_t groups, int32_t n, int32_t k,
                                          const void* packed_b, void* workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/* M-grouped GEMM, masked layout: for each group g and i < clamp(masked_m[g], 0, max_m),
 * d[g, i, :] = bf16(A[g, i, :] . B[g]^T); other rows of d are not written.
 *   a u8 [groups][max_m][k], a_sf u8 [groups][max_m][4*ceil(k/512)], d u16 [groups][max_m][n]
 *   masked_m  i32 [groups] device (read on the device: the call never synchronises)
 *   expected_m  the expected rows per group, a hint that picks the row-tile size
 *               (any value gives the same results). */
int moe_m_grouped_fp8_fp4_gemm_masked(uint16_t* d, const uint8_t* a, const uint8_t* a_sf,
                                      const int32_t* masked_m, int32_t groups, int32_t max_m,
                                      int32_t expected_m, int32_t n, int32_t k,
                                      const void* packed_b, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream);

/* FP8 cast: x bf16 [rows][cols] (finite values; cols a multiple of 128) ->
 *   x_fp8  u8 [rows][cols] e4m3 codes, x_sf  u8 [rows][4*ceil(cols/512)] UE8M0,
 * per 1x128 block: byte = max(s + 127, 0) with s the least integer such that
 * amax <= 448 * 2^s (s = 0 for an all-zero block), code = e4m3 round-to-nearest-even of
 * x * 2^-(byte - 127); scale bytes past the row's last block are written as 0. The output
 * is the x_fp8 / x_sf input of moe_forward and the A operand of the GEMMs above.
 * rows = 0 launches nothing. */
int moe_cast_to_fp8(const uint16_t* x, int32_t rows, int32_t cols, uint8_t* x_fp8,
                    uint8_t* x_sf, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_FP8_FP4_GEMM_H */
